"""Pins for the oracle's FP8 Q and P attention variant.

An independent dense formulation (torch's float8_e4m3fn casts for the Q and
P codes, numpy for the rest, no paging) must agree to 1e-12; closed forms:
equal keys give the mean of V (every P code is equal), constant V gives the
constant, one visible token gives its value; and the variant stays close to
exact attention (it quantizes Q and the softmax weights to 3 mantissa bits).

The variant's tolerance (kvqo_decode_attn_fp8qp_tol) has pins of its own in
test_oracle_fp8qp_tol.py."""
import math

import numpy as np
import pytest
import torch

import oracle
from quantized_decode_attention_calibrate_amd import workloads

from test_oracle_attention import calibrated, dense_dequant_fp8
from test_oracle_multiquery import caches

LOG2E = 1.4426950408889634


def e4m3(x: np.ndarray) -> np.ndarray:
    """value(E4M3(x)) for |x| <= 448 (torch's cast rounds to nearest even)."""
    return torch.from_numpy(np.asarray(x, dtype=np.float32)).to(torch.float8_e4m3fn).to(torch.float64).numpy()


def dense_fp8qp(w, q, kc, vc, qs, ks, vs, sm, window=0):
    qq = q.float().numpy()
    B, q_len, Hq, D = qq.shape
    qv = e4m3(np.clip(qq / np.float32(qs), -448, 448))           # value of qc (IEEE fp32 division)
    c = float(np.float32(float(sm) * float(qs) * float(ks) * LOG2E))
    Kd = dense_dequant_fp8(w.k, ks) / np.float64(np.float32(ks))   # code values of K
    Vd = dense_dequant_fp8(w.v, vs) / np.float64(np.float32(vs))
    out = np.zeros((B, q_len, Hq, D))
    for b, (s0, L) in enumerate(zip(w.seq_starts, w.seq_lens)):
        for i in range(q_len):
            p = L - q_len + i
            lo = max(0, p - window + 1) if window else 0
            if p < 0:
                continue
            for h in range(Hq):
                g = h // (Hq // w.Hkv)
                x = c * (Kd[s0 + lo:s0 + p + 1, g, :] @ qv[b, i, h])
                R = math.ceil(x.max())
                pc = e4m3(448.0 * np.exp2(x - R))
                out[b, i, h] = float(np.float32(vs)) * (pc[:, None] * Vd[s0 + lo:s0 + p + 1, g, :]).sum(0) / pc.sum()
    return out


def run(w, q, qs, ks, vs, sm=0.125, window=0):
    kc, vc = caches(w, oracle.KV_FP8, ks, vs)
    return oracle.decode_attn_fp8qp(q, kc, vc, w.block_tables, w.seq_lens, w.Hkv, 16, qs, ks, vs, sm,
                                    window=window), kc, vc


def q_scale(q):
    return float(oracle.calibrate([oracle.amax_bf16(q)])[0])


@pytest.mark.parametrize("q_len,window,D", [(1, 0, 64), (3, 0, 128), (2, 20, 64), (1, 0, 256)])
def test_fp8qp_matches_dense(q_len, window, D):
    w = workloads.make("mixed64", seed=71, seq_lens=[45, 3, 130], shape=dict(Hq=8, Hkv=2, D=D))
    q = workloads.mq_queries(w, q_len, seed=2)
    ks, vs = calibrated(w)
    qs = q_scale(q)
    out, kc, vc = run(w, q, qs, ks, vs, window=window)
    ref = dense_fp8qp(w, q, kc, vc, qs, ks, vs, 0.125, window)
    assert np.abs(out - ref).max() < 1e-12


def test_fp8qp_closed_forms():
    w = workloads.make("tiny", seed=72, seq_lens=[60, 1])
    w.k[:] = w.k[0:1]   # equal keys: every P code is 448
    ks, vs = calibrated(w)
    q = w.q[:, None]
    out, _, _ = run(w, q, q_scale(q), ks, vs)
    Vd = dense_dequant_fp8(w.v, vs)
    for b, (s0, L) in enumerate(zip(w.seq_starts, w.seq_lens)):
        for h in range(w.Hq):
            assert np.abs(out[b, 0, h] - Vd[s0:s0 + L, h // w.G].mean(0)).max() < 1e-13
    w2 = workloads.make("tiny", seed=73, seq_lens=[90, 17])
    w2.v[:] = 1.5
    out2, _, _ = run(w2, w2.q[:, None], q_scale(w2.q), 0.03, 1.0 / 64)
    assert np.abs(out2 - 1.5).max() < 1e-13


def test_fp8qp_close_to_exact_attention():
    # 3-bit Q and P: every score and weight moves by a few per cent (rel L2 ~9e-2 on this N(0,1) data)
    w = workloads.make("gptoss65k", seed=74, seq_lens=[2000, 500], shape=dict(Hq=16, Hkv=2))
    q = workloads.mq_queries(w, 2, seed=3)
    ks, vs = calibrated(w)
    out, kc, vc = run(w, q, q_scale(q), ks, vs)
    exact = oracle.decode_attn_mq(q, kc, vc, oracle.KV_FP8, w.block_tables, w.seq_lens, w.Hkv, 16, ks, vs, 0.125,
                                  nthreads=8)
    rel = np.linalg.norm(out - exact) / np.linalg.norm(exact)
    assert 1e-2 < rel < 0.15, rel
