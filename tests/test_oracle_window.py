"""Pins for the oracle's sliding-window decode: query i (token position
p = L - q_len + i) sees tokens max(0, p - W + 1) .. p.  Checked against an
independent dense formulation with an explicit band mask, the closed form at
W = 1 (each query returns its own token's value), full attention when the
window covers the sequence, and full attention over a re-paged sequence that
holds only the window's tokens."""
import numpy as np
import pytest
import torch

import oracle
from quantized_decode_attention_calibrate_amd import workloads

from test_oracle_attention import calibrated, dense_dequant_fp8
from test_oracle_multiquery import caches


def dense_window(w, q, Kd, Vd, sm_scale, W):
    qq = q.float().double().numpy()
    B, q_len, Hq, D = qq.shape
    out = np.zeros((B, q_len, Hq, D))
    for b, (s0, L) in enumerate(zip(w.seq_starts, w.seq_lens)):
        if L == 0:
            continue
        t = np.arange(L)[None, :]
        p = (L - q_len + np.arange(q_len))[:, None]
        band = (t <= p) & (t > p - W)
        for h in range(Hq):
            g = h // (Hq // w.Hkv)
            sc = np.float64(np.float32(sm_scale)) * (qq[b, :, h, :] @ Kd[s0:s0 + L, g, :].T)
            sc = np.where(band, sc, -np.inf)
            for i in range(q_len):
                if not band[i].any():
                    continue
                e = np.exp(sc[i] - sc[i].max())
                out[b, i, h] = (e[:, None] * Vd[s0:s0 + L, g, :]).sum(0) / e.sum()
    return out


@pytest.mark.parametrize("q_len", [1, 3])
@pytest.mark.parametrize("W", [1, 5, 16, 40, 1000])
def test_window_matches_dense_band(q_len, W):
    w = workloads.make("mixed64", seed=31, seq_lens=[37, 2, 90], shape=dict(Hq=8, Hkv=2, D=64))
    q = workloads.mq_queries(w, q_len, seed=1)
    ks, vs = calibrated(w)
    kc, vc = caches(w, oracle.KV_FP8, ks, vs)
    out = oracle.decode_attn_mq(q, kc, vc, oracle.KV_FP8, w.block_tables, w.seq_lens, w.Hkv, 16, ks, vs, 0.125,
                                window=W)
    ref = dense_window(w, q, dense_dequant_fp8(w.k, ks), dense_dequant_fp8(w.v, vs), 0.125, W)
    assert np.abs(out - ref).max() < 1e-12


def test_window_one_returns_own_value():
    w = workloads.make("tiny", seed=32, seq_lens=[20, 7])
    q = workloads.mq_queries(w, 4, seed=2)
    kc, vc = caches(w, oracle.KV_BF16, 1.0, 1.0)
    out = oracle.decode_attn_mq(q, kc, vc, oracle.KV_BF16, w.block_tables, w.seq_lens, w.Hkv, 16, 1.0, 1.0, 0.125,
                                window=1)
    for b, (s0, L) in enumerate(zip(w.seq_starts, w.seq_lens)):
        for i in range(4):
            for h in range(w.Hq):
                assert np.array_equal(out[b, i, h], w.v[s0 + L - 4 + i, h // w.G].double().numpy())


def test_window_covering_the_sequence_is_full_attention():
    w = workloads.make("tiny", seed=33, seq_lens=[50, 31])
    q = workloads.mq_queries(w, 2, seed=3)
    ks, vs = calibrated(w)
    kc, vc = caches(w, oracle.KV_FP8, ks, vs)
    full = oracle.decode_attn_mq(q, kc, vc, oracle.KV_FP8, w.block_tables, w.seq_lens, w.Hkv, 16, ks, vs, 0.125)
    wide = oracle.decode_attn_mq(q, kc, vc, oracle.KV_FP8, w.block_tables, w.seq_lens, w.Hkv, 16, ks, vs, 0.125,
                                 window=50)
    assert np.array_equal(full, wide)


def test_window_equals_a_sequence_of_its_tokens_only():
    # the newest query's W-token window, written as a sequence of its own
    w = workloads.make("tiny", seed=34, seq_lens=[77])
    W = 23
    ks, vs = calibrated(w)
    kc, vc = caches(w, oracle.KV_FP8, ks, vs)
    out = oracle.decode_attn_mq(w.q[:, None], kc, vc, oracle.KV_FP8, w.block_tables, w.seq_lens, w.Hkv, 16, ks, vs,
                                0.125, window=W)
    w2 = workloads.make("tiny", seed=35, seq_lens=[W])
    k2, v2 = w.k[77 - W:].clone(), w.v[77 - W:].clone()
    kc2, vc2 = oracle.new_caches(oracle.KV_FP8, w2.num_blocks, w.Hkv, w.D, 16)
    oracle.cache_write(k2, v2, w2.slot_mapping, kc2, vc2, oracle.KV_FP8, ks, vs)
    ref = oracle.decode_attn(w.q, kc2, vc2, oracle.KV_FP8, w2.block_tables, [W], w.Hkv, 16, ks, vs, 0.125)
    assert np.array_equal(out[:, 0], ref)
