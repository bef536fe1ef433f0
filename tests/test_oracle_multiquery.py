"""Pins for the oracle's multi-query decode (the verification step of
speculative decoding: the q_len newest tokens of a sequence attend at once,
each causally).  Checked against an independent dense formulation with an
explicit causal mask, against closed forms that depend on the causal count
(equal keys give the mean of V over each query's visible prefix), and against
the single-query oracle on the prefix each query sees."""
import numpy as np
import pytest
import torch

import oracle
from quantized_decode_attention_calibrate_amd import workloads

from test_oracle_attention import calibrated, dense_dequant_fp8


def dense_mq(w, q, Kd, Vd, sm_scale):
    """fp64 reference: per sequence contiguous K/V, causal mask as an explicit
    boolean matrix [q_len][L] (query i sees tokens t <= L - q_len + i)."""
    qq = q.float().double().numpy()
    B, q_len, Hq, D = qq.shape
    out = np.zeros((B, q_len, Hq, D))
    for b, (s0, L) in enumerate(zip(w.seq_starts, w.seq_lens)):
        if L == 0:
            continue
        mask = np.arange(L)[None, :] <= (L - q_len + np.arange(q_len))[:, None]
        for h in range(Hq):
            g = h // (Hq // w.Hkv)
            sc = np.float64(np.float32(sm_scale)) * (qq[b, :, h, :] @ Kd[s0:s0 + L, g, :].T)   # [q_len][L]
            sc = np.where(mask, sc, -np.inf)
            for i in range(q_len):
                if not mask[i].any():
                    continue
                p = np.exp(sc[i] - sc[i].max())
                out[b, i, h] = (p[:, None] * Vd[s0:s0 + L, g, :]).sum(0) / p.sum()
    return out


def caches(w, kvd, ks, vs):
    kc, vc = oracle.new_caches(kvd, w.num_blocks, w.Hkv, w.D, w.block_size)
    oracle.cache_write(w.k, w.v, w.slot_mapping, kc, vc, kvd, ks, vs)
    return kc, vc


@pytest.mark.parametrize("q_len", [1, 2, 4, 7])
@pytest.mark.parametrize("kvd,D,shape", [(oracle.KV_FP8, 64, dict(Hq=16, Hkv=2)),
                                         (oracle.KV_FP8, 128, dict(Hq=4, Hkv=4)),
                                         (oracle.KV_BF16, 64, dict(Hq=8, Hkv=2))])
def test_multiquery_matches_dense_causal(q_len, kvd, D, shape):
    w = workloads.make("mixed64", seed=11, seq_lens=[37, 3, 80], shape=dict(shape, D=D))
    q = workloads.mq_queries(w, q_len, seed=1)
    ks, vs = calibrated(w) if kvd == oracle.KV_FP8 else (1.0, 1.0)
    kc, vc = caches(w, kvd, ks, vs)
    sm = np.float32(1.0 / np.sqrt(D))
    out = oracle.decode_attn_mq(q, kc, vc, kvd, w.block_tables, w.seq_lens, w.Hkv, 16, ks, vs, float(sm))
    if kvd == oracle.KV_FP8:
        Kd, Vd = dense_dequant_fp8(w.k, ks), dense_dequant_fp8(w.v, vs)
    else:
        Kd, Vd = w.k.double().numpy(), w.v.double().numpy()
    ref = dense_mq(w, q, Kd, Vd, sm)
    assert np.abs(out - ref).max() < 1e-12


def test_each_query_is_single_query_attention_on_its_prefix():
    w = workloads.make("tiny", seed=12, seq_lens=[50, 19])
    q_len = 5
    q = workloads.mq_queries(w, q_len, seed=2)
    ks, vs = calibrated(w)
    kc, vc = caches(w, oracle.KV_FP8, ks, vs)
    out = oracle.decode_attn_mq(q, kc, vc, oracle.KV_FP8, w.block_tables, w.seq_lens, w.Hkv, 16, ks, vs, 0.125)
    for i in range(q_len):
        lens = [L - q_len + 1 + i for L in w.seq_lens]
        one = oracle.decode_attn(q[:, i], kc, vc, oracle.KV_FP8, w.block_tables, lens, w.Hkv, 16, ks, vs, 0.125)
        assert np.array_equal(out[:, i], one)
    # the newest query sees the whole sequence: the single-query decode of w.q
    full = oracle.decode_attn(w.q, kc, vc, oracle.KV_FP8, w.block_tables, w.seq_lens, w.Hkv, 16, ks, vs, 0.125)
    assert np.array_equal(out[:, q_len - 1], full)


def test_equal_keys_give_prefix_means():
    w = workloads.make("tiny", seed=13, seq_lens=[21, 40])
    w.k[:] = w.k[0:1]
    q_len = 6
    q = workloads.mq_queries(w, q_len, seed=3)
    ks, vs = calibrated(w)
    kc, vc = caches(w, oracle.KV_FP8, ks, vs)
    out = oracle.decode_attn_mq(q, kc, vc, oracle.KV_FP8, w.block_tables, w.seq_lens, w.Hkv, 16, ks, vs, 0.125)
    Vd = dense_dequant_fp8(w.v, vs)
    for b, (s0, L) in enumerate(zip(w.seq_starts, w.seq_lens)):
        for i in range(q_len):
            n = L - q_len + 1 + i
            for h in range(w.Hq):
                assert np.abs(out[b, i, h] - Vd[s0:s0 + n, h // w.G].mean(0)).max() < 1e-13


def test_queries_before_the_sequence_start_are_zero():
    # 3 tokens, 5 queries: queries 0 and 1 would sit before the first token
    w = workloads.make("tiny", seed=14, seq_lens=[3, 0])
    q = workloads.mq_queries(w, 5, seed=4)
    ks, vs = calibrated(w)
    kc, vc = caches(w, oracle.KV_FP8, ks, vs)
    out = oracle.decode_attn_mq(q, kc, vc, oracle.KV_FP8, w.block_tables, w.seq_lens, w.Hkv, 16, ks, vs, 0.125)
    assert (out[0, :2] == 0).all() and (out[1] == 0).all()
    Vd = dense_dequant_fp8(w.v, vs)
    for h in range(w.Hq):
        assert np.array_equal(out[0, 2, h], Vd[0, h // w.G])   # one visible token: v_0
