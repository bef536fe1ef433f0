"""Pins for the oracle's paged cache write and decode attention (CPU only).

The oracle reads a paged cache through block tables; these tests compare it
with an independent dense formulation (torch's float8 cast for the codes,
numpy softmax on contiguous per-sequence arrays, no paging), so a wrong
layout, block-table lookup, GQA mapping or scale placement fails.  Closed
forms: equal keys give mean(V); constant V gives that constant (the weights
sum to one); one token gives v_0; an empty sequence gives 0.  Physical block
placement does not change the result at all.
"""
import numpy as np
import pytest
import torch

import oracle
from quantized_decode_attention_calibrate_amd import workloads


def dense_dequant_fp8(x: torch.Tensor, scale: float) -> np.ndarray:
    y = (x.float() / torch.tensor(np.float32(scale))).clamp(-448, 448)
    return y.to(torch.float8_e4m3fn).to(torch.float64).numpy() * np.float64(np.float32(scale))


def dense_attention(w, Kd, Vd, sm_scale):
    """Dense fp64 reference: per sequence contiguous K/V, numpy softmax."""
    q = w.q.float().double().numpy()
    out = np.zeros((w.B, w.Hq, w.D))
    for b, (s0, L) in enumerate(zip(w.seq_starts, w.seq_lens)):
        for h in range(w.Hq):
            g = h // w.G
            if L == 0:
                continue
            Kb = Kd[s0:s0 + L, g, :]
            Vb = Vd[s0:s0 + L, g, :]
            sc = np.float64(np.float32(sm_scale)) * (Kb @ q[b, h])
            p = np.exp(sc - sc.max())
            out[b, h] = (p[:, None] * Vb).sum(0) / p.sum()
    return out


def oracle_path(w, kv_dtype, k_scale=1.0, v_scale=1.0, sm_scale=None, slots=None):
    kc, vc = oracle.new_caches(kv_dtype, w.num_blocks, w.Hkv, w.D, w.block_size)
    oracle.cache_write(w.k, w.v, w.slot_mapping if slots is None else slots, kc, vc, kv_dtype,
                       k_scale, v_scale)
    sm = np.float32(1.0 / np.sqrt(w.D)) if sm_scale is None else sm_scale
    return oracle.decode_attn(w.q, kc, vc, kv_dtype, w.block_tables, w.seq_lens, w.Hkv, w.block_size,
                              k_scale, v_scale, float(sm)), kc, vc


def calibrated(w):
    return (float(oracle.calibrate([oracle.amax_bf16(w.k)])[0]),
            float(oracle.calibrate([oracle.amax_bf16(w.v)])[0]))


def test_fp8_attention_matches_dense_formulation():
    w = workloads.make("tiny", seed=0)
    ks, vs = calibrated(w)
    out, _, _ = oracle_path(w, oracle.KV_FP8, ks, vs)
    ref = dense_attention(w, dense_dequant_fp8(w.k, ks), dense_dequant_fp8(w.v, vs),
                          np.float32(1.0 / 8.0))
    assert np.abs(out - ref).max() < 1e-12


def test_bf16_attention_matches_dense_formulation():
    w = workloads.make("tiny", seed=1, seq_lens=[33, 1, 16, 70], shape=dict(Hq=6, Hkv=2, D=64))
    out, _, _ = oracle_path(w, oracle.KV_BF16)
    ref = dense_attention(w, w.k.double().numpy(), w.v.double().numpy(), np.float32(1.0 / 8.0))
    assert np.abs(out - ref).max() < 1e-12


@pytest.mark.parametrize("D", [64, 128, 256])
def test_gqa_groups_and_head_dims(D):
    w = workloads.make("mixed64", seed=4, seq_lens=[40, 17], shape=dict(Hq=8, Hkv=2, D=D))
    ks, vs = calibrated(w)
    out, _, _ = oracle_path(w, oracle.KV_FP8, ks, vs)
    ref = dense_attention(w, dense_dequant_fp8(w.k, ks), dense_dequant_fp8(w.v, vs),
                          np.float32(1.0 / np.sqrt(D)))
    assert np.abs(out - ref).max() < 1e-12


def test_equal_keys_give_mean_of_values():
    w = workloads.make("tiny", seed=2, seq_lens=[45, 300])
    w.k[:] = w.k[0:1]          # every token, same key row
    ks, vs = calibrated(w)
    out, _, _ = oracle_path(w, oracle.KV_FP8, ks, vs)
    Vd = dense_dequant_fp8(w.v, vs)
    for b, (s0, L) in enumerate(zip(w.seq_starts, w.seq_lens)):
        for h in range(w.Hq):
            mean = Vd[s0:s0 + L, h // w.G, :].mean(0)
            assert np.abs(out[b, h] - mean).max() < 1e-13


def test_constant_values_weights_sum_to_one():
    w = workloads.make("tiny", seed=3)
    w.v[:] = 1.5
    out, _, _ = oracle_path(w, oracle.KV_FP8, 1.0, 1.0)
    assert np.abs(out - 1.5).max() < 1e-13


def test_single_token_and_empty_sequence():
    w = workloads.make("tiny", seed=5, seq_lens=[1, 0, 2])
    ks, vs = calibrated(w)
    out, _, _ = oracle_path(w, oracle.KV_FP8, ks, vs)
    Vd = dense_dequant_fp8(w.v, vs)
    for h in range(w.Hq):
        assert np.array_equal(out[0, h], Vd[0, h // w.G])
    assert (out[1] == 0).all()


def test_physical_block_placement_is_irrelevant():
    w = workloads.make("tiny", seed=6)
    ks, vs = calibrated(w)
    out1, _, _ = oracle_path(w, oracle.KV_FP8, ks, vs)
    perm = torch.randperm(w.num_blocks, generator=torch.Generator().manual_seed(9))
    bt2 = perm[w.block_tables.long()].to(torch.int32)
    for b, L in enumerate(w.seq_lens):  # unused table entries stay 0
        bt2[b, (L + 15) // 16:] = 0
    slots2 = perm[w.slot_mapping // 16] * 16 + w.slot_mapping % 16
    w2 = workloads.Workload(**{**w.__dict__, "block_tables": bt2, "slot_mapping": slots2})
    out2, _, _ = oracle_path(w2, oracle.KV_FP8, ks, vs)
    assert np.array_equal(out1, out2)


def test_cache_write_skips_negative_slots_and_leaves_other_bytes():
    w = workloads.make("tiny", seed=7, seq_lens=[20, 9])
    ks, vs = calibrated(w)
    kc, vc = oracle.new_caches(oracle.KV_FP8, w.num_blocks, w.Hkv, w.D, w.block_size, fill=0xA5)
    sm = w.slot_mapping.clone()
    sm[::3] = -1
    oracle.cache_write(w.k, w.v, sm, kc, vc, oracle.KV_FP8, ks, vs)
    written = set(int(s) for s in sm if s >= 0)
    kq = np.asarray(kc).reshape(w.num_blocks, w.Hkv, w.block_size, w.D)
    for blk in range(w.num_blocks):
        for off in range(w.block_size):
            if blk * 16 + off not in written:
                assert (kq[blk, :, off, :] == 0xA5).all()
    # written bytes equal the element-wise quantization of their source, at
    # the documented places: K [block][head][offset][dim], V [block][head][dim][offset]
    vq = np.asarray(vc).reshape(w.num_blocks, w.Hkv, w.D, w.block_size)
    Kd, Vd = dense_dequant_fp8(w.k, ks), dense_dequant_fp8(w.v, vs)
    table = oracle.e4m3_table()
    for t in range(w.T):
        s = int(sm[t])
        if s < 0:
            continue
        assert np.array_equal(table[kq[s // 16, :, s % 16, :]] * np.float64(np.float32(ks)), Kd[t])
        assert np.array_equal(table[vq[s // 16, :, :, s % 16]] * np.float64(np.float32(vs)), Vd[t])


def test_attention_units_subset_matches_full():
    w = workloads.make("tiny", seed=8)
    ks, vs = calibrated(w)
    out, kc, vc = oracle_path(w, oracle.KV_FP8, ks, vs)
    units = [(1, 3), (0, 0), (1, 1)]
    sub = oracle.decode_attn(w.q, kc, vc, oracle.KV_FP8, w.block_tables, w.seq_lens, w.Hkv, 16, ks, vs,
                             0.125, units=units, nthreads=3)
    for i, (b, h) in enumerate(units):
        assert np.array_equal(sub[i], out[b, h])
    full_mt = oracle.decode_attn(w.q, kc, vc, oracle.KV_FP8, w.block_tables, w.seq_lens, w.Hkv, 16, ks, vs,
                                 0.125, nthreads=4)
    assert np.array_equal(full_mt, out)


def test_reconstruction_cosine_reported():
    w = workloads.make("tiny", seed=0)
    ks, _ = calibrated(w)
    c_cal = oracle.fp8_cos_sim(w.k, ks)
    c_one = oracle.fp8_cos_sim(w.k, 1.0)
    assert 0.99 < c_cal <= 1.0 and 0.99 < c_one <= 1.0
    # a tensor far below the E4M3 normal range: scale 1.0 underflows, calibration does not
    tiny = (w.k.float() * 1e-4).to(torch.bfloat16)
    ts = float(oracle.calibrate([oracle.amax_bf16(tiny)])[0])
    assert oracle.fp8_cos_sim(tiny, ts) > 0.99 > oracle.fp8_cos_sim(tiny, 1.0)
