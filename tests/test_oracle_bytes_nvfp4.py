"""Byte accounting pinned to the pages' printed numbers, and the oracle's NVFP4
(block-scaled E2M1) write pinned by exact reconstruction, an error bound and,
bit for bit, an independent dense quantizer (numpy fp32 arithmetic, torch's
RNE float8 cast for the block scale, a midpoint-count E2M1 rounding) on
seeded data, on block scales exactly at every E4M3 rounding midpoint, on
inputs where the fp32 quotient alone decides the block-scale tie, and on
E2M1 ties under block scales that are not powers of two.

Pages: the calibration guide (BF16 element 2 B, FP8 1 B, so the FP8 payload
is half) and the Run 26 video description (24,576 B/token in BF16 for
gpt-oss-20b; 3 GB / 1.5 GB / 0.75 GB at 128k; 4.5 bits per number, 1.8x
smaller than FP8).
"""
import json
import os

import numpy as np
import pytest
import torch

import oracle
from quantized_decode_attention_calibrate_amd import workloads

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_numbers.json")))
GiB = 2 ** 30


def per_token_bytes(kv_dtype, Hkv, D, bs=16):
    kc, vc = oracle.new_caches(kv_dtype, 1, Hkv, D, bs)
    return (kc.nbytes + vc.nbytes) / bs


def test_fp8_block_is_half_of_bf16():
    for Hkv, D in [(8, 64), (4, 256), (8, 128), (2, 64)]:
        assert per_token_bytes(oracle.KV_FP8, Hkv, D) * 2 == per_token_bytes(oracle.KV_BF16, Hkv, D)
        assert per_token_bytes(oracle.KV_FP8, Hkv, D) == Hkv * D * 2 * GOLDEN["fp8_bytes_per_elem"]["value"]


def test_gptoss_bytes_per_token_and_128k_footprint():
    layer = per_token_bytes(oracle.KV_BF16, 8, 64)
    assert layer == 2048
    printed = GOLDEN["bf16_kv_bytes_per_token_gptoss20b"]["value"]
    assert printed % layer == 0 and printed // layer == 12   # 12 full-attention layers
    fp = GOLDEN["kv_footprint_128k_gb"]["value"]
    n = 131072
    assert n * printed == fp["bf16"] * GiB
    assert n * 12 * per_token_bytes(oracle.KV_FP8, 8, 64) == fp["fp8"] * GiB
    nv = n * 12 * per_token_bytes(oracle.KV_NVFP4, 8, 64)
    payload = n * 12 * 8 * 64 * 2 * 0.5          # 4-bit codes only
    assert payload == fp["nvfp4_rate"] * GiB
    assert nv == pytest.approx(0.84375 * GiB)    # with the E4M3 block scales


def test_nvfp4_bits_per_number():
    for D in (64, 128, 256):
        r = oracle.nvfp4_region_bytes(D, 16)
        bits = 8 * r / (16 * D)
        assert bits == GOLDEN["nvfp4_bits_per_num"]["value"]
    assert round(8 / 4.5, 1) == GOLDEN["nvfp4_vs_fp8_ratio"]["value"]
    assert oracle.nvfp4_region_bytes(64, 16) == 576


def _bits(t):
    return t.view(torch.int16).numpy().view(np.uint16)


def test_nvfp4_exact_for_representable_values():
    # gscale 1: a group whose max is 6 gets block scale E4M3(6 / 6) = 1.0 and
    # every E2M1-representable element reconstructs exactly
    rng = np.random.default_rng(0)
    grid = np.array([0, .5, 1, 1.5, 2, 3, 4, 6])
    T, Hkv, D = 16, 2, 64
    vals = rng.choice(grid, size=(T, Hkv, D)) * rng.choice([-1, 1], size=(T, Hkv, D))
    vals[:, :, ::16] = 6.0
    k = torch.tensor(vals, dtype=torch.bfloat16)
    v = torch.tensor(-vals, dtype=torch.bfloat16)
    kc, vc = oracle.new_caches(oracle.KV_NVFP4, 1, Hkv, D, 16)
    oracle.nvfp4_cache_write(k, v, np.arange(T), kc, vc, 16, 1.0, 1.0)
    kd = oracle.nvfp4_values(kc, "k", range(T), Hkv, D, 16, 1.0)
    vd = oracle.nvfp4_values(vc, "v", range(T), Hkv, D, 16, 1.0)
    assert np.array_equal(kd, vals) and np.array_equal(vd, -vals)
    # scale code of every group is 0x38 (1.0)
    assert (kc[0, :, 16 * D // 2:] == 0x38).all()


def test_nvfp4_error_bound_and_layout():
    w = workloads.make("tiny", seed=11, seq_lens=[37])
    gk = float(oracle.nvfp4_calibrate([oracle.amax_bf16(w.k)])[0])
    gv = float(oracle.nvfp4_calibrate([oracle.amax_bf16(w.v)])[0])
    kc, vc = oracle.new_caches(oracle.KV_NVFP4, w.num_blocks, w.Hkv, w.D, 16)
    oracle.nvfp4_cache_write(w.k, w.v, w.slot_mapping, kc, vc, 16, gk, gv)
    for x, cache, which, gs in ((w.k, kc, "k", gk), (w.v, vc, "v", gv)):
        xd = x.double().numpy()
        got = oracle.nvfp4_values(cache, which, w.slot_mapping.tolist(), w.Hkv, w.D, 16, gs)
        # per 16-element group: effective scale e = value(bscale) * gscale and
        # |x - xhat| <= half the local E2M1 gap times e, or the saturation excess
        for t in range(w.T):
            for g in range(w.Hkv):
                for grp in range(w.D // 16):
                    xs = xd[t, g, grp * 16:(grp + 1) * 16]
                    hs = got[t, g, grp * 16:(grp + 1) * 16]
                    amax = np.abs(xs).max()
                    e_ideal = amax / 6.0
                    # block scale is E4M3-rounded: within 1/16 relative of ideal
                    assert np.abs(np.abs(hs).max() - amax) <= amax * (1 / 16 + 1 / 6) + 1e-30
                    y = np.abs(xs) / e_ideal
                    gap = np.where(y < 2, 0.5, np.where(y < 4, 1.0, 2.0))
                    assert (np.abs(xs - hs) <= (gap / 2 * (1 + 1 / 15) + 6 / 15) * e_ideal + 1e-30).all()
                    assert (np.sign(hs) * np.sign(xs) >= 0).all()


def test_nvfp4_attention_matches_dense_formulation():
    w = workloads.make("nvfp4_131k", seed=12, seq_lens=[50, 23], shape=dict(Hq=8, Hkv=2, D=64))
    gk = float(oracle.nvfp4_calibrate([oracle.amax_bf16(w.k)])[0])
    gv = float(oracle.nvfp4_calibrate([oracle.amax_bf16(w.v)])[0])
    kc, vc = oracle.new_caches(oracle.KV_NVFP4, w.num_blocks, w.Hkv, w.D, 16)
    oracle.nvfp4_cache_write(w.k, w.v, w.slot_mapping, kc, vc, 16, gk, gv)
    out = oracle.decode_attn(w.q, kc, vc, oracle.KV_NVFP4, w.block_tables, w.seq_lens, w.Hkv, 16, gk, gv,
                             0.125)
    slots = w.slot_mapping.tolist()
    Kd = oracle.nvfp4_values(kc, "k", slots, w.Hkv, w.D, 16, gk)
    Vd = oracle.nvfp4_values(vc, "v", slots, w.Hkv, w.D, 16, gv)
    q = w.q.double().numpy()
    for b, (s0, L) in enumerate(zip(w.seq_starts, w.seq_lens)):
        for h in range(w.Hq):
            g = h // w.G
            sc = np.float64(0.125) * (Kd[s0:s0 + L, g] @ q[b, h])
            p = np.exp(sc - sc.max())
            ref = (p[:, None] * Vd[s0:s0 + L, g]).sum(0) / p.sum()
            assert np.abs(out[b, h] - ref).max() < 1e-12


# ---- an independent dense quantizer, compared with the oracle bit for bit ----

E2M1_MIDPOINTS = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])


def e2m1_codes(y: np.ndarray) -> np.ndarray:
    """Round-to-nearest-even E2M1 codes of float32 y, saturating at 6: the
    number of rounding midpoints below |y| is the nearest code; on a midpoint
    (a tie between codes j and j + 1) the even one.  Sign bit 3 from y's sign."""
    a = np.abs(y.astype(np.float64))
    idx = np.searchsorted(E2M1_MIDPOINTS, a, side="left")
    tie = np.isin(a, E2M1_MIDPOINTS)
    idx = np.where(tie & (idx % 2 == 1), idx + 1, idx)
    return (idx | np.where(np.signbit(y), 8, 0)).astype(np.uint8)


def dense_nvfp4(x: torch.Tensor, gscale: float):
    """The block-scaled 4-bit write of bf16 x [T][Hkv][D] as numpy arrays:
    block scale codes [T][Hkv][D/16] (torch's RNE float8 cast of the clamped
    fp32 ratio) and E2M1 codes [T][Hkv][D]."""
    T, H, D = x.shape
    xf = x.float().numpy().reshape(T, H, D // 16, 16)
    bamax = np.abs(xf).max(-1)
    top = np.float32(6.0) * np.float32(gscale)
    ratio = (bamax / top).astype(np.float32)
    sc = torch.from_numpy(np.clip(ratio, 0, 448)).to(torch.float8_e4m3fn)
    e = (sc.to(torch.float32).numpy() * np.float32(gscale)).astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        y = (xf / e[..., None]).astype(np.float32)
    codes = np.where(e[..., None] == 0, 0, e2m1_codes(y)).astype(np.uint8)
    return sc.view(torch.uint8).numpy(), codes.reshape(T, H, D)


def dense_nvfp4_caches(k, v, slots, num_blocks, gk, gv, bs=16):
    """Paged NVFP4 caches in the documented layout, built from dense_nvfp4."""
    T, H, D = k.shape
    r = oracle.nvfp4_region_bytes(D, bs)
    kc = np.zeros((num_blocks, H, r), np.uint8)
    vc = np.zeros((num_blocks, H, r), np.uint8)
    ksc, kcode = dense_nvfp4(k, gk)
    vsc, vcode = dense_nvfp4(v, gv)
    for t, s in enumerate(np.asarray(slots)):
        if s < 0:
            continue
        blk, off = s // bs, s % bs
        for g in range(H):
            kr, vr = kc[blk, g], vc[blk, g]
            row = kcode[t, g]
            kr[off * D // 2:(off + 1) * D // 2] = row[0::2] | (row[1::2] << 4)     # element 2i low nibble
            kr[bs * D // 2 + off * (D // 16):bs * D // 2 + (off + 1) * (D // 16)] = ksc[t, g]
            sh = 4 * (off % 2)                                                    # token 2j low nibble
            col = vr[:bs * D // 2].reshape(D, bs // 2)
            col[:, off // 2] = (col[:, off // 2] & (0xF0 >> sh)) | (vcode[t, g] << sh)
            vr[bs * D // 2:].reshape(D // 16, bs)[:, off] = vsc[t, g]
    return kc, vc


def test_nvfp4_write_equals_a_dense_quantizer_on_seeded_data():
    w = workloads.make("nvfp4_131k", seed=13, seq_lens=[70, 33], shape=dict(Hq=8, Hkv=2, D=128))
    gk = float(oracle.nvfp4_calibrate([oracle.amax_bf16(w.k)])[0])
    gv = float(oracle.nvfp4_calibrate([oracle.amax_bf16(w.v)])[0])
    kc, vc = oracle.new_caches(oracle.KV_NVFP4, w.num_blocks, w.Hkv, w.D, 16)
    oracle.nvfp4_cache_write(w.k, w.v, w.slot_mapping, kc, vc, 16, gk, gv)
    dk, dv = dense_nvfp4_caches(w.k, w.v, w.slot_mapping.numpy(), w.num_blocks, gk, gv)
    assert np.array_equal(kc, dk) and np.array_equal(vc, dv)


def e4m3_midpoints() -> np.ndarray:
    vals = np.unique(np.abs(torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn)
                            .to(torch.float64).numpy()))
    vals = vals[np.isfinite(vals)]
    return (vals[:-1] + vals[1:]) / 2


def test_nvfp4_block_scales_at_e4m3_midpoints_and_e2m1_ties():
    # gscale 0.5: 6 * gscale = 3 exactly, so a block amax of 3m gives the ratio m
    # exactly for every E4M3 rounding midpoint m (3m has at most 7 significant
    # bits: exact in bf16); also one bf16 step either side of 3m
    mids = e4m3_midpoints()
    assert len(mids) == 126
    amaxes = []
    for m in mids:
        a = torch.tensor(3 * m, dtype=torch.bfloat16)
        assert float(a) == 3 * m
        up = (a.view(torch.int16) + 1).view(torch.bfloat16)
        dn = (a.view(torch.int16) - 1).view(torch.bfloat16)
        amaxes += [float(a), float(up), float(dn)]
    # blocks with amax 6 at gscale 0.5 take the scale 2.0, so e = 1.0 and the
    # elements are divided by 1: every E2M1 midpoint and its neighbours, both signs
    ties = np.concatenate([E2M1_MIDPOINTS, np.nextafter(E2M1_MIDPOINTS.astype(np.float32), 0),
                           np.nextafter(E2M1_MIDPOINTS.astype(np.float32), 10), [0.0, 1e-3, 5.9, 6.0]])
    H, D = 2, 64
    n_groups = len(amaxes) + 4
    T = -(-n_groups // (H * D // 16))
    rng = np.random.default_rng(14)
    x = rng.uniform(-1, 1, size=(T, H, D // 16, 16)) * 0.01
    flat = x.reshape(-1, 16)
    for i, a in enumerate(amaxes):
        flat[i, :] *= a
        flat[i, i % 16] = a if i % 2 else -a
    for j in range(4):                      # four blocks of E2M1 ties (amax 6)
        row = flat[len(amaxes) + j]
        row[:] = np.resize(ties, 16) * (1 if j % 2 else -1)
        row[0] = 6.0
        row[1] = -0.0 if j == 0 else row[1]
    xb = torch.tensor(x.reshape(T, H, D), dtype=torch.bfloat16)
    assert np.array_equal(xb.float().numpy().reshape(-1, 16)[:len(amaxes)].__abs__().max(1),
                          np.array(amaxes, dtype=np.float32))
    slots = np.random.default_rng(15).permutation(T)     # any slot order
    nb = -(-T // 16)
    kc, vc = oracle.new_caches(oracle.KV_NVFP4, nb, H, D, 16)
    oracle.nvfp4_cache_write(xb, xb, slots, kc, vc, 16, 0.5, 0.5)
    dk, dv = dense_nvfp4_caches(xb, xb, slots, nb, 0.5, 0.5)
    assert np.array_equal(kc, dk) and np.array_equal(vc, dv)
    # the ties were hit: half the exact-midpoint blocks round down to an even code
    sc, _ = dense_nvfp4(xb, 0.5)
    mid_codes = sc.reshape(-1)[:len(amaxes):3]
    assert (mid_codes % 2 == 0).all()


def test_nvfp4_quotients_are_fp32_divisions_at_ties():
    """Inputs where the definition's fp32 steps decide a code.  Block scales:
    for these global scales 6 * gscale rounds in fp32, and bamax /
    fp32(6 * gscale) lands exactly on an E4M3 rounding midpoint (a tie that
    goes to the even code) while the exact quotient does not (found by a
    search over fp32 global scales and bf16 block maxima).  Elements: E2M1
    midpoints times block scales e that are not powers of two (e = value of
    the block scale times gscale 0.5), where x / e is the tie itself and a
    product with a rounded 1 / e is not."""
    H, D = 1, 64
    rng = np.random.default_rng(16)
    # (gscale, block maxima) with the fp32 quotient on an E4M3 midpoint
    cases = [(0.7850877642631531, [0.08740234375, 0.1748046875, 0.349609375, 0.69921875]),
             (0.40208330750465393, [0.01177978515625])]
    for gs, maxima in cases:
        gs = float(np.float32(gs))
        x = rng.uniform(-1, 1, size=(len(maxima), H, D // 16, 16)) * 1e-3
        for t, a in enumerate(maxima):
            x[t, :, :, 3] = a
        xb = torch.tensor(x.reshape(len(maxima), H, D), dtype=torch.bfloat16)
        ratio = (np.float32(max(maxima)) / (np.float32(6.0) * np.float32(gs))).astype(np.float32)
        assert float(ratio) * (6.0 * gs) != max(maxima)          # the fp32 quotient is not the exact one
        kc, vc = oracle.new_caches(oracle.KV_NVFP4, 1, H, D, 16)
        oracle.nvfp4_cache_write(xb, xb, np.arange(len(maxima)), kc, vc, 16, gs, gs)
        dk, dv = dense_nvfp4_caches(xb, xb, np.arange(len(maxima)), 1, gs, gs)
        assert np.array_equal(kc, dk) and np.array_equal(vc, dv)
    # E2M1 ties under block scales 1.125 .. 1.875 (and two binades of each)
    svals = [m * 2.0 ** k for m in (1.125, 1.25, 1.375, 1.5, 1.625, 1.75, 1.875) for k in (-3, 0, 2)]
    T = len(svals)
    x = np.zeros((T, H, D // 16, 16))
    for t, s in enumerate(svals):
        e = s * 0.5
        row = np.concatenate([E2M1_MIDPOINTS, -E2M1_MIDPOINTS, [0.5, 6.0]]) * e   # exact in bf16
        x[t, :, :, :] = row
    xb = torch.tensor(x.reshape(T, H, D), dtype=torch.bfloat16)
    assert np.array_equal(xb.float().numpy(), x.reshape(T, H, D).astype(np.float32))
    nb = -(-T // 16)
    kc, vc = oracle.new_caches(oracle.KV_NVFP4, nb, H, D, 16)
    oracle.nvfp4_cache_write(xb, xb, np.arange(T), kc, vc, 16, 0.5, 0.5)
    dk, dv = dense_nvfp4_caches(xb, xb, np.arange(T), nb, 0.5, 0.5)
    assert np.array_equal(kc, dk) and np.array_equal(vc, dv)
    sc, codes = dense_nvfp4(xb, 0.5)
    assert np.array_equal(sc.view(np.uint8), np.broadcast_to(
        torch.tensor(svals, dtype=torch.float32).to(torch.float8_e4m3fn).view(torch.uint8).numpy()[:, None, None],
        sc.shape))
    # every tie went to the even code: 0.25->0, 0.75->2(1.0), 1.25->2, 1.75->4, 2.5->4, 3.5->6, 5->6
    assert np.array_equal(codes[:, 0, :7] & 7, np.broadcast_to([0, 2, 2, 4, 4, 6, 6], (T, 7)))
