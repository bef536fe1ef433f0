"""GPU invariants of decode attention that hold without the oracle's numbers.

- FP8 against BF16: the FP8 kernel over codes with power-of-two scales
  equals, to fp32 rounding noise, the BF16 kernel over the dequantized
  values (value(code) * scale is exact in bf16 then), so the fused dequant
  adds nothing beyond the codes themselves.
- Equal keys give the mean of the values; one token gives its own value
  (to the weight split's ~2^-21).
- Repeated calls give identical bits (decode, multi-query, NVFP4): no
  reduction depends on timing.
Values are checked against numpy over the cache bytes decoded with the
oracle's pinned E4M3 table."""
import numpy as np
import pytest
import torch

import oracle
from quantized_decode_attention_calibrate_amd import workloads

from gpu_common import Setup, bits_u8, gpu_or_skip, kvq, say
from test_gpu_nvfp4 import NvSetup

pytestmark = pytest.mark.gpu

POW2 = (2.0 ** -3, 2.0 ** -3)   # k_scale, v_scale: exact dequantized products


@pytest.fixture(scope="module")
def K():
    gpu_or_skip()
    return kvq()


def dequant_bf16(codes: np.ndarray, scale: float) -> torch.Tensor:
    """value(code) * scale as bf16 (exact for a power-of-two scale; the NaN
    codes of unwritten slots stay NaN)."""
    vals = (oracle.e4m3_table()[codes] * scale).astype(np.float32)
    t = torch.from_numpy(vals).to(torch.bfloat16)
    ref = torch.from_numpy(vals)
    fin = torch.isfinite(ref)
    assert torch.equal(t.float()[fin], ref[fin]) and torch.isnan(t.float()[~fin]).all(), "not exact in bf16"
    return t


def attend(K, s, kc, vc, kv, ks, vs, split=0):
    w = s.w
    out = torch.empty(w.B, w.Hq, w.D, dtype=torch.float32, device="cuda")
    ws = K.new_workspace(w.B, w.Hq, w.Hkv, w.D, w.max_seq_len, split)
    K.kvq_paged_decode_attn(s.q, kc, vc, kv, s.bt, s.sl, w.max_seq_len, w.Hkv, ks, vs, s.sm_scale, out, ws,
                            split_tokens=split)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("shape,lens", [(dict(Hq=16, Hkv=2), [1000, 4097, 65]),
                                        (dict(Hq=16, Hkv=4, D=128), [777, 2049]),
                                        (dict(Hq=12, Hkv=2, D=256), [1500, 90])])
def test_fp8_equals_bf16_over_the_dequantized_values(K, shape, lens):
    w = workloads.make("gptoss65k", seed=131, seq_lens=lens, shape=shape)
    s = Setup(w, 1, scales=POW2)
    kb = dequant_bf16(bits_u8(s.kc), POW2[0]).cuda()
    vb = dequant_bf16(bits_u8(s.vc), POW2[1]).cuda()
    for split in (0, 128):
        o8 = attend(K, s, s.kc, s.vc, K.KVQ_KV_FP8_E4M3, *POW2, split=split).cpu().numpy()
        o16 = attend(K, s, kb, vb, K.KVQ_KV_BF16, 1.0, 1.0, split=split).cpu().numpy()
        d = np.abs(o8.astype(np.float64) - o16)
        rel = float(np.sqrt((d ** 2).sum() / (o16.astype(np.float64) ** 2).sum()))
        say(f"  fp8 vs bf16 D={w.D} split={split}: max_abs={d.max():.2e} rel_l2={rel:.2e}")
        # (P enters the BF16 path's MFMAs as bf16 hi + lo, ~2^-16, and the FP8
        # path's as f16 hi + lo, ~2^-21: the rest is fp32 summation order)
        assert d.max() < 3e-5 and rel < 5e-6   # measured: <= 6.6e-6 and 1.0e-6


@pytest.mark.parametrize("kv", [1, 0], ids=["fp8", "bf16"])
def test_equal_keys_give_the_mean_value(K, kv):
    w = workloads.make("gptoss65k", seed=132, seq_lens=[3000, 64, 1], shape=dict(Hq=16, Hkv=2))
    w.k[:] = w.k[0]                          # every token has the same key (per head)
    s = Setup(w, kv, scales=POW2)
    out = attend(K, s, s.kc, s.vc, kv, *POW2 if kv == 1 else (1.0, 1.0)).cpu().numpy()
    # mean over each sequence's tokens of the cached values (decoded from the bytes)
    vb = bits_u8(s.vc)
    if kv == 1:
        vals = oracle.e4m3_table()[vb] * POW2[1]                       # [nb][Hkv][D][16]
    else:
        vals = vb.view(np.uint16).astype(np.uint32) << 16
        vals = vals.view(np.float32).astype(np.float64)
    G = w.Hq // w.Hkv
    for b, L in enumerate(w.seq_lens):
        slots = w.slot_mapping[w.seq_starts[b]:w.seq_starts[b] + L].numpy()
        v = vals[slots // 16, :, :, slots % 16]                       # [L][Hkv][D]
        want = v.mean(axis=0)
        got = out[b].reshape(w.Hkv, G, w.D)
        assert np.abs(got - want[:, None, :]).max() < 1e-5 * max(1.0, np.abs(want).max()), b


@pytest.mark.parametrize("kv", [1, 0], ids=["fp8", "bf16"])
def test_one_token_gives_its_value(K, kv):
    w = workloads.make("gptoss65k", seed=133, seq_lens=[1, 1, 1], shape=dict(Hq=16, Hkv=2))
    s = Setup(w, kv, scales=POW2)
    out = attend(K, s, s.kc, s.vc, kv, *POW2 if kv == 1 else (1.0, 1.0)).cpu().numpy()
    vb = bits_u8(s.vc)
    if kv == 1:
        vals = oracle.e4m3_table()[vb] * POW2[1]
    else:
        vals = (vb.view(np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    G = w.Hq // w.Hkv
    for b in range(w.B):
        slot = int(w.slot_mapping[w.seq_starts[b]])
        want = vals[slot // 16, :, :, slot % 16]                       # [Hkv][D]
        # one weight: the hi + lo split of exp2(~0 + offset) carries it to ~2^-21
        got = out[b].reshape(w.Hkv, G, w.D)
        assert np.abs(got - want[:, None, :]).max() <= 1e-6 * max(1.0, np.abs(want).max()), b


def test_repeated_calls_are_bit_identical(K):
    w = workloads.make("gptoss65k", seed=134, seq_lens=[5000, 700, 64], shape=dict(Hq=16, Hkv=2))
    s = Setup(w, 1)
    outs = [attend(K, s, s.kc, s.vc, 1, s.ks, s.vs, split=256) for _ in range(3)]
    assert all(torch.equal(outs[0], o) for o in outs[1:])
    # multi-query
    q = workloads.mq_queries(w, 4, seed=2).cuda()
    ws = K.new_workspace_mq(w.B, 4, w.Hq, w.Hkv, w.D, w.max_seq_len, 256)
    mq = []
    for _ in range(3):
        o = torch.empty(w.B, 4, w.Hq, w.D, dtype=torch.float32, device="cuda")
        K.kvq_paged_decode_attn_mq(q, s.kc, s.vc, 1, s.bt, s.sl, w.max_seq_len, w.Hkv, s.ks, s.vs, s.sm_scale, o,
                                   ws, split_tokens=256)
        mq.append(o)
    torch.cuda.synchronize()
    assert all(torch.equal(mq[0], o) for o in mq[1:])
    # NVFP4
    n = NvSetup(K, w)
    a = n.attend(torch.float32, split_tokens=256)
    b = n.attend(torch.float32, split_tokens=256)
    assert torch.equal(a, b)
