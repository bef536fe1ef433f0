"""GPU parity for the block-scaled 4-bit (NVFP4-style) path against the oracle.

- E2M1 decode of all 256 code bytes (both nibbles) times every non-negative
  finite E4M3 block-scale code, built as the decode kernel builds its f16
  operands, equals value(code) * value(scale) exactly;
- kvq_nvfp4_cache_write produces byte-identical caches to the oracle's NVFP4
  write (codes, block scales, untouched bytes, and the other token's nibble
  in shared V bytes);
- NVFP4 decode attention matches the oracle's fp64 attention over the same
  dequantized values within max abs 2e-3 / rel L2 1e-3 (fp32 epilogue), and
  bf16 output equals the fp32 output rounded to nearest even; physical block
  placement changes nothing.  The full 2 x 131,072 shape is checked on every
  unit in test_gpu_fullsize.py.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from quantized_decode_attention_calibrate_amd import workloads

from gpu_common import assert_attention_close, gpu_or_skip, kvq, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def K():
    gpu_or_skip()
    return kvq()


def test_e2m1_decode_all_codes_and_scales(K):
    codes = torch.arange(256, dtype=torch.uint8, device="cuda")
    e2 = np.array([oracle.e2m1_value(c) for c in range(16)])
    want_lo, want_hi = e2[np.arange(256) & 15], e2[np.arange(256) >> 4]
    table = oracle.e4m3_table()
    out = torch.empty(512, dtype=torch.float16, device="cuda")
    for sc in range(0, 0x7F):            # every non-negative finite block-scale code
        K.kvq_e2m1_decode(codes, sc, out)
        got = out.float().cpu().double().numpy().reshape(256, 2)
        assert np.array_equal(got[:, 0], want_lo * table[sc]) and np.array_equal(got[:, 1], want_hi * table[sc]), sc
        if sc:
            assert np.array_equal(np.signbit(got[:, 0]), np.signbit(want_lo))


def gpu_gscales(K, w):
    amax = torch.zeros(2, dtype=torch.float32, device="cuda")
    K.kvq_amax_bf16(w.k.cuda(), amax[0:1])
    K.kvq_amax_bf16(w.v.cuda(), amax[1:2])
    return K.kvq_nvfp4_calibrate(amax.cpu().tolist())


def write_both(K, w, slots, gk, gv, fill=0xFF):
    kc, vc = K.new_nvfp4_caches(w.num_blocks, w.Hkv, w.D)
    kc.fill_(fill)
    vc.fill_(fill)
    K.kvq_nvfp4_cache_write(w.k.cuda(), w.v.cuda(), slots.cuda(), kc, vc, gk, gv)
    okc, ovc = oracle.new_caches(oracle.KV_NVFP4, w.num_blocks, w.Hkv, w.D, 16, fill=fill)
    oracle.nvfp4_cache_write(w.k, w.v, slots, okc, ovc, 16, gk, gv)
    return kc, vc, okc, ovc


@pytest.mark.parametrize("name,seed,lens,shape", [
    ("tiny", 0, None, None),
    ("mixed64", 1, [33, 1, 250, 0], dict(Hq=8, Hkv=2, D=128)),
    ("agents126k", 2, [70, 19], dict(Hq=12, Hkv=2, D=256, calib_tokens=64)),
])
def test_nvfp4_cache_write_matches_oracle(K, name, seed, lens, shape):
    w = workloads.make(name, seed=seed, seq_lens=lens, shape=shape)
    gk, gv = gpu_gscales(K, w)
    kc, vc, okc, ovc = write_both(K, w, w.slot_mapping, gk, gv)
    assert np.array_equal(kc.cpu().numpy(), okc) and np.array_equal(vc.cpu().numpy(), ovc)


def test_nvfp4_write_keeps_the_other_nibble(K):
    # write only even tokens, then only odd ones, over a sentinel: shared V
    # bytes must end up identical to the oracle's, nibble by nibble
    w = workloads.make("tiny", seed=3, seq_lens=[64, 37])
    gk, gv = gpu_gscales(K, w)
    even = w.slot_mapping.clone()
    even[1::2] = -1
    odd = w.slot_mapping.clone()
    odd[0::2] = -1
    kc, vc, okc, ovc = write_both(K, w, even, gk, gv, fill=0x5A)
    assert np.array_equal(vc.cpu().numpy(), ovc)
    K.kvq_nvfp4_cache_write(w.k.cuda(), w.v.cuda(), odd.cuda(), kc, vc, gk, gv)
    oracle.nvfp4_cache_write(w.k, w.v, odd, okc, ovc, 16, gk, gv)
    assert np.array_equal(kc.cpu().numpy(), okc) and np.array_equal(vc.cpu().numpy(), ovc)


@pytest.mark.parametrize("order", ["offset5", "offset1_reversed", "shuffled", "pairs_split"])
def test_nvfp4_write_any_slot_order(K, order):
    # windows of 16 input tokens write whole V bytes when both slots of a byte
    # are adjacent in the window, else nibbles; every order must give the
    # oracle's bytes
    w = workloads.make("mixed64", seed=11, seq_lens=[203], shape=dict(Hq=4, Hkv=2, D=64))
    T, nb = w.T, 16
    if order == "offset5":
        sm = torch.arange(T, dtype=torch.int64) + 5
    elif order == "offset1_reversed":
        sm = torch.arange(T, dtype=torch.int64).flip(0) + 1
    elif order == "shuffled":
        sm = torch.randperm(nb * 16, generator=torch.Generator().manual_seed(3))[:T].to(torch.int64)
    else:   # token 2j -> slot 2j+1 and 2j+1 -> 2j: partners adjacent but swapped
        sm = torch.arange(T, dtype=torch.int64) ^ 1
    gk, gv = gpu_gscales(K, w)
    kc, vc = K.new_nvfp4_caches(nb, w.Hkv, w.D)
    kc.fill_(0x3C)
    vc.fill_(0x3C)
    K.kvq_nvfp4_cache_write(w.k.cuda(), w.v.cuda(), sm.cuda(), kc, vc, gk, gv)
    okc, ovc = oracle.new_caches(oracle.KV_NVFP4, nb, w.Hkv, w.D, 16, fill=0x3C)
    oracle.nvfp4_cache_write(w.k, w.v, sm, okc, ovc, 16, gk, gv)
    assert np.array_equal(kc.cpu().numpy(), okc) and np.array_equal(vc.cpu().numpy(), ovc)


CASES = [
    ("tiny", 0, None, None),
    ("nvfp4_131k", 1, [1000, 4097], dict(Hq=16, Hkv=2)),
    ("mixed64", 2, [1, 0, 2049, 777, 65], dict(Hq=16, Hkv=4, D=128)),
    ("agents126k", 3, [3000, 127], dict(Hq=12, Hkv=2, D=256, calib_tokens=256)),
    ("mixed64", 4, [129, 700], dict(Hq=16, Hkv=1, D=64)),
]


class NvSetup:
    def __init__(self, K, w, scales=None, write_newest=True):
        self.K, self.w = K, w
        self.gk, self.gv = scales if scales is not None else gpu_gscales(K, w)
        self.kc, self.vc = K.new_nvfp4_caches(w.num_blocks, w.Hkv, w.D)
        self.kc.fill_(0xFF)
        self.vc.fill_(0xFF)
        K.kvq_nvfp4_cache_write(w.k.cuda(), w.v.cuda(), w.prefill_slots().cuda(), self.kc, self.vc, self.gk, self.gv)
        rows = w.last_token_rows()
        rows = rows[rows >= 0]
        if write_newest:
            K.kvq_nvfp4_cache_write(w.k[rows].cuda(), w.v[rows].cuda(), w.slot_mapping[rows].contiguous().cuda(),
                                    self.kc, self.vc, self.gk, self.gv)
        self.sm = float(np.float32(1.0 / math.sqrt(w.D)))

    def attend(self, dtype=torch.float32, split_tokens=0, bt=None):
        w, K = self.w, self.K
        out = torch.empty(w.B, w.Hq, w.D, dtype=dtype, device="cuda")
        ws = K.new_workspace(w.B, w.Hq, w.Hkv, w.D, w.max_seq_len, split_tokens)
        sl = torch.tensor(w.seq_lens, dtype=torch.int32, device="cuda")
        K.kvq_nvfp4_paged_decode_attn(w.q.cuda(), self.kc, self.vc, (w.block_tables if bt is None else bt).cuda(),
                                      sl, w.max_seq_len, w.Hkv, self.gk, self.gv, self.sm, out, ws,
                                      split_tokens=split_tokens)
        torch.cuda.synchronize()
        return out

    def oracle(self):
        w = self.w
        okc, ovc = oracle.new_caches(oracle.KV_NVFP4, w.num_blocks, w.Hkv, w.D, 16, fill=0xFF)
        oracle.nvfp4_cache_write(w.k, w.v, w.slot_mapping, okc, ovc, 16, self.gk, self.gv)
        assert np.array_equal(self.kc.cpu().numpy(), okc) and np.array_equal(self.vc.cpu().numpy(), ovc)
        return oracle.decode_attn(w.q, okc, ovc, oracle.KV_NVFP4, w.block_tables, w.seq_lens, w.Hkv, 16,
                                  self.gk, self.gv, self.sm, nthreads=8)


@pytest.mark.parametrize("case", range(len(CASES)))
def test_nvfp4_attention_matches_oracle(K, case):
    name, seed, lens, shape = CASES[case]
    w = workloads.make(name, seed=seed, seq_lens=lens, shape=shape)
    s = NvSetup(K, w)
    ref = s.oracle()
    out32 = s.attend(torch.float32)
    assert_attention_close(out32.cpu().numpy(), ref, f"nvfp4 {name} lens={w.seq_lens} D={w.D} G={w.G}")
    out16 = s.attend(torch.bfloat16)
    assert torch.equal(out16.cpu().view(torch.int16), out32.cpu().to(torch.bfloat16).view(torch.int16))
    for b, L in enumerate(w.seq_lens):
        if L == 0:
            assert (out32[b] == 0).all()
    for st in (64, 192):
        assert_attention_close(s.attend(torch.float32, split_tokens=st).cpu().numpy(), ref, f"  split {st}")


def test_nvfp4_physical_placement_is_bit_identical(K):
    w = workloads.make("nvfp4_131k", seed=7, seq_lens=[900, 333], shape=dict(Hq=16, Hkv=2))
    s1 = NvSetup(K, w)
    perm = torch.randperm(w.num_blocks, generator=torch.Generator().manual_seed(3))
    bt2 = perm[w.block_tables.long()].to(torch.int32)
    for b, L in enumerate(w.seq_lens):
        bt2[b, (L + 15) // 16:] = 0
    slots2 = perm[w.slot_mapping // 16] * 16 + w.slot_mapping % 16
    w2 = workloads.Workload(**{**w.__dict__, "block_tables": bt2, "slot_mapping": slots2})
    s2 = NvSetup(K, w2, scales=(s1.gk, s1.gv))
    assert torch.equal(s1.attend(), s2.attend())
