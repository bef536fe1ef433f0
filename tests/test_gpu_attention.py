"""GPU parity for split-K paged decode attention against the oracle.

Each case writes the caches with kvq_cache_write (checked byte-identical to
the oracle's), runs kvq_paged_decode_attn with the fp32 epilogue and compares
with the oracle's fp64 attention over the same dequantized values: max abs
error <= 2e-3 and relative L2 <= 1e-3.  The bf16 output must equal the fp32
output rounded to nearest even, bit for bit.  Shapes span several 64-token
chunks and splits, ragged tails, empty and one-token sequences, D in
{64, 128, 256} and GQA groups 1..16, for both kernel families and both cache
dtypes.  Invariants: physical block placement changes nothing (bit
identical); the split length changes only rounding; constant V gives that
constant.
"""
import numpy as np
import pytest
import torch

import oracle
from quantized_decode_attention_calibrate_amd import workloads

from gpu_common import Setup, assert_attention_close, bits_u8, gpu_or_skip, kvq, say

pytestmark = pytest.mark.gpu

VALU, MFMA = 1, 2

CASES = [
    # name, seed, seq_lens, shape
    ("tiny", 0, None, None),                                                   # 300, 517; G 2
    ("gptoss65k", 1, [1000, 4097], dict(Hq=16, Hkv=2)),                        # G 8, D 64
    ("mixed64", 2, [1, 0, 2049, 777, 64, 65], dict(Hq=16, Hkv=4, D=128)),       # G 4, D 128
    ("agents126k", 3, [3000, 127], dict(Hq=12, Hkv=2, D=256, calib_tokens=512)),  # G 6, D 256
    ("mixed64", 4, [129, 700], dict(Hq=16, Hkv=1, D=64)),                       # G 16
    ("mixed64", 5, [64, 1500], dict(Hq=2, Hkv=2, D=128)),                       # G 1
    ("mixed64", 6, [700, 33, 1], dict(Hq=16, Hkv=1, D=256)),                    # G 16 at D 256: largest LDS
]


@pytest.fixture(scope="module")
def K():
    gpu_or_skip()
    return kvq()


_cache = {}


def prepared(case, kv):
    key = (case, kv)
    if key not in _cache:
        name, seed, lens, shape = CASES[case]
        w = workloads.make(name, seed=seed, seq_lens=lens, shape=shape)
        s = Setup(w, kv)
        kc, vc = s.oracle_caches()
        assert np.array_equal(bits_u8(s.kc), kc.view(np.uint8)), "cache write differs from oracle"
        assert np.array_equal(bits_u8(s.vc), vc.view(np.uint8)), "cache write differs from oracle"
        ref = s.oracle_attention(kc, vc)
        _cache.clear()
        _cache[key] = (s, ref)
    return _cache[key]


@pytest.mark.parametrize("impl", [VALU, MFMA])
@pytest.mark.parametrize("kv", [1, 0])
@pytest.mark.parametrize("case", range(len(CASES)))
def test_attention_matches_oracle(K, case, kv, impl):
    s, ref = prepared(case, kv)
    say(f"case {CASES[case][0]} lens={s.w.seq_lens} Hq={s.w.Hq} Hkv={s.w.Hkv} D={s.w.D} kv={kv} impl={impl}")
    out32 = s.attend(torch.float32, impl=impl)
    assert_attention_close(out32.cpu().numpy(), ref, f"{CASES[case][0]} kv={kv} impl={impl}")
    out16 = s.attend(torch.bfloat16, impl=impl)
    assert torch.equal(out16.cpu().view(torch.int16), out32.cpu().to(torch.bfloat16).view(torch.int16))
    # empty sequences give exact zeros
    for b, L in enumerate(s.w.seq_lens):
        if L == 0:
            assert (out32[b] == 0).all()


@pytest.mark.parametrize("impl", [VALU, MFMA])
def test_split_length_only_changes_rounding(K, impl):
    s, ref = prepared(1, 1)
    outs = [s.attend(torch.float32, impl=impl, split_tokens=st).cpu().numpy() for st in (64, 192, 1024, 8192)]
    for o in outs:
        assert_attention_close(o, ref, f"split impl={impl}")
    assert np.abs(outs[0] - outs[-1]).max() < 2e-5


def test_families_agree(K):
    s, ref = prepared(3, 1)
    a = s.attend(torch.float32, impl=VALU).cpu().numpy()
    b = s.attend(torch.float32, impl=MFMA).cpu().numpy()
    assert np.abs(a - b).max() < 2e-3


@pytest.mark.parametrize("impl", [VALU, MFMA])
def test_physical_placement_is_bit_identical(K, impl):
    w = workloads.make("gptoss65k", seed=7, seq_lens=[900, 333], shape=dict(Hq=16, Hkv=2))
    s1 = Setup(w, 1)
    perm = torch.randperm(w.num_blocks, generator=torch.Generator().manual_seed(3))
    bt2 = perm[w.block_tables.long()].to(torch.int32)
    for b, L in enumerate(w.seq_lens):
        bt2[b, (L + 15) // 16:] = 0
    slots2 = perm[w.slot_mapping // 16] * 16 + w.slot_mapping % 16
    w2 = workloads.Workload(**{**w.__dict__, "block_tables": bt2, "slot_mapping": slots2})
    s2 = Setup(w2, 1, scales=(s1.ks, s1.vs))
    o1 = s1.attend(torch.float32, impl=impl)
    o2 = s2.attend(torch.float32, impl=impl)
    assert torch.equal(o1, o2)


def test_contiguous_layout_is_bit_identical(K):
    """The benchmark's contiguous-block layout (physical blocks in logical
    order) gives the permuted layout's outputs bit for bit."""
    w = workloads.make("gptoss65k", seed=7, seq_lens=[900, 333], shape=dict(Hq=16, Hkv=2))
    wc = workloads.make("gptoss65k", seed=7, seq_lens=[900, 333], shape=dict(Hq=16, Hkv=2), contiguous=True)
    assert torch.equal(w.k, wc.k) and not torch.equal(w.block_tables, wc.block_tables)
    s1 = Setup(w, 1)
    s2 = Setup(wc, 1, scales=(s1.ks, s1.vs))
    assert torch.equal(s1.attend(torch.float32, impl=MFMA), s2.attend(torch.float32, impl=MFMA))


@pytest.mark.parametrize("impl", [VALU, MFMA])
def test_constant_values_give_the_constant(K, impl):
    w = workloads.make("gptoss65k", seed=8, seq_lens=[2000, 5], shape=dict(Hq=16, Hkv=2))
    w.v[:] = 1.5
    s = Setup(w, 1, scales=(0.05, 1.0 / 64))
    out = s.attend(torch.float32, impl=impl).cpu().numpy()
    assert np.abs(out - 1.5).max() < 1e-5
