"""GPU parity for sliding-window decode against the oracle.

Query i (token position p = L - q_len + i) sees tokens max(0, p - W + 1) .. p.
Windows of 1, 16, 100, 128 and 1000 tokens over sequences whose window
starts mid-block and mid-chunk, with several splits, single and multi-query,
FP8 / BF16 / NVFP4 caches: max abs 2e-3 / rel L2 1e-3 against the oracle's
fp64, bf16 = RNE(fp32).  Block-table entries of blocks wholly before the
first query's window are replaced by a block full of 0xFF (NaN codes in every
format) and the result must not change: the kernel never reads them.  A
window at least as long as the sequence equals full attention bit for bit.
"""
import numpy as np
import pytest
import torch

import oracle
from quantized_decode_attention_calibrate_amd import workloads

from gpu_common import assert_attention_close, gpu_or_skip, kvq, say
from test_gpu_multiquery import oracle_mq, run_mq, setup

pytestmark = pytest.mark.gpu

CASES = [
    # name, seed, seq_lens, shape, q_len, window, split_tokens
    ("gptoss65k", 41, [1000, 4097, 70], dict(Hq=16, Hkv=2), 1, 128, 0),
    ("gptoss65k", 42, [3001, 700, 3], dict(Hq=16, Hkv=2), 3, 100, 64),
    ("gptoss65k", 43, [2500, 129], dict(Hq=16, Hkv=2), 1, 1, 0),
    ("mixed64", 44, [777, 1500, 16], dict(Hq=16, Hkv=4, D=128), 4, 1000, 128),
    ("agents126k", 45, [1200, 97], dict(Hq=12, Hkv=2, D=256, calib_tokens=256), 2, 16, 64),
]


@pytest.fixture(scope="module")
def K():
    gpu_or_skip()
    return kvq()


def poisoned_table(w, q_len, window, kv_bytes_fill):
    """Block ids of blocks wholly before every query's window -> an extra block
    (index num_blocks) that the caller fills with 0xFF."""
    bt = w.block_tables.clone()
    for b, L in enumerate(w.seq_lens):
        first = max(0, L - q_len - window + 1)
        bt[b, :first // 16] = w.num_blocks
    return bt


@pytest.mark.parametrize("kv", [1, 0, 2])
@pytest.mark.parametrize("case", range(len(CASES)))
def test_window_matches_oracle(K, case, kv):
    name, seed, lens, shape, q_len, W, split = CASES[case]
    w = workloads.make(name, seed=seed, seq_lens=lens, shape=shape)
    say(f"window case {case}: lens={lens} Hq={w.Hq} Hkv={w.Hkv} D={w.D} q_len={q_len} W={W} split={split} kv={kv}")
    # one spare block at index num_blocks for the poisoned table entries
    w_spare = workloads.Workload(**{**w.__dict__, "num_blocks": w.num_blocks + 1})
    s = setup(K, w_spare, kv)
    s.kc.view(torch.uint8)[w.num_blocks].fill_(0xFF)
    s.vc.view(torch.uint8)[w.num_blocks].fill_(0xFF)
    q = workloads.mq_queries(w, q_len, seed=seed)
    ref = oracle_mq(s, q, kv, window=W)
    out32 = run_mq(K, s, q, kv, split, window=W)
    assert_attention_close(out32.cpu().numpy(), ref, f"window case={case} kv={kv}")
    out16 = run_mq(K, s, q, kv, split, torch.bfloat16, window=W)
    assert torch.equal(out16.cpu().view(torch.int16), out32.cpu().to(torch.bfloat16).view(torch.int16))
    poisoned = run_mq(K, s, q, kv, split, window=W, bt=poisoned_table(w, q_len, W, 0xFF))
    assert torch.equal(poisoned, out32)


@pytest.mark.parametrize("kv", [1, 2])
def test_wide_window_is_full_attention(K, kv):
    w = workloads.make("gptoss65k", seed=46, seq_lens=[900, 333], shape=dict(Hq=16, Hkv=2))
    s = setup(K, w, kv)
    q = workloads.mq_queries(w, 2, seed=1)
    full = run_mq(K, s, q, kv, 128)
    wide = run_mq(K, s, q, kv, 128, window=900)
    assert torch.equal(full, wide)
