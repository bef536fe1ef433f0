"""GPU parity for multi-query decode (the verification step of speculative
decoding) against the oracle's causal multi-query attention.

The q_len newest tokens of each sequence are in the cache; query i attends
to tokens 0 .. L - q_len + i.  Shapes cover every column-tile count (G * q_len
up to 16, 32 and 64), D 64 / 128 / 256, several splits with a split boundary
inside the last q_len tokens, sequences shorter than q_len (queries before
the start give 0) and empty ones, for FP8, BF16 and NVFP4 caches.  Checks:
max abs 2e-3 / rel L2 1e-3 against the oracle's fp64 (fp32 epilogue), bf16
output = RNE(fp32 output), and q_len = 1 through the multi-query call, as
well as the newest query of any q_len, equal the single-token decode bit for
bit (FP8 / BF16: same kernel arithmetic per column).
"""
import math

import numpy as np
import pytest
import torch

import oracle
from quantized_decode_attention_calibrate_amd import workloads

from gpu_common import Setup, assert_attention_close, gpu_or_skip, kvq, say
from test_gpu_nvfp4 import NvSetup

pytestmark = pytest.mark.gpu

CASES = [
    # name, seed, seq_lens, shape, q_len, split_tokens
    ("gptoss65k", 21, [1000, 4097, 3], dict(Hq=16, Hkv=2), 2, 0),          # G 8 x 2 = 16 columns
    ("gptoss65k", 22, [700, 130, 0], dict(Hq=16, Hkv=2), 4, 128),          # 32 columns, split inside the tail
    ("gptoss65k", 23, [2049, 64, 5], dict(Hq=16, Hkv=2), 8, 64),           # 64 columns, q_len > L for one seq
    ("mixed64", 24, [777, 1500], dict(Hq=16, Hkv=4, D=128), 8, 256),        # G 4 x 8 = 32 at D 128
    ("agents126k", 25, [1200, 97], dict(Hq=12, Hkv=2, D=256, calib_tokens=256), 2, 0),  # G 6 x 2 at D 256
    ("mixed64", 26, [300, 16], dict(Hq=2, Hkv=2, D=64), 16, 64),            # G 1 x 16
]


@pytest.fixture(scope="module")
def K():
    gpu_or_skip()
    return kvq()


def run_mq(K, s, q, kv, split_tokens, dtype=torch.float32, window=0, bt=None):
    w = s.w
    B, q_len = q.shape[0], q.shape[1]
    out = torch.empty(B, q_len, w.Hq, w.D, dtype=dtype, device="cuda")
    ws = K.new_workspace_mq(B, q_len, w.Hq, w.Hkv, w.D, w.max_seq_len, split_tokens, window=window)
    sl = torch.tensor(w.seq_lens, dtype=torch.int32, device="cuda")
    bt = (w.block_tables if bt is None else bt).cuda()
    if kv == 2:
        K.kvq_nvfp4_paged_decode_attn_mq(q.cuda(), s.kc, s.vc, bt, sl, w.max_seq_len, w.Hkv, s.gk, s.gv, s.sm,
                                         out, ws, split_tokens=split_tokens, window=window)
    else:
        K.kvq_paged_decode_attn_mq(q.cuda(), s.kc, s.vc, kv, bt, s.sl, w.max_seq_len, w.Hkv, s.ks, s.vs,
                                   s.sm_scale, out, ws, split_tokens=split_tokens, window=window)
    torch.cuda.synchronize()
    return out


def oracle_mq(s, q, kv, window=0):
    w = s.w
    if kv == 2:
        okc, ovc = oracle.new_caches(oracle.KV_NVFP4, w.num_blocks, w.Hkv, w.D, 16, fill=0xFF)
        oracle.nvfp4_cache_write(w.k, w.v, w.slot_mapping, okc, ovc, 16, s.gk, s.gv)
        return oracle.decode_attn_mq(q, okc, ovc, oracle.KV_NVFP4, w.block_tables, w.seq_lens, w.Hkv, 16,
                                     s.gk, s.gv, s.sm, nthreads=8, window=window)
    kc, vc = s.oracle_caches()
    kvd = oracle.KV_FP8 if kv == 1 else oracle.KV_BF16
    return oracle.decode_attn_mq(q, kc, vc, kvd, w.block_tables, w.seq_lens, w.Hkv, 16, s.ks, s.vs, s.sm_scale,
                                 nthreads=8, window=window)


def setup(K, w, kv):
    return NvSetup(K, w) if kv == 2 else Setup(w, kv)


@pytest.mark.parametrize("kv", [1, 0, 2])
@pytest.mark.parametrize("case", range(len(CASES)))
def test_multiquery_matches_oracle(K, case, kv):
    name, seed, lens, shape, q_len, split = CASES[case]
    w = workloads.make(name, seed=seed, seq_lens=lens, shape=shape)
    say(f"mq case {case}: lens={lens} Hq={w.Hq} Hkv={w.Hkv} D={w.D} q_len={q_len} split={split} kv={kv}")
    s = setup(K, w, kv)
    q = workloads.mq_queries(w, q_len, seed=seed)
    ref = oracle_mq(s, q, kv)
    out32 = run_mq(K, s, q, kv, split)
    assert_attention_close(out32.cpu().numpy(), ref, f"mq case={case} kv={kv}")
    out16 = run_mq(K, s, q, kv, split, torch.bfloat16)
    assert torch.equal(out16.cpu().view(torch.int16), out32.cpu().to(torch.bfloat16).view(torch.int16))
    for b, L in enumerate(w.seq_lens):   # queries before the sequence start, and empty sequences
        for i in range(q_len):
            if L - q_len + 1 + i <= 0:
                assert (out32[b, i] == 0).all()


@pytest.mark.parametrize("kv", [1, 0])
def test_single_query_paths_agree_bitwise(K, kv):
    name, seed, lens, shape, q_len, split = CASES[2]
    w = workloads.make(name, seed=seed, seq_lens=[2049, 64, 9], shape=shape)
    s = Setup(w, kv)
    one = s.attend(torch.float32, impl=2, split_tokens=64)
    mq1 = run_mq(K, s, w.q[:, None], kv, 64)
    assert torch.equal(mq1[:, 0], one)
    for ql in (2, 4, 8):   # the newest query sees the whole sequence
        q = workloads.mq_queries(w, ql, seed=5)
        assert torch.equal(run_mq(K, s, q, kv, 64)[:, ql - 1], one), ql


def test_multiquery_rejects_unsupported_shapes(K):
    w = workloads.make("agents126k", seed=1, seq_lens=[100], shape=dict(Hq=12, Hkv=2, D=256, calib_tokens=64))
    s = Setup(w, 1)
    q = workloads.mq_queries(w, 3, seed=1)   # G 6 x 3 = 18 columns > 16 at D 256
    with pytest.raises(K.KvqError):
        run_mq(K, s, q, 1, 0)
