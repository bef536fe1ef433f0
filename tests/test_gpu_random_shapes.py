"""Randomized shape coverage of the decode path against the oracle.

Each case draws, from its own fixed seed, a head dim, GQA group, KV head
count, query count, batch of sequence lengths (empty, one token, around
block and chunk boundaries, several splits), sliding window, split length
and cache format (FP8, BF16, NVFP4), within the shapes the library supports,
and compares the multi-query call with the oracle's causal attention (max abs
2e-3 / rel L2 1e-3, fp32 epilogue).  Single-query cases without a window also
run the one-call step (kvq_paged_decode_attn_append) on caches that hold the
prefill only, and check its cache bytes against the oracle's write and its
output against the multi-query call, bit for bit."""
import numpy as np
import pytest
import torch

from quantized_decode_attention_calibrate_amd import workloads

from gpu_common import Setup, assert_attention_close, bits_u8, gpu_or_skip, kvq, say
from test_gpu_multiquery import oracle_mq, run_mq, setup

pytestmark = pytest.mark.gpu

LENS = [0, 1, 2, 15, 16, 17, 63, 64, 65, 200, 511, 512, 513, 1000, 2047, 3001]
N_CASES = 30


def draw(i):
    r = np.random.default_rng(7000 + i)
    D = int(r.choice([64, 128, 256]))
    cols = {64: 64, 128: 32, 256: 16}[D]          # columns G * q_len the kernel holds at this D
    G = int(r.choice([g for g in (1, 2, 3, 4, 6, 8, 16) if g <= cols]))
    q_len = int(r.integers(1, min(16, cols // G) + 1))
    Hkv = int(r.choice([1, 2, 3]))
    lens = [int(x) for x in r.choice(LENS, size=int(r.integers(1, 5)))]
    window = int(r.choice([0, 0, 0, 1, 7, 64, 100, 700]))
    split = int(r.choice([0, 64, 128, 192, 512]))
    kv = int(r.choice([1, 0, 2]))
    return dict(D=D, G=G, Hkv=Hkv, q_len=q_len, lens=lens, window=window, split=split, kv=kv)


@pytest.fixture(scope="module")
def K():
    gpu_or_skip()
    return kvq()


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_shape_matches_oracle(K, i):
    c = draw(i)
    say(f"random case {i}: {c}")
    w = workloads.make("mixed64", seed=7000 + i, seq_lens=c["lens"],
                       shape=dict(Hq=c["G"] * c["Hkv"], Hkv=c["Hkv"], D=c["D"]))
    s = setup(K, w, c["kv"])
    q = workloads.mq_queries(w, c["q_len"], seed=i)
    ref = oracle_mq(s, q, c["kv"], window=c["window"])
    got = run_mq(K, s, q, c["kv"], c["split"], window=c["window"])
    assert_attention_close(got.cpu().numpy(), ref, f"random case {i}")

    if c["q_len"] == 1 and c["window"] == 0 and c["kv"] != 2:
        fused = Setup(w, c["kv"], scales=(s.ks, s.vs), write_newest=False)
        rows = w.last_token_rows()
        safe = rows.clamp(min=0)
        slots = torch.where(rows >= 0, w.slot_mapping[safe], torch.full_like(rows, -1)).cuda()
        out = torch.empty(w.B, w.Hq, w.D, dtype=torch.float32, device="cuda")
        ws = K.new_workspace(w.B, w.Hq, w.Hkv, w.D, w.max_seq_len, c["split"])
        K.kvq_paged_decode_attn_append(w.k[safe].contiguous().cuda(), w.v[safe].contiguous().cuda(), slots,
                                       q[:, 0].contiguous().cuda(), fused.kc, fused.vc, c["kv"], fused.bt, fused.sl,
                                       w.max_seq_len, w.Hkv, s.ks, s.vs, s.sm_scale, out, ws,
                                       split_tokens=c["split"])
        torch.cuda.synchronize()
        kc_ref, vc_ref = fused.oracle_caches()
        assert np.array_equal(bits_u8(fused.kc).reshape(-1), kc_ref.view(np.uint8).reshape(-1))
        assert np.array_equal(bits_u8(fused.vc).reshape(-1), vc_ref.view(np.uint8).reshape(-1))
        assert np.array_equal(out.cpu().numpy().view(np.uint32), got[:, 0].cpu().numpy().view(np.uint32))
