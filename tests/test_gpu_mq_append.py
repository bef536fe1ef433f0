"""GPU parity for the speculative-verification step in one launch
(kvq_paged_decode_attn_mq_append): the q_len new tokens of every sequence
are written by the waves that read them, and all q_len queries attend.

The caches hold everything but the q_len newest tokens of each sequence
(unwritten slots poisoned with 0xFF, an FP8 and a bf16 NaN), so a new token
read before it was written would poison its sequence.  Checked against the
oracle (every cache byte equals its write of all tokens; attention within
the path's tolerance) and against the two-launch step on the same inputs
(kvq_cache_write of the new tokens, then kvq_paged_decode_attn_mq): the same
cache bytes and bit-identical outputs.  Cases: new tokens inside one chunk,
across a chunk boundary, across a split boundary (64-token splits), a
sequence shorter than q_len and one exactly q_len long, an empty sequence,
skipped slots, a sliding window, q_len 1 to 16, D 64, 128 and 256, FP8 and BF16.
At q_len 1 both entry points run the one-token writer; the single-token
call kvq_paged_decode_attn_append is checked the same way."""
import numpy as np
import pytest
import torch

import oracle
from quantized_decode_attention_calibrate_amd import workloads

from gpu_common import assert_attention_close, bits_u8, gpu_or_skip, gpu_calibrate, kvq, say

pytestmark = pytest.mark.gpu

CASES = [
    # seed, seq_lens, shape, q_len, split, window
    (151, [1000, 130, 64, 4, 2, 0], dict(Hq=16, Hkv=2), 4, 0, 0),       # 130: across chunk 128; 4 = q_len; 2 < q_len
    (152, [1000, 130, 67, 70], dict(Hq=16, Hkv=2), 8, 64, 0),          # 64-token splits: 67 and 70 cross a split
    (153, [777, 2049, 33], dict(Hq=16, Hkv=4, D=128), 8, 256, 0),       # D 128, two column tiles
    (154, [500, 129, 16], dict(Hq=4, Hkv=4), 16, 0, 0),                 # q_len 16, G 1
    (155, [900, 260], dict(Hq=16, Hkv=2), 4, 128, 100),                 # sliding window
    (156, [300, 65], dict(Hq=16, Hkv=2), 1, 64, 0),                     # one new token
    (159, [300, 65, 1], dict(Hq=16, Hkv=2), 1, 64, 40),                # one new token, window: the multi-query entry
    # D 256 (agents126k-shaped, G 6, 12 columns): a writer lane holds 4 dims (8-byte
    # bf16 row loads, 4-byte FP8 / 8-byte BF16 K stores); 65 and 129: across a chunk
    (160, [300, 65, 129, 2], dict(Hq=12, Hkv=2, D=256, calib_tokens=64), 2, 0, 0),
    (161, [200, 65, 128], dict(Hq=12, Hkv=2, D=256, calib_tokens=64), 2, 64, 0),   # 64-token splits: 65 crosses one
]


@pytest.fixture(scope="module")
def K():
    gpu_or_skip()
    return kvq()


def new_rows(w, q_len):
    """bf16 [B][q_len][Hkv][D] rows of the q_len newest tokens and their slots
    [B][q_len] (-1 for positions below 0)."""
    k = torch.zeros(w.B, q_len, w.Hkv, w.D, dtype=torch.bfloat16)
    v = torch.zeros_like(k)
    slots = torch.full((w.B, q_len), -1, dtype=torch.int64)
    for b, L in enumerate(w.seq_lens):
        for i in range(q_len):
            p = L - q_len + i
            if p >= 0:
                row = w.seq_starts[b] + p
                k[b, i], v[b, i] = w.k[row], w.v[row]
                slots[b, i] = w.slot_mapping[row]
    return k, v, slots


def prefill_caches(K, w, kv, ks, vs, q_len):
    """Caches with every token but the q_len newest of each sequence."""
    kc, vc = K.new_caches(kv, w.num_blocks, w.Hkv, w.D)
    kc.view(torch.uint8).fill_(0xFF)
    vc.view(torch.uint8).fill_(0xFF)
    sm = w.slot_mapping.clone()
    for b, L in enumerate(w.seq_lens):
        sm[w.seq_starts[b] + max(L - q_len, 0):w.seq_starts[b] + L] = -1
    if w.T:
        K.kvq_cache_write(w.k.cuda(), w.v.cuda(), sm.cuda(), kc, vc, kv, ks, vs)
    return kc, vc


@pytest.mark.parametrize("kv", [1, 0], ids=["fp8", "bf16"])
@pytest.mark.parametrize("case", range(len(CASES)))
def test_mq_append_matches_oracle_and_two_launches(K, case, kv):
    seed, lens, shape, q_len, split, window = CASES[case]
    w = workloads.make("gptoss65k", seed=seed, seq_lens=lens, shape=shape)
    say(f"mq append case {case} kv={kv}: lens={lens} q_len={q_len} D={w.D} split={split} window={window}")
    if kv == 1:
        ks, vs = gpu_calibrate(K, w.k.cuda()), gpu_calibrate(K, w.v.cuda())
    else:
        ks = vs = 1.0
    sm = float(np.float32(1.0 / np.sqrt(w.D)))
    q = workloads.mq_queries(w, q_len, seed=seed).cuda()
    k_new, v_new, slots = new_rows(w, q_len)
    k_new, v_new, slots = k_new.cuda(), v_new.cuda(), slots.cuda()
    bt = w.block_tables.cuda()
    sl = torch.tensor(w.seq_lens, dtype=torch.int32, device="cuda")

    # one launch
    kc, vc = prefill_caches(K, w, kv, ks, vs, q_len)
    out = torch.empty(w.B, q_len, w.Hq, w.D, dtype=torch.float32, device="cuda")
    ws = K.new_workspace_mq(w.B, q_len, w.Hq, w.Hkv, w.D, w.max_seq_len, split, window=window)
    if q_len == 1 and window == 0:   # the single-token entry point: the same one-token writer
        K.kvq_paged_decode_attn_append(k_new[:, 0], v_new[:, 0], slots[:, 0].contiguous(), q[:, 0].contiguous(), kc,
                                       vc, kv, bt, sl, w.max_seq_len, w.Hkv, ks, vs, sm, out[:, 0], ws,
                                       split_tokens=split)
    else:
        K.kvq_paged_decode_attn_mq_append(k_new, v_new, slots, q, kc, vc, kv, bt, sl, w.max_seq_len, w.Hkv, ks, vs,
                                          sm, out, ws, split_tokens=split, window=window)
    torch.cuda.synchronize()

    # the oracle: caches with all tokens, multi-query attention
    kvd = oracle.KV_FP8 if kv == 1 else oracle.KV_BF16
    fill = 0xFF if kv == 1 else 0xFFFF
    okc, ovc = oracle.new_caches(kvd, w.num_blocks, w.Hkv, w.D, 16, fill=fill)
    oracle.cache_write(w.k, w.v, w.slot_mapping, okc, ovc, kvd, ks, vs)
    assert np.array_equal(bits_u8(kc).reshape(-1), okc.view(np.uint8).reshape(-1))
    assert np.array_equal(bits_u8(vc).reshape(-1), ovc.view(np.uint8).reshape(-1))
    ref = oracle.decode_attn_mq(q.cpu(), okc, ovc, kvd, w.block_tables, w.seq_lens, w.Hkv, 16, ks, vs, sm,
                                nthreads=8, window=window)
    got = out.cpu().numpy()
    assert_attention_close(got, ref, f"mq append case {case} kv={kv}")

    # two launches on the same inputs
    kc2, vc2 = prefill_caches(K, w, kv, ks, vs, q_len)
    K.kvq_cache_write(k_new.view(-1, w.Hkv, w.D), v_new.view(-1, w.Hkv, w.D), slots.view(-1), kc2, vc2, kv, ks, vs)
    out2 = torch.empty_like(out)
    K.kvq_paged_decode_attn_mq(q, kc2, vc2, kv, bt, sl, w.max_seq_len, w.Hkv, ks, vs, sm, out2, ws,
                               split_tokens=split, window=window)
    torch.cuda.synchronize()
    assert torch.equal(kc2.view(torch.uint8), kc.view(torch.uint8))
    assert torch.equal(vc2.view(torch.uint8), vc.view(torch.uint8))
    assert torch.equal(out2.view(torch.int32), out.view(torch.int32))


def test_mq_append_skipped_slots_write_nothing(K):
    w = workloads.make("gptoss65k", seed=157, seq_lens=[400, 90], shape=dict(Hq=16, Hkv=2))
    q_len = 4
    ks, vs = gpu_calibrate(K, w.k.cuda()), gpu_calibrate(K, w.v.cuda())
    kc, vc = prefill_caches(K, w, 1, ks, vs, q_len)
    before_k, before_v = bits_u8(kc).copy(), bits_u8(vc).copy()
    k_new, v_new, slots = new_rows(w, q_len)
    skip = slots.clone()
    skip[0, 1] = -1
    skip[1, :] = -1
    q = workloads.mq_queries(w, q_len, seed=3).cuda()
    out = torch.empty(w.B, q_len, w.Hq, w.D, dtype=torch.float32, device="cuda")
    ws = K.new_workspace_mq(w.B, q_len, w.Hq, w.Hkv, w.D, w.max_seq_len)
    K.kvq_paged_decode_attn_mq_append(k_new.cuda(), v_new.cuda(), skip.cuda(), q, kc, vc, 1, w.block_tables.cuda(),
                                      torch.tensor(w.seq_lens, dtype=torch.int32, device="cuda"), w.max_seq_len,
                                      w.Hkv, ks, vs, float(np.float32(1 / 8)), out, ws)
    torch.cuda.synchronize()
    # exactly the slots of sequence 0's new tokens 0, 2, 3 changed
    written = {int(slots[0, i]) for i in (0, 2, 3)}
    kb, vb = bits_u8(kc), bits_u8(vc)
    changed = set()
    for blk, g, off, _ in zip(*np.nonzero(kb != before_k)):
        changed.add(int(blk) * 16 + int(off))
    for blk, g, d, off in zip(*np.nonzero(vb != before_v)):
        changed.add(int(blk) * 16 + int(off))
    assert changed <= written and len(changed) > 0


def test_mq_append_rejects_bad_arguments(K):
    w = workloads.make("tiny", seed=158, seq_lens=[40])
    L = K.lib()
    fake = torch.zeros(4096, dtype=torch.uint8, device="cuda")
    P = fake.data_ptr()
    base = (P, P, w.Hkv * w.D, P, P, 4, 0, P, P)
    # every call below is rejected before anything is launched
    tail = (P, 4, P, 64, 1, w.Hq, w.Hkv, w.D, 16, 4, 0.5, 0.5, 0.125, P, 1, P, fake.numel(), None, 0)
    assert L.kvq_paged_decode_attn_mq_append(*base, 2, *tail) == K.KVQ_EINVAL          # NVFP4 not supported
    assert L.kvq_paged_decode_attn_mq_append(P, P, w.Hkv * w.D - 8, P, P, 4, 0, P, P, 1, *tail) == K.KVQ_EINVAL
    assert L.kvq_paged_decode_attn_mq_append(P, P, w.Hkv * w.D, P, P, 17, 0, P, P, 1, *tail) == K.KVQ_EINVAL
    assert L.kvq_paged_decode_attn_mq_append(P + 2, P, w.Hkv * w.D, P, P, 4, 0, P, P, 1, *tail) == K.KVQ_EINVAL
