"""GPU checks of the checked build (libkvq_check.so, compiled with
-DKVQ_CHECK=1): valid calls give the release library's bytes and outputs bit
for bit with no flag set, and each contract violation sets its flag and is
replaced by a safe access (block 0, a clamped length, a skipped write).

Every violation here stays inside memory the test allocated: the library is
told a smaller num_blocks than the caches hold, the block tables have spare
columns, the workspaces are oversized, and the block-copy cache pointer
starts one block into its buffer.  So even a check that failed to fire could
not touch memory outside the test's buffers; it would only leave its flag
unset and fail the test."""
import ctypes

import numpy as np
import pytest
import torch

from quantized_decode_attention_calibrate_amd import workloads

from gpu_common import Setup, bits_u8, gpu_or_skip, kvq, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def K():
    gpu_or_skip()
    return kvq()


@pytest.fixture(scope="module")
def C(K):
    return K.open_library(K.CHECK_LIB_PATH)


def P(t):
    return t.data_ptr()


def flags(K, C):
    torch.cuda.synchronize()
    return K.kvq_check_flags(clear=True, L=C)


def attend(L, s, out, ws, seq_lens=None, num_blocks=None, bt=None, max_blocks=None):
    """kvq_paged_decode_attn_ex through library handle L (raw pointers)."""
    w = s.w
    bt = s.bt if bt is None else bt
    st = L.kvq_paged_decode_attn_ex(P(s.q), P(s.kc), P(s.vc), s.kv_dtype, P(bt),
                                    bt.shape[1] if max_blocks is None else max_blocks,
                                    P(s.sl if seq_lens is None else seq_lens), w.max_seq_len, w.B, w.Hq, w.Hkv,
                                    w.D, 16, s.kc.shape[0] if num_blocks is None else num_blocks, s.ks, s.vs,
                                    s.sm_scale, P(out), 1, P(ws), ws.numel(), None, 0, 0)
    torch.cuda.synchronize()
    return st


def write(L, s, kc, vc, slots, num_blocks, k=None, v=None):
    w = s.w
    k = s.k if k is None else k
    v = s.v if v is None else v
    st = L.kvq_cache_write(P(k), P(v), w.Hkv * w.D, P(slots), slots.numel(), w.Hkv, w.D, P(kc), P(vc),
                           num_blocks, 16, s.kv_dtype, s.ks, s.vs, None)
    torch.cuda.synchronize()
    return st


def setup(kv, seed=121, lens=(700, 2100, 65)):
    w = workloads.make("gptoss65k", seed=seed, seq_lens=list(lens), shape=dict(Hq=16, Hkv=2))
    return Setup(w, kv)


@pytest.mark.parametrize("kv", [1, 0], ids=["fp8", "bf16"])
def test_valid_calls_match_the_release_build(K, C, kv):
    s = setup(kv)
    w = s.w
    flags(K, C)                         # start from a clear word
    # cache write: the same bytes
    kc, vc = K.new_caches(kv, w.num_blocks, w.Hkv, w.D)
    kc.view(torch.uint8).fill_(0xFF)
    vc.view(torch.uint8).fill_(0xFF)
    slots = w.slot_mapping.cuda()
    assert write(C, s, kc, vc, slots, w.num_blocks) == 0
    assert flags(K, C) == 0
    assert np.array_equal(bits_u8(kc), bits_u8(s.kc)) and np.array_equal(bits_u8(vc), bits_u8(s.vc))
    # decode: the same outputs, single split and several
    for split in (0, 64):
        ws = K.new_workspace(w.B, w.Hq, w.Hkv, w.D, w.max_seq_len, split)
        ref = s.attend(torch.float32, split_tokens=split)
        out = torch.empty_like(ref)
        st = C.kvq_paged_decode_attn_ex(P(s.q), P(s.kc), P(s.vc), kv, P(s.bt), s.bt.shape[1], P(s.sl),
                                        w.max_seq_len, w.B, w.Hq, w.Hkv, w.D, 16, w.num_blocks, s.ks, s.vs,
                                        s.sm_scale, P(out), 1, P(ws), ws.numel(), None, 0, split)
        torch.cuda.synchronize()
        assert st == 0
        assert flags(K, C) == 0
        assert torch.equal(out.view(torch.int32), ref.view(torch.int32)), split


def test_block_id_past_num_blocks_reads_block_zero(K, C):
    s = setup(1, seed=122)
    w = s.w
    # the library is told half the blocks the caches hold: table entries in
    # the upper half are inside the allocation but past the declared count
    declared = w.num_blocks // 2
    assert int(s.bt.max()) >= declared
    # the same call on the release library with those entries set to block 0
    bt0 = torch.where(s.bt >= declared, torch.zeros_like(s.bt), s.bt)
    ws = torch.zeros(2 * K.kvq_decode_workspace_bytes(w.B, w.Hq, w.Hkv, w.D, w.max_seq_len), dtype=torch.uint8,
                     device="cuda")
    flags(K, C)
    out = torch.empty(w.B, w.Hq, w.D, dtype=torch.float32, device="cuda")
    say("checked build: block ids past num_blocks")
    assert attend(C, s, out, ws, num_blocks=declared) == 0
    got = flags(K, C)
    assert got & K.KVQ_CHECK_BLOCK_ID, got
    ref = torch.empty_like(out)
    assert attend(K.lib(), s, ref, ws, bt=bt0) == 0
    assert torch.equal(out.view(torch.int32), ref.view(torch.int32))


def test_seq_len_past_max_is_clamped(K, C):
    s = setup(1, seed=123, lens=(700, 2100, 65))
    w = s.w
    # spare table columns and an oversized workspace keep an unchecked
    # over-long sequence inside the test's buffers
    # (entries past each sequence's blocks are 0, a valid block: the clamped
    # length and the reference read them)
    extra = 64
    bt = torch.zeros(w.B, s.bt.shape[1] + extra, dtype=torch.int32, device="cuda")
    bt[:, :s.bt.shape[1]] = s.bt
    ws = torch.zeros(4 * K.kvq_decode_workspace_bytes(w.B, w.Hq, w.Hkv, w.D, w.max_seq_len), dtype=torch.uint8,
                     device="cuda")
    long = s.sl.clone()
    long[0] = w.max_seq_len + 40           # past max_seq_len: clamped to max_seq_len
    short = s.sl.clone()
    short[0] = w.max_seq_len
    flags(K, C)
    out = torch.empty(w.B, w.Hq, w.D, dtype=torch.float32, device="cuda")
    say("checked build: seq_len past max_seq_len")
    assert attend(C, s, out, ws, seq_lens=long, bt=bt) == 0
    got = flags(K, C)
    assert got & K.KVQ_CHECK_SEQ_LEN, got
    ref = torch.empty_like(out)
    assert attend(K.lib(), s, ref, ws, seq_lens=short, bt=bt) == 0
    assert torch.equal(out.view(torch.int32), ref.view(torch.int32))
    # a negative length is clamped to 0: the sequence's rows are zero
    neg = s.sl.clone()
    neg[2] = -3
    assert attend(C, s, out, ws, seq_lens=neg, bt=bt) == 0
    assert flags(K, C) & K.KVQ_CHECK_SEQ_LEN
    assert (out[2] == 0).all()


@pytest.mark.parametrize("kv", [1, 0], ids=["fp8", "bf16"])
def test_slot_past_num_blocks_is_skipped(K, C, kv):
    s = setup(kv, seed=124, lens=(300, 40))
    w = s.w
    declared = w.num_blocks // 2
    kc, vc = K.new_caches(kv, w.num_blocks, w.Hkv, w.D)
    kc.view(torch.uint8).fill_(0xAB)
    vc.view(torch.uint8).fill_(0xAB)
    slots = torch.tensor([3, declared * 16 + 7, 17], dtype=torch.int64, device="cuda")
    k3, v3 = s.k[:3].contiguous(), s.v[:3].contiguous()
    flags(K, C)
    say("checked build: slot past num_blocks")
    assert write(C, s, kc, vc, slots, declared, k=k3, v=v3) == 0
    assert flags(K, C) & K.KVQ_CHECK_SLOT
    kb, vb = bits_u8(kc), bits_u8(vc)
    blk = declared                          # the skipped slot's block: untouched
    assert (kb[blk] == 0xAB).all() and (vb[blk] == 0xAB).all()
    # the valid slots were written as the release library writes them
    kr, vr = K.new_caches(kv, w.num_blocks, w.Hkv, w.D)
    kr.view(torch.uint8).fill_(0xAB)
    vr.view(torch.uint8).fill_(0xAB)
    keep = torch.tensor([3, -1, 17], dtype=torch.int64, device="cuda")
    K.kvq_cache_write(k3, v3, keep, kr, vr, kv, s.ks, s.vs)
    torch.cuda.synchronize()
    assert np.array_equal(kb, bits_u8(kr)) and np.array_equal(vb, bits_u8(vr))


def test_fused_append_slot_past_num_blocks_is_skipped(K, C):
    s = setup(1, seed=125, lens=(300, 40))
    w = s.w
    declared = w.num_blocks // 2
    rows = w.last_token_rows()
    k_new, v_new = s.k[rows.cuda()].contiguous(), s.v[rows.cuda()].contiguous()
    slots = torch.tensor([declared * 16 + 2, -1], dtype=torch.int64, device="cuda")
    before = bits_u8(s.kc).copy()
    ws = torch.zeros(2 * K.kvq_decode_workspace_bytes(w.B, w.Hq, w.Hkv, w.D, w.max_seq_len), dtype=torch.uint8,
                     device="cuda")
    out = torch.empty(w.B, w.Hq, w.D, dtype=torch.float32, device="cuda")
    flags(K, C)
    say("checked build: fused append slot past num_blocks")
    st = C.kvq_paged_decode_attn_append(P(k_new), P(v_new), w.Hkv * w.D, P(slots), P(s.q), P(s.kc), P(s.vc), 1,
                                        P(s.bt), s.bt.shape[1], P(s.sl), w.max_seq_len, w.B, w.Hq, w.Hkv, w.D, 16,
                                        declared, s.ks, s.vs, s.sm_scale, P(out), 1, P(ws), ws.numel(), None, 0)
    torch.cuda.synchronize()
    assert st == 0
    got = flags(K, C)
    assert got & K.KVQ_CHECK_SLOT, got
    assert np.array_equal(bits_u8(s.kc), before)


def test_mq_fused_append_slot_past_num_blocks_is_skipped(K, C):
    s = setup(1, seed=126, lens=(300, 40))
    w = s.w
    declared = w.num_blocks // 2
    ql = 4
    k_new = torch.zeros(w.B, ql, w.Hkv, w.D, dtype=torch.bfloat16, device="cuda")
    v_new = torch.zeros_like(k_new)
    slots = torch.full((w.B, ql), -1, dtype=torch.int64, device="cuda")
    slots[0, 1] = declared * 16 + 5                     # the only slot given: past the declared blocks
    q = workloads.mq_queries(w, ql, seed=1).cuda()
    before_k, before_v = bits_u8(s.kc).copy(), bits_u8(s.vc).copy()
    ws = torch.zeros(K.kvq_decode_workspace_bytes_mq(w.B, ql, w.Hq, w.Hkv, w.D, w.max_seq_len), dtype=torch.uint8,
                     device="cuda")
    out = torch.empty(w.B, ql, w.Hq, w.D, dtype=torch.float32, device="cuda")
    flags(K, C)
    say("checked build: multi-query fused append slot past num_blocks")
    st = C.kvq_paged_decode_attn_mq_append(P(k_new), P(v_new), w.Hkv * w.D, P(slots), P(q), ql, 0, P(s.kc),
                                           P(s.vc), 1, P(s.bt), s.bt.shape[1], P(s.sl), w.max_seq_len, w.B, w.Hq,
                                           w.Hkv, w.D, 16, declared, s.ks, s.vs, s.sm_scale, P(out), 1, P(ws),
                                           ws.numel(), None, 0)
    torch.cuda.synchronize()
    assert st == 0
    got = flags(K, C)
    assert got & K.KVQ_CHECK_SLOT, got
    assert np.array_equal(bits_u8(s.kc), before_k) and np.array_equal(bits_u8(s.vc), before_v)


def test_block_copy_negative_id_is_skipped(K, C):
    bb = 4096
    base = torch.arange(8 * bb, dtype=torch.int32, device="cuda").view(torch.uint8)[: 8 * bb].contiguous()
    cache = base[bb:]                       # block -1 of `cache` is base's first block: still the test's memory
    ids = torch.tensor([2, -1, 5], dtype=torch.int32, device="cuda")
    dst = torch.full((3 * bb,), 0x5A, dtype=torch.uint8, device="cuda")
    flags(K, C)
    say("checked build: negative block-copy id")
    assert C.kvq_gather_blocks(P(cache), bb, P(ids), 3, P(dst), None) == 0
    assert flags(K, C) & K.KVQ_CHECK_BLOCK_ID
    d = dst.view(3, bb)
    assert torch.equal(d[0], cache.view(-1, bb)[2]) and torch.equal(d[2], cache.view(-1, bb)[5])
    assert (d[1] == 0x5A).all()
