"""GPU parity for the fused append (kvq_paged_decode_attn_append): one launch
that writes each sequence's newest token into the cache and attends.

The caches hold the prefill only (unwritten slots poisoned with 0xFF, an FP8
and a bf16 NaN), so a newest token the kernel read before writing it would
poison its sequence's output.  Checked against the oracle: every cache byte
after the call equals the oracle's cache write of all tokens, and the
attention is within the path's tolerance of the oracle's.  Also checked
against the two-launch path on the same inputs (kvq_cache_write then
kvq_paged_decode_attn): the same cache bytes and bit-identical outputs.
Shapes cover D 64 / 128 / 256, newest tokens at every position class in a
chunk (first, last, mid-block, a whole multiple of the chunk; odd and even
slots, which matters for NVFP4's shared V code bytes), one- and many-split
plans, an empty sequence, and a sequence whose slot is -1, for FP8, BF16 and
NVFP4 caches."""
import numpy as np
import pytest
import torch

import oracle
from quantized_decode_attention_calibrate_amd import workloads

from gpu_common import Setup, assert_attention_close, bits_u8, gpu_or_skip, kvq, say
from test_gpu_nvfp4 import NvSetup

pytestmark = pytest.mark.gpu

CASES = [
    # name, seed, seq_lens, shape, split_tokens
    ("gptoss65k", 91, [1000, 4097, 70, 64, 1, 0, 4096], dict(Hq=16, Hkv=2), 0),
    ("gptoss65k", 92, [1000, 4097, 70, 64, 1, 129], dict(Hq=16, Hkv=2), 64),
    ("gptoss65k", 93, [3000, 17], dict(Hq=16, Hkv=2), 8192),
    ("mixed64", 94, [777, 1536, 65, 2], dict(Hq=16, Hkv=4, D=128), 256),
    ("agents126k", 95, [1200, 97, 128], dict(Hq=12, Hkv=2, D=256, calib_tokens=256), 0),
]


@pytest.fixture(scope="module")
def K():
    gpu_or_skip()
    return kvq()


def newest(w, dev="cuda"):
    """k / v rows [B][Hkv][D] of each sequence's newest token and its slot (-1 if empty)."""
    rows = w.last_token_rows()
    safe = rows.clamp(min=0)
    k_new = w.k[safe].contiguous().to(dev)
    v_new = w.v[safe].contiguous().to(dev)
    slots = torch.where(rows >= 0, w.slot_mapping[safe], torch.full_like(rows, -1)).to(dev)
    return k_new, v_new, slots


def append_call(K, s, k_new, v_new, slots, split, kc=None, vc=None):
    w = s.w
    out = torch.empty(w.B, w.Hq, w.D, dtype=torch.float32, device="cuda")
    ws = K.new_workspace(w.B, w.Hq, w.Hkv, w.D, w.max_seq_len, split)
    if isinstance(s, NvSetup):
        sl = torch.tensor(w.seq_lens, dtype=torch.int32, device="cuda")
        K.kvq_nvfp4_paged_decode_attn_append(k_new, v_new, slots, w.q.cuda(), s.kc, s.vc, w.block_tables.cuda(),
                                             sl, w.max_seq_len, w.Hkv, s.gk, s.gv, s.sm, out, ws, split_tokens=split)
    else:
        K.kvq_paged_decode_attn_append(k_new, v_new, slots, s.q, s.kc if kc is None else kc,
                                       s.vc if vc is None else vc, s.kv_dtype, s.bt, s.sl, w.max_seq_len, w.Hkv,
                                       s.ks, s.vs, s.sm_scale, out, ws, split_tokens=split)
    torch.cuda.synchronize()
    return out


def nvfp4_oracle(s):
    """The oracle's NVFP4 caches of every token and its attention over them."""
    w = s.w
    okc, ovc = oracle.new_caches(oracle.KV_NVFP4, w.num_blocks, w.Hkv, w.D, 16, fill=0xFF)
    oracle.nvfp4_cache_write(w.k, w.v, w.slot_mapping, okc, ovc, 16, s.gk, s.gv)
    ref = oracle.decode_attn(w.q, okc, ovc, oracle.KV_NVFP4, w.block_tables, w.seq_lens, w.Hkv, 16, s.gk, s.gv,
                             s.sm, nthreads=8)
    return okc, ovc, ref


@pytest.mark.parametrize("kv", [1, 0, 2], ids=["fp8", "bf16", "nvfp4"])
@pytest.mark.parametrize("case", range(len(CASES)))
def test_append_matches_oracle_and_two_launches(K, case, kv):
    name, seed, lens, shape, split = CASES[case]
    w = workloads.make(name, seed=seed, seq_lens=lens, shape=shape)
    say(f"append case {case} kv={kv}: lens={lens} Hq={w.Hq} Hkv={w.Hkv} D={w.D} split={split}")
    if kv == 2:
        fused = NvSetup(K, w, write_newest=False)
        two = NvSetup(K, w, scales=(fused.gk, fused.gv), write_newest=False)
        k_new, v_new, slots = newest(w)
        got = append_call(K, fused, k_new, v_new, slots, split).cpu().numpy()
        okc, ovc, ref = nvfp4_oracle(fused)
        assert np.array_equal(fused.kc.cpu().numpy(), okc) and np.array_equal(fused.vc.cpu().numpy(), ovc)
        assert_attention_close(got, ref, f"append case {case} nvfp4")
        K.kvq_nvfp4_cache_write(k_new, v_new, slots, two.kc, two.vc, two.gk, two.gv)
        out2 = two.attend(torch.float32, split_tokens=split).cpu().numpy()
        assert torch.equal(two.kc, fused.kc) and torch.equal(two.vc, fused.vc)
        assert np.array_equal(got.view(np.uint32), out2.view(np.uint32))
        return
    fused = Setup(w, kv, write_newest=False)
    two = Setup(w, kv, scales=(fused.ks, fused.vs), write_newest=False)
    k_new, v_new, slots = newest(w)
    got = append_call(K, fused, k_new, v_new, slots, split).cpu().numpy()

    # every cache byte equals the oracle's write of all tokens
    kc_ref, vc_ref = fused.oracle_caches()
    assert np.array_equal(bits_u8(fused.kc).reshape(-1), kc_ref.view(np.uint8).reshape(-1))
    assert np.array_equal(bits_u8(fused.vc).reshape(-1), vc_ref.view(np.uint8).reshape(-1))
    ref = fused.oracle_attention(kc_ref, vc_ref)
    assert_attention_close(got, ref, f"append case {case} kv={kv}")

    # the two-launch path on the same inputs
    K.kvq_cache_write(k_new, v_new, slots, two.kc, two.vc, kv, two.ks, two.vs)
    out2 = two.attend(torch.float32, impl=2, split_tokens=split).cpu().numpy()
    assert np.array_equal(bits_u8(two.kc), bits_u8(fused.kc)) and np.array_equal(bits_u8(two.vc), bits_u8(fused.vc))
    assert np.array_equal(got.view(np.uint32), out2.view(np.uint32))


def test_append_negative_slot_writes_nothing(K):
    w = workloads.make("gptoss65k", seed=96, seq_lens=[500, 33], shape=dict(Hq=16, Hkv=2))
    s = Setup(w, 1)                      # the newest tokens are already in the cache
    k_new, v_new, slots = newest(w)
    before_k, before_v = bits_u8(s.kc).copy(), bits_u8(s.vc).copy()
    # other values for the newest rows, but slot -1 for sequence 0: its bytes stay
    k_other, v_other = (k_new * 2).contiguous(), (v_new * -1).contiguous()
    slots_skip = slots.clone()
    slots_skip[0] = -1
    got = append_call(K, s, k_other, v_other, slots_skip, 0).cpu().numpy()
    after_k, after_v = bits_u8(s.kc), bits_u8(s.vc)
    changed_k = np.flatnonzero(before_k.reshape(-1) != after_k.reshape(-1))
    changed_v = np.flatnonzero(before_v.reshape(-1) != after_v.reshape(-1))
    # only sequence 1's newest slot changed (K row bytes and V column bytes of that slot)
    slot1 = int(slots[1])
    blk, off = slot1 // 16, slot1 % 16
    D, Hkv = w.D, w.Hkv
    k_rows = {((blk * Hkv + g) * 16 + off) for g in range(Hkv)}
    assert {int(i) // D for i in changed_k} <= k_rows and len(changed_k) > 0
    assert {(int(i) // 16 // D // Hkv, int(i) % 16) for i in changed_v} == {(blk, off)}
    # sequence 0 attends to its unchanged cache: same as the plain decode call
    ref0 = s.attend(torch.float32, impl=2).cpu().numpy()[0]
    assert np.array_equal(got[0].view(np.uint32), ref0.view(np.uint32))


def test_append_rejects_bad_arguments(K):
    w = workloads.make("tiny", seed=97, seq_lens=[40])
    s = Setup(w, 1, write_newest=False)
    k_new, v_new, slots = newest(w)
    out = torch.empty(w.B, w.Hq, w.D, dtype=torch.float32, device="cuda")
    ws = K.new_workspace(w.B, w.Hq, w.Hkv, w.D, w.max_seq_len)
    L = K.lib()
    P = lambda t: t.data_ptr()
    args = lambda stride, kvd, ks: (P(k_new), P(v_new), stride, P(slots), P(s.q), P(s.kc), P(s.vc), kvd, P(s.bt),
                                    s.bt.shape[1], P(s.sl), w.max_seq_len, w.B, w.Hq, w.Hkv, w.D, 16,
                                    s.kc.shape[0], ks, s.vs, s.sm_scale, P(out), 1, P(ws),
                                    ws.numel(), None, 0)
    assert L.kvq_paged_decode_attn_append(*args(w.Hkv * w.D - 8, 1, s.ks)) == K.KVQ_EINVAL   # stride too short
    assert L.kvq_paged_decode_attn_append(*args(w.Hkv * w.D + 4, 1, s.ks)) == K.KVQ_EINVAL   # stride not 8-aligned
    assert L.kvq_paged_decode_attn_append(*args(w.Hkv * w.D, 2, s.ks)) == K.KVQ_EINVAL       # NVFP4 not supported
    assert L.kvq_paged_decode_attn_append(*args(w.Hkv * w.D, 1, -1.0)) == K.KVQ_EINVAL       # bad scale
    torch.cuda.synchronize()
    # nothing was enqueued: the newest slot still holds the poison byte
    slot = int(slots[0])
    assert bits_u8(s.kc)[slot // 16, 0, slot % 16, 0] == 0xFF
