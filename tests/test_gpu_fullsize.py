"""Full-size parity: every workload at its real shape, in the launch
configuration the benchmark times (automatic split plan, MFMA family; for
gptoss65k also the one-call step kvq_paged_decode_attn_append that the
benchmark times, where the decode kernel writes the newest tokens), checked
on sampled (sequence, KV head) units that the oracle can afford:

- the sampled head's paged K and V bytes (gathered through the block table)
  equal the oracle's cache write of the same rows, bit for bit;
- attention of all G query heads of that KV head matches the oracle's fp64
  attention within max abs 2e-3 / relative L2 1e-3 (fp32 epilogue), and the
  bf16 output equals the fp32 output rounded to nearest even.

The oracle lays the sampled sequence out contiguously (its result does not
depend on physical block placement, which the CPU suite pins).
"""
import math

import numpy as np
import pytest
import torch

import oracle
from quantized_decode_attention_calibrate_amd import workloads

from gpu_common import assert_attention_close, gpu_or_skip, kvq, say

pytestmark = pytest.mark.gpu

# workload -> sampled (sequence, KV head) units; None = the longest and shortest sequences
SAMPLES = {
    "gptoss65k": [(0, 5)],
    "agents126k": [(1, 2), (3, 0)],
    "mixed64": None,
    "nvfp4_131k": [(1, 7)],
}


@pytest.fixture(scope="module")
def K():
    gpu_or_skip()
    return kvq()


def run_gpu(K, w, kv_dtype, fused=False):
    dev = "cuda"
    q, k, v = w.q, w.k, w.v
    if kv_dtype == K.KVQ_KV_FP8_E4M3:
        amax = torch.zeros(2, dtype=torch.float32, device=dev)
        K.kvq_amax_bf16(w.calib_k if w.calib_k is not None else k, amax[0:1])
        K.kvq_amax_bf16(w.calib_v if w.calib_v is not None else v, amax[1:2])
        ks, vs = K.kvq_calibrate(amax.cpu().tolist())
    else:
        ks, vs = 1.0, 1.0
    kc, vc = K.new_caches(kv_dtype, w.num_blocks, w.Hkv, w.D, device=dev)
    K.kvq_cache_write(k, v, w.prefill_slots(), kc, vc, kv_dtype, ks, vs)
    all_rows = w.last_token_rows().to(dev)
    rows = all_rows[all_rows >= 0]
    if not fused:
        K.kvq_cache_write(k[rows], v[rows], w.slot_mapping[rows].contiguous(), kc, vc, kv_dtype, ks, vs)
    sl = torch.tensor(w.seq_lens, dtype=torch.int32, device=dev)
    ws = K.new_workspace(w.B, w.Hq, w.Hkv, w.D, w.max_seq_len)
    sm = float(np.float32(1.0 / math.sqrt(w.D)))
    outs = {}
    for dt in (torch.float32, torch.bfloat16):
        out = torch.empty(w.B, w.Hq, w.D, dtype=dt, device=dev)
        if fused:   # the decode step as one call: the newest tokens are written by the decode kernel
            safe = all_rows.clamp(min=0)
            slots = torch.where(all_rows >= 0, w.slot_mapping[safe], torch.full_like(all_rows, -1)).contiguous()
            K.kvq_paged_decode_attn_append(k[safe].contiguous(), v[safe].contiguous(), slots, q, kc, vc, kv_dtype,
                                           w.block_tables, sl, w.max_seq_len, w.Hkv, ks, vs, sm, out, ws)
        else:
            K.kvq_paged_decode_attn(q, kc, vc, kv_dtype, w.block_tables, sl, w.max_seq_len, w.Hkv, ks, vs, sm, out,
                                    ws)
        outs[dt] = out
    torch.cuda.synchronize()
    return kc, vc, ks, vs, sm, outs


FULL_CASES = [(name, kv, False) for name in SAMPLES for kv in (1, 0)] + [
    # the benchmark's step: one kvq_paged_decode_attn_append call
    ("gptoss65k", 1, True), ("gptoss65k", 0, True), ("mixed64", 1, True)]


@pytest.mark.parametrize("name,kv,fused", FULL_CASES)
def test_fullsize_sampled_units(K, name, kv, fused):
    w = workloads.make(name, device="cuda", seed=0)
    say(f"full size {name}: B={w.B} L_max={w.max_seq_len} sum L={sum(w.seq_lens)} Hq={w.Hq} Hkv={w.Hkv} "
        f"D={w.D} kv={kv} fused={fused} split={K.kvq_decode_plan_split_tokens(w.B, w.Hkv, w.max_seq_len)}")
    kc, vc, ks, vs, sm, outs = run_gpu(K, w, kv, fused)
    units = SAMPLES[name]
    if units is None:
        order = np.argsort(w.seq_lens)
        units = [(int(order[-1]), 3), (int(order[0]), 6)]
    kvd = oracle.KV_FP8 if kv == 1 else oracle.KV_BF16
    G = w.G
    for b, g in units:
        L = w.seq_lens[b]
        s0 = w.seq_starts[b]
        nblk = (L + 15) // 16
        say(f"  unit b={b} g={g} L={L}")
        k_rows = w.k[s0:s0 + L, g:g + 1, :].cpu()
        v_rows = w.v[s0:s0 + L, g:g + 1, :].cpu()
        okc, ovc = oracle.new_caches(kvd, nblk, 1, w.D, 16)
        oracle.cache_write(k_rows, v_rows, np.arange(L), okc, ovc, kvd, ks, vs)
        # the GPU's paged bytes of this head, gathered in logical order
        phys = w.block_tables[b, :nblk].long()
        gk = kc[phys, g].cpu().contiguous().view(torch.uint8).numpy()
        gv = vc[phys, g].cpu().contiguous().view(torch.uint8).numpy()
        full = L // 16   # compare whole blocks, then the written part of the last one
        ok = okc.view(np.uint8).reshape(nblk, 16, -1)
        ov = ovc.view(np.uint8).reshape(nblk, -1, 16 * (2 if kv == 0 else 1))
        gk = gk.reshape(nblk, 16, -1)
        gv = gv.reshape(nblk, w.D, -1)
        assert np.array_equal(gk[:full], ok[:full]) and np.array_equal(gv[:full], ov[:full])
        tail = L - 16 * full
        if tail:
            eb = 2 if kv == 0 else 1
            assert np.array_equal(gk[full, :tail], ok[full, :tail])
            assert np.array_equal(gv[full, :, :tail * eb], ov[full, :, :tail * eb])
        qh = w.q[b:b + 1, g * G:(g + 1) * G, :].cpu()
        ref = oracle.decode_attn(qh, okc, ovc, kvd, np.arange(nblk, dtype=np.int32)[None, :], [L], 1, 16,
                                 ks, vs, sm, nthreads=min(G, 8))
        got = outs[torch.float32][b, g * G:(g + 1) * G].cpu().numpy()[None]
        assert_attention_close(got, ref, f"{name} kv={kv} fused={fused} b={b} g={g}")
        o16 = outs[torch.bfloat16][b, g * G:(g + 1) * G].cpu()
        assert torch.equal(o16.view(torch.int16),
                           outs[torch.float32][b, g * G:(g + 1) * G].cpu().to(torch.bfloat16).view(torch.int16))
