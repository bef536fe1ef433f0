"""Full-size parity: every workload at its real shape, in the launch
configuration the benchmark times (automatic split plan, MFMA family; for
gptoss65k also the one-call step kvq_paged_decode_attn_append that the
benchmark times, where the decode kernel writes the newest tokens), checked
on every (sequence, KV head) unit -- for mixed64 every KV head of its
longest and its shortest sequence:

- amax and the calibrated scales: the GPU's kvq_amax_bf16 + kvq_calibrate
  (kvq_nvfp4_calibrate) over the full tensors (agents126k: its separate
  calibration sample) equal the oracle's amax_bf16 + calibrate exactly;
- each unit's paged K and V bytes (gathered through the block table) equal
  the oracle's cache write of the same rows with the oracle's scales, bit
  for bit;
- attention of all G query heads of every unit matches the oracle's fp64
  attention within max abs 2e-3 / relative L2 1e-3 per unit (fp32
  epilogue), and the bf16 output equals the fp32 output rounded to nearest
  even.

The oracle lays the units out contiguously, one after another, in one cache
(its result does not depend on physical block placement, which the CPU suite
pins), and spreads its cache write and attention over the host's cores.
"""
import math
import os

import numpy as np
import pytest
import torch

import oracle
from quantized_decode_attention_calibrate_amd import workloads

from gpu_common import assert_attention_close, gpu_or_skip, kvq, say

pytestmark = pytest.mark.gpu

NVFP4 = 2
NTHREADS = max(1, min(16, len(os.sched_getaffinity(0))))


@pytest.fixture(scope="module")
def K():
    gpu_or_skip()
    return kvq()


def units_of(name, w):
    """(sequence, KV head) units checked: all, or for mixed64 every head of
    the longest and the shortest sequence."""
    if name == "mixed64":
        order = np.argsort(w.seq_lens, kind="stable")
        seqs = [int(order[-1]), int(order[0])]
    else:
        seqs = list(range(w.B))
    return [(b, g) for b in seqs for g in range(w.Hkv)]


def scales(K, w, kv):
    """The GPU's (amax, scales) and the oracle's, from the full calibration
    tensors; FP8 and NVFP4 (BF16 has none)."""
    src_k = w.calib_k if w.calib_k is not None else w.k
    src_v = w.calib_v if w.calib_v is not None else w.v
    amax = torch.zeros(2, dtype=torch.float32, device="cuda")
    K.kvq_amax_bf16(src_k, amax[0:1])
    K.kvq_amax_bf16(src_v, amax[1:2])
    g_amax = amax.cpu().tolist()
    o_amax = [oracle.amax_bf16(src_k.cpu()), oracle.amax_bf16(src_v.cpu())]
    if kv == NVFP4:
        return g_amax, list(K.kvq_nvfp4_calibrate(g_amax)), o_amax, [float(x) for x in oracle.nvfp4_calibrate(o_amax)]
    return g_amax, list(K.kvq_calibrate(g_amax)), o_amax, [float(x) for x in oracle.calibrate(o_amax)]


def run_gpu(K, w, kv, ks, vs, fused=False):
    dev = "cuda"
    q, k, v = w.q, w.k, w.v
    if kv == NVFP4:
        kc, vc = K.new_nvfp4_caches(w.num_blocks, w.Hkv, w.D, device=dev)
        write = lambda kk, vv, sl: K.kvq_nvfp4_cache_write(kk, vv, sl, kc, vc, ks, vs)
    else:
        kc, vc = K.new_caches(kv, w.num_blocks, w.Hkv, w.D, device=dev)
        write = lambda kk, vv, sl: K.kvq_cache_write(kk, vv, sl, kc, vc, kv, ks, vs)
    write(k, v, w.prefill_slots())
    all_rows = w.last_token_rows().to(dev)
    rows = all_rows[all_rows >= 0]
    if not fused:
        write(k[rows], v[rows], w.slot_mapping[rows].contiguous())
    sl = torch.tensor(w.seq_lens, dtype=torch.int32, device=dev)
    ws = K.new_workspace(w.B, w.Hq, w.Hkv, w.D, w.max_seq_len)
    sm = float(np.float32(1.0 / math.sqrt(w.D)))
    outs = {}
    for dt in (torch.float32, torch.bfloat16):
        out = torch.empty(w.B, w.Hq, w.D, dtype=dt, device=dev)
        if fused:   # the decode step as one call: the newest tokens are written by the decode kernel
            safe = all_rows.clamp(min=0)
            slots = torch.where(all_rows >= 0, w.slot_mapping[safe], torch.full_like(all_rows, -1)).contiguous()
            K.kvq_paged_decode_attn_append(k[safe].contiguous(), v[safe].contiguous(), slots, q, kc, vc, kv,
                                           w.block_tables, sl, w.max_seq_len, w.Hkv, ks, vs, sm, out, ws)
        elif kv == NVFP4:
            K.kvq_nvfp4_paged_decode_attn(q, kc, vc, w.block_tables, sl, w.max_seq_len, w.Hkv, ks, vs, sm, out, ws)
        else:
            K.kvq_paged_decode_attn(q, kc, vc, kv, w.block_tables, sl, w.max_seq_len, w.Hkv, ks, vs, sm, out,
                                    ws)
        outs[dt] = out
    torch.cuda.synchronize()
    return kc, vc, sm, outs


FULL_CASES = [(name, kv, False) for name in ("gptoss65k", "agents126k", "mixed64", "nvfp4_131k") for kv in (1, 0)] + [
    ("nvfp4_131k", NVFP4, False),
    # the benchmark's step: one kvq_paged_decode_attn_append call
    ("gptoss65k", 1, True), ("gptoss65k", 0, True), ("mixed64", 1, True)]


@pytest.mark.parametrize("name,kv,fused", FULL_CASES)
def test_fullsize_every_unit(K, name, kv, fused):
    w = workloads.make(name, device="cuda", seed=0)
    units = units_of(name, w)
    say(f"full size {name}: B={w.B} L_max={w.max_seq_len} sum L={sum(w.seq_lens)} Hq={w.Hq} Hkv={w.Hkv} "
        f"D={w.D} kv={kv} fused={fused} split={K.kvq_decode_plan_split_tokens(w.B, w.Hkv, w.max_seq_len)} "
        f"units={len(units)} oracle threads={NTHREADS}")
    if kv == 0:
        ks = vs = 1.0
    else:
        g_amax, g_sc, o_amax, o_sc = scales(K, w, kv)
        say(f"  amax gpu {g_amax} oracle {o_amax}; scales gpu {g_sc} oracle {o_sc}")
        assert g_amax == o_amax and g_sc == o_sc
        ks, vs = o_sc
    kc, vc, sm, outs = run_gpu(K, w, kv, ks, vs, fused)

    # the oracle's cache of the units, one after another: unit u's logical block
    # j is its block base[u] + j, and its tokens are written in order
    G = w.G
    lens = [w.seq_lens[b] for b, _ in units]
    nblk = [(L + 15) // 16 for L in lens]
    base = np.concatenate([[0], np.cumsum(nblk)[:-1]]).astype(np.int64)
    k_rows = torch.cat([w.k[w.seq_starts[b]:w.seq_starts[b] + L, g:g + 1].cpu() for (b, g), L in zip(units, lens)])
    v_rows = torch.cat([w.v[w.seq_starts[b]:w.seq_starts[b] + L, g:g + 1].cpu() for (b, g), L in zip(units, lens)])
    slots = np.concatenate([16 * base[u] + np.arange(L) for u, L in enumerate(lens)])
    kvd = {1: oracle.KV_FP8, 0: oracle.KV_BF16, NVFP4: oracle.KV_NVFP4}[kv]
    okc, ovc = oracle.new_caches(kvd, int(sum(nblk)), 1, w.D, 16)
    if kv == NVFP4:
        oracle.nvfp4_cache_write(k_rows, v_rows, slots, okc, ovc, 16, ks, vs, nthreads=NTHREADS)
    else:
        oracle.cache_write(k_rows, v_rows, slots, okc, ovc, kvd, ks, vs, nthreads=NTHREADS)
    del k_rows, v_rows
    bt = np.zeros((len(units), max(nblk)), dtype=np.int32)
    for u, n in enumerate(nblk):
        bt[u, :n] = base[u] + np.arange(n)
    q_units = torch.stack([w.q[b, g * G:(g + 1) * G].cpu() for b, g in units])
    ref = oracle.decode_attn(q_units, okc, ovc, kvd, bt, lens, 1, 16, ks, vs, sm, nthreads=NTHREADS)

    ok8 = okc.view(np.uint8).reshape(int(sum(nblk)), -1)
    ov8 = ovc.view(np.uint8).reshape(int(sum(nblk)), -1)
    eb = 2 if kv == 0 else 1
    for u, (b, g) in enumerate(units):
        L, n = lens[u], nblk[u]
        phys = w.block_tables[b, :n].long()
        gk = kc[phys, g].cpu().contiguous().view(torch.uint8).numpy().reshape(n, -1)
        gv = vc[phys, g].cpu().contiguous().view(torch.uint8).numpy().reshape(n, -1)
        ok, ov = ok8[base[u]:base[u] + n], ov8[base[u]:base[u] + n]
        full = L // 16   # whole blocks, then the written part of the last one
        assert np.array_equal(gk[:full], ok[:full]) and np.array_equal(gv[:full], ov[:full]), (b, g)
        tail = L - 16 * full
        if tail:
            if kv == NVFP4:   # region: codes, then scales; compare the tail tokens' codes and scales
                nk = gk[full].reshape(-1)
                okt = ok[full].reshape(-1)
                row = w.D // 2
                assert np.array_equal(nk[:tail * row], okt[:tail * row])
                sc0 = 16 * row
                assert np.array_equal(nk[sc0:sc0 + tail * (w.D // 16)], okt[sc0:sc0 + tail * (w.D // 16)])
                nv = gv[full].reshape(-1)
                ovt = ov[full].reshape(-1)
                for d in range(w.D):   # V codes [D][8]: tokens 2j (low) and 2j + 1 (high) of dim d
                    cb, ob = nv[d * 8:d * 8 + 8], ovt[d * 8:d * 8 + 8]
                    for t in range(tail):
                        assert (cb[t // 2] >> (4 * (t % 2))) & 15 == (ob[t // 2] >> (4 * (t % 2))) & 15
                sv, osv = nv[sc0:].reshape(w.D // 16, 16), ovt[sc0:].reshape(w.D // 16, 16)
                assert np.array_equal(sv[:, :tail], osv[:, :tail])
            else:
                assert np.array_equal(gk[full].reshape(16, -1)[:tail], ok[full].reshape(16, -1)[:tail])
                assert np.array_equal(gv[full].reshape(w.D, -1)[:, :tail * eb], ov[full].reshape(w.D, -1)[:, :tail * eb])
        got = outs[torch.float32][b, g * G:(g + 1) * G].cpu().numpy()[None]
        assert_attention_close(got, ref[u:u + 1], f"{name} kv={kv} fused={fused} b={b} g={g}")
        o16 = outs[torch.bfloat16][b, g * G:(g + 1) * G].cpu()
        assert torch.equal(o16.view(torch.int16),
                           outs[torch.float32][b, g * G:(g + 1) * G].cpu().to(torch.bfloat16).view(torch.int16))
