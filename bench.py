"""Benchmark: FP8 paged decode attention on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload gptoss65k]

A step is one decode step of one full-attention layer of the gpt-oss-20b-shaped
workload (64 query / 8 KV heads, head dim 64, one sequence of 65,536 tokens):
kvq_cache_write of the newest token's K/V into the FP8 paged cache, then
kvq_paged_decode_attn over all 65,536 tokens.  Steps rotate over 12 distinct
layer caches (the model's 12 full-attention layers, 768 MiB of FP8 KV), so each
step reads its cache from HBM rather than the 256 MB last-level cache.  Inputs
are synthetic (seeded N(0,1) with 0.5% x10 outliers) and resident in HBM
before timing starts.

Prints one JSON line.  `value` is achieved HBM GB/s: algorithmic bytes of a
step (KV bytes read once per KV head, block table, seq lens, q, out, the new
token's K/V in and codes out) over the step time.  Also reported: KV tokens
scanned/s, the BF16-KV step for comparison, the roofline of the dominant
kernel (decode attention) and the CPU oracle timed on a bounded sample.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
NVFP4 = 2            # cache format tag for Layers (the C ABI has separate NVFP4 calls)
NVFP4_BYTES = 0.5625  # 4.5 bits per element: E2M1 code + one E4M3 scale per 16
METRIC = "FP8 paged decode-attn achieved HBM GB/s (% of peak) + KV tokens scanned/s"
PROFILES = os.path.join(ROOT, "profiles")
KERNEL_SOURCES = ["quantized_decode_attention_calibrate_amd/csrc/kvq_attn.hip",
                  "quantized_decode_attention_calibrate_amd/csrc/kvq_device.h",
                  "quantized_decode_attention_calibrate_amd/csrc/kvq_internal.h",
                  "quantized_decode_attention_calibrate_amd/build.py"]   # (its compiler flags)


def _code_only(text: str, python: bool) -> str:
    """The text without comments and blank space, so that editing a comment
    does not mark the compiled kernel as changed."""
    import re
    if python:
        text = re.sub(r'"""(?:.|\n)*?"""', "", text)
        text = re.sub(r"#[^\n]*", "", text)
    else:
        text = re.sub(r"/\*(?:.|\n)*?\*/", "", text)
        text = re.sub(r"//[^\n]*", "", text)
    return re.sub(r"\s+", " ", text).strip()


def kernel_source_hash() -> str:
    """Hash of the kernel sources and build flags (code only; comments and
    whitespace do not count).  A stored traffic summary is used only while it
    matches."""
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(os.path.join(ROOT, p), encoding="utf-8") as f:
            h.update(_code_only(f.read(), p.endswith(".py")).encode())
    return h.hexdigest()[:16]


def step_bytes(B, Hq, Hkv, D, seq_lens, kv_elem_bytes, n_new):
    """Algorithmic HBM bytes of one step: (decode attention, cache write)."""
    tokens = sum(seq_lens)
    kv = tokens * Hkv * 2 * D * kv_elem_bytes
    table = sum((L + 15) // 16 for L in seq_lens) * 4 + B * 4
    qo = 2 * B * Hq * D * 2
    write = n_new * (Hkv * D * 2 * 2 + Hkv * D * 2 * kv_elem_bytes + 8)
    return int(kv + table + qo), int(write)


def layers_for(w, kv_elem_bytes, cap=12):
    """Enough distinct layer caches that one rotation exceeds 1 GiB (beyond the
    256 MB last-level cache), at most `cap`."""
    per_layer = int(sum(w.seq_lens) * w.Hkv * w.D * 2 * kv_elem_bytes)
    return max(2, min(cap, -(-(1 << 30) // max(per_layer, 1))))


class Layers:
    """R layer caches of one workload, written by the library.

    GPU memory freed between measurements stays in PyTorch's cache (no
    torch.cuda.empty_cache()): returning gigabytes to the driver and
    allocating the next workload's caches at once made that workload's calls
    ~4% slower until a second or so later (measured: agents126k FP8 181 ->
    188 us right after a release, 181 us again after a 2 s pause)."""

    def __init__(self, K, w, kv_dtype, R, dev):
        import torch
        self.K, self.w, self.kv_dtype, self.R = K, w, kv_dtype, R
        self.q = w.q.to(dev)
        k, v = w.k.to(dev), w.v.to(dev)
        self.bt = w.block_tables.to(dev)
        self.sl = torch.tensor(w.seq_lens, dtype=torch.int32, device=dev)
        self.nvfp4 = kv_dtype == NVFP4
        if kv_dtype != K.KVQ_KV_BF16:
            amax = torch.zeros(2, dtype=torch.float32, device=dev)
            K.kvq_amax_bf16(k, amax[0:1])
            K.kvq_amax_bf16(v, amax[1:2])
            cal = K.kvq_nvfp4_calibrate if self.nvfp4 else K.kvq_calibrate
            self.ks, self.vs = cal(amax.cpu().tolist())
        else:
            self.ks, self.vs = 1.0, 1.0
        all_rows = w.last_token_rows().to(dev)
        rows = all_rows[all_rows >= 0]
        self.new_k = k[rows].contiguous()
        self.new_v = v[rows].contiguous()
        self.new_slots = w.slot_mapping.to(dev)[rows].contiguous()
        # per sequence (slot -1 for an empty one) for the fused append call
        safe = all_rows.clamp(min=0)
        self.app_k, self.app_v = k[safe].contiguous(), v[safe].contiguous()
        self.app_slots = torch.where(all_rows >= 0, w.slot_mapping.to(dev)[safe],
                                     torch.full_like(all_rows, -1)).contiguous()
        self.caches = []
        pre = w.prefill_slots().to(dev)
        for _ in range(R):
            if self.nvfp4:
                kc, vc = K.new_nvfp4_caches(w.num_blocks, w.Hkv, w.D, device=dev)
                K.kvq_nvfp4_cache_write(k, v, pre, kc, vc, self.ks, self.vs)
            else:
                kc, vc = K.new_caches(kv_dtype, w.num_blocks, w.Hkv, w.D, device=dev)
                K.kvq_cache_write(k, v, pre, kc, vc, kv_dtype, self.ks, self.vs)
            self.caches.append((kc, vc))
        del k, v
        self.out = torch.empty(w.B, w.Hq, w.D, dtype=torch.bfloat16, device=dev)
        self.ws = K.new_workspace(w.B, w.Hq, w.Hkv, w.D, w.max_seq_len, device=dev)
        self.sm = float(1.0 / math.sqrt(w.D))
        # The timed loops call the library through PreparedCall: arguments are
        # marshalled and checked once per layer cache, so a step costs one
        # ctypes call per launch on the host and stays device-bound.
        self._prep = {}
        self.prepare_all()
        # Each cache then gets its newest token (the prefill wrote every token
        # but that one), so an attention call on its own reads only written
        # slots, and is read once with that call (untimed), so a short timed
        # run does not catch the first reads of each cache.  A step rewrites
        # the same token with the same bytes.
        for i in range(self.R):
            self.run("write", i)
            self.run("attend", i)
        torch.cuda.synchronize()
        # ... and keeps the GPU busy with that call for SETTLE_MS, so a short
        # timed run (a few warmup steps) starts at the clock a decode loop
        # runs at rather than on the way up to it
        settle(torch, lambda i: self.run("attend", i), self.R)

    def prepare_all(self, impl=0):
        """Marshals every call kind for every layer cache now, so no timed loop
        pays the Python-side argument checks of a call it has not made before
        (a loop with fewer warmup steps than layer caches otherwise prepares
        the rest inside its timed region: measured as one 4-step block of a
        20-step run at 28-31 us per step against 19-20 us for the others)."""
        for kind in ("write", "append", "attend"):
            for i in range(self.R):
                self._prepared(kind, i, impl)

    def _prepared(self, kind, i, impl=0):
        key = (kind, i % self.R, impl)
        call = self._prep.get(key)
        if call is None:
            call = {"write": self.write, "append": self.append, "attend": self.attend}[kind](i, impl, prepare=True)
            self._prep[key] = call
        return call

    def run(self, kind, i, impl=0):
        self._prepared(kind, i, impl)()

    def write(self, i, impl=0, prepare=False):
        kc, vc = self.caches[i % self.R]
        if self.nvfp4:
            return self.K.kvq_nvfp4_cache_write(self.new_k, self.new_v, self.new_slots, kc, vc, self.ks, self.vs,
                                                prepare=prepare)
        return self.K.kvq_cache_write(self.new_k, self.new_v, self.new_slots, kc, vc, self.kv_dtype, self.ks,
                                      self.vs, prepare=prepare)

    def append(self, i, impl=0, prepare=False):
        """The step as one call: the new token's cache write fused into the decode."""
        kc, vc = self.caches[i % self.R]
        w = self.w
        if self.nvfp4:
            return self.K.kvq_nvfp4_paged_decode_attn_append(self.app_k, self.app_v, self.app_slots, self.q, kc,
                                                             vc, self.bt, self.sl, w.max_seq_len, w.Hkv, self.ks,
                                                             self.vs, self.sm, self.out, self.ws, prepare=prepare)
        return self.K.kvq_paged_decode_attn_append(self.app_k, self.app_v, self.app_slots, self.q, kc, vc,
                                                   self.kv_dtype, self.bt, self.sl, w.max_seq_len, w.Hkv, self.ks,
                                                   self.vs, self.sm, self.out, self.ws, prepare=prepare)

    def attend(self, i, impl=0, prepare=False):
        kc, vc = self.caches[i % self.R]
        w = self.w
        if self.nvfp4:
            return self.K.kvq_nvfp4_paged_decode_attn(self.q, kc, vc, self.bt, self.sl, w.max_seq_len, w.Hkv,
                                                      self.ks, self.vs, self.sm, self.out, self.ws, prepare=prepare)
        return self.K.kvq_paged_decode_attn(self.q, kc, vc, self.kv_dtype, self.bt, self.sl, w.max_seq_len,
                                            w.Hkv, self.ks, self.vs, self.sm, self.out, self.ws, impl=impl,
                                            prepare=prepare)


SETTLE_MS = 50.0


def settle(torch, fn, min_calls, min_ms=SETTLE_MS):
    """Untimed calls fn(0), fn(1), ... until at least min_calls have run and
    at least min_ms of wall time has passed.  The loops that measure the
    attention call alone start from the GPU's steady clock this way: after a
    short warmup the clock is still rising, which made NVFP4 calls ~5% slower
    (40.4-41.4 us after 10 calls, 38.2-38.4 us after 200) and FP8 ~2%.
    Returns the number of calls made."""
    n = 0
    t0 = time.perf_counter()
    while n < min_calls or (time.perf_counter() - t0) * 1e3 < min_ms:
        for _ in range(10):
            fn(n)
            n += 1
        torch.cuda.synchronize()
    return n


def time_steps(torch, layers, steps, warmup, impl=0, fused=False):
    """Returns (ms per step, mean ms of the attention call alone), HIP events
    on the launch stream.  A step is the new token's cache write and the
    decode attention: one kvq_paged_decode_attn_append call (fused), or
    kvq_cache_write then kvq_paged_decode_attn."""
    layers.prepare_all(impl)

    def step(i):
        if fused:
            layers.run("append", i)
        else:
            layers.run("write", i)
            layers.run("attend", i, impl)
    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    st = torch.cuda.current_stream()
    # events at the ends of 5 equal blocks of the timed steps: the mean over all
    # of them is the result, the blocks give its spread
    nb = 5 if steps >= 5 else 1
    marks = [round(steps * j / nb) for j in range(nb + 1)]
    ev = [torch.cuda.Event(enable_timing=True) for _ in marks]
    ev[0].record(st)
    for i in range(steps):
        step(i)
        if i + 1 in marks[1:]:
            ev[marks.index(i + 1)].record(st)
    torch.cuda.synchronize()
    step_ms = ev[0].elapsed_time(ev[-1]) / steps
    layers.spread = sorted(ev[j].elapsed_time(ev[j + 1]) / (marks[j + 1] - marks[j]) for j in range(nb))
    # the attention call alone (split kernel + merge kernel), back to back over
    # the rotated layer caches: its mean launch duration on the launch stream.
    # A diagnostic for the format comparisons, measured the same way for every
    # format: its own warmup (settle) and at least 200 calls, so neither the
    # first launch after an idle GPU (several us) nor the clock's ramp is
    # charged to a short loop
    n_attn = max(steps, 200)
    settle(torch, lambda i: layers.run("attend", i, impl), max(warmup, 10))
    a0, a1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a0.record(st)
    for i in range(n_attn):
        layers.run("attend", i, impl)
    a1.record(st)
    torch.cuda.synchronize()
    attn_ms = a0.elapsed_time(a1) / n_attn
    return step_ms, attn_ms


def measure_prefill_write(torch, K, name, reps=5):
    """Cache write of a whole prefill (every token of every sequence) per
    format: bytes = bf16 K and V read + cache bytes written (+ slots)."""
    from quantized_decode_attention_calibrate_amd import workloads
    w = workloads.make(name, device="cuda", seed=0)
    slots = w.slot_mapping
    T = w.T
    rec = {"tokens": T, "Hkv": w.Hkv, "D": w.D}
    st = torch.cuda.current_stream()
    for tag, eb in (("fp8", 1.0), ("bf16", 2.0), ("nvfp4", NVFP4_BYTES)):
        if tag == "nvfp4":
            kc, vc = K.new_nvfp4_caches(w.num_blocks, w.Hkv, w.D, device="cuda")
            fn = lambda: K.kvq_nvfp4_cache_write(w.k, w.v, slots, kc, vc, 0.01, 0.01)
        else:
            kv = K.KVQ_KV_FP8_E4M3 if tag == "fp8" else K.KVQ_KV_BF16
            kc, vc = K.new_caches(kv, w.num_blocks, w.Hkv, w.D, device="cuda")
            fn = lambda kv=kv: K.kvq_cache_write(w.k, w.v, slots, kc, vc, kv, 0.01, 0.01)
        fn()
        torch.cuda.synchronize()
        a0, a1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a0.record(st)
        for _ in range(reps):
            fn()
        a1.record(st)
        torch.cuda.synchronize()
        us = a0.elapsed_time(a1) / reps * 1e3
        byts = T * w.Hkv * w.D * 2 * (2 + eb) + T * 8
        rec[tag] = {"us": round(us, 1), "gbps": round(byts / (us * 1e-6) / 1e9, 1)}
        del kc, vc
    del w
    return rec


def measure_offload(torch, K, name, reps=5):
    """Offload of one layer's whole cache (every block of every sequence, K then
    V) to pinned host memory and its restore, per format: the host tier moves
    kvq_cache_block_bytes per block, so FP8 halves and NVFP4 cuts to 0.28 x
    the BF16 bytes."""
    from quantized_decode_attention_calibrate_amd import workloads
    w = workloads.make(name, device="cpu", seed=0)
    ids = torch.cat([w.block_tables[b, :(L + 15) // 16] for b, L in enumerate(w.seq_lens)]).to(torch.int32)
    ids = ids.cuda()
    n = ids.numel()
    rec = {"blocks": n}
    st = torch.cuda.current_stream()
    for tag, fmt in (("bf16", K.KVQ_KV_BF16), ("fp8", K.KVQ_KV_FP8_E4M3), ("nvfp4", K.KVQ_FORMAT_NVFP4)):
        bb = K.kvq_cache_block_bytes(fmt, w.Hkv, w.D)
        if fmt == K.KVQ_FORMAT_NVFP4:
            kc, vc = K.new_nvfp4_caches(w.num_blocks, w.Hkv, w.D, device="cuda")
        else:
            kc, vc = K.new_caches(fmt, w.num_blocks, w.Hkv, w.D, device="cuda")
        staging = torch.empty(2 * n * bb, dtype=torch.uint8, device="cuda")
        host = torch.empty(2 * n * bb, dtype=torch.uint8, pin_memory=True)
        times = {}
        for what, fn in (("offload", lambda: K.kvq_offload_blocks(kc, vc, bb, ids, staging, host)),
                         ("restore", lambda: K.kvq_restore_blocks(host, staging, bb, ids, kc, vc))):
            fn()
            torch.cuda.synchronize()
            a0, a1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a0.record(st)
            for _ in range(reps):
                fn()
            a1.record(st)
            torch.cuda.synchronize()
            times[what] = a0.elapsed_time(a1) / reps * 1e3
        rec[tag] = {"block_bytes": bb, "host_bytes": 2 * n * bb, "offload_us": round(times["offload"], 1),
                    "restore_us": round(times["restore"], 1),
                    "offload_gbps": round(2 * n * bb / (times["offload"] * 1e-6) / 1e9, 1)}
        del kc, vc, staging, host
    return rec


def measure_multiquery(torch, K, name, q_lens, steps, warmup):
    """Multi-query decode (speculative-decoding verification) on one
    workload's FP8 caches: the q_len newest tokens attend at once.  Reports
    the call time next to the single-query call on the same rotated caches
    (the cache is read once per call either way)."""
    from quantized_decode_attention_calibrate_amd import workloads
    w = workloads.make(name, device="cuda", seed=0)
    L = Layers(K, w, K.KVQ_KV_FP8_E4M3, layers_for(w, 1), "cuda")
    st = torch.cuda.current_stream()
    attn_b1, _ = step_bytes(w.B, w.Hq, w.Hkv, w.D, w.seq_lens, 1, w.B)
    rec = {"B": w.B, "max_seq_len": w.max_seq_len, "Hq": w.Hq, "Hkv": w.Hkv, "D": w.D, "kv": "fp8_e4m3"}

    def timed(fn):
        settle(torch, fn, warmup)
        a0, a1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a0.record(st)
        for i in range(steps):
            fn(i)
        a1.record(st)
        torch.cuda.synchronize()
        return a0.elapsed_time(a1) / steps * 1e3

    def prepared(make):
        """Per layer cache, the call marshalled once (see Layers.run)."""
        calls = [make(*L.caches[r]) for r in range(L.R)]
        return lambda i: calls[i % L.R]()

    t1 = timed(lambda i: L.run("attend", i))
    rec["q_len_1_us"] = round(t1, 2)
    # sliding window (gpt-oss alternates full layers with 128-token windows):
    # the call reads only the window's blocks
    for W in (128, 4096):
        q1 = w.q[:, None].contiguous()
        out = torch.empty(w.B, 1, w.Hq, w.D, dtype=torch.bfloat16, device="cuda")
        ws = K.new_workspace_mq(w.B, 1, w.Hq, w.Hkv, w.D, w.max_seq_len, window=W)

        us = timed(prepared(lambda kc, vc, q1=q1, out=out, ws=ws, W=W: K.kvq_paged_decode_attn_mq(
            q1, kc, vc, K.KVQ_KV_FP8_E4M3, L.bt, L.sl, w.max_seq_len, w.Hkv, L.ks, L.vs, L.sm, out, ws, window=W,
            prepare=True)))
        wb, _ = step_bytes(w.B, w.Hq, w.Hkv, w.D, [min(W, n) for n in w.seq_lens], 1, w.B)
        rec[f"window_{W}"] = {"attn_us": round(us, 2), "attn_gbps": round(wb / (us * 1e-6) / 1e9, 1)}
    for ql in q_lens:
        q = workloads.mq_queries(w, ql, seed=0).cuda()
        out = torch.empty(w.B, ql, w.Hq, w.D, dtype=torch.bfloat16, device="cuda")
        ws = K.new_workspace_mq(w.B, ql, w.Hq, w.Hkv, w.D, w.max_seq_len)

        us = timed(prepared(lambda kc, vc, q=q, out=out, ws=ws: K.kvq_paged_decode_attn_mq(
            q, kc, vc, K.KVQ_KV_FP8_E4M3, L.bt, L.sl, w.max_seq_len, w.Hkv, L.ks, L.vs, L.sm, out, ws,
            prepare=True)))
        # bytes: the KV scan once plus q_len x (q in, out)
        byts = attn_b1 + (ql - 1) * 2 * w.B * w.Hq * w.D * 2
        rec[f"q_len_{ql}"] = {"attn_us": round(us, 2), "attn_gbps": round(byts / (us * 1e-6) / 1e9, 1),
                              "over_q_len_1": round(us / t1, 3),
                              "kv_tokens_verified_per_s": round(sum(w.seq_lens) * ql / (us * 1e-6), 1)}
        # the verification step with the q_len new tokens' cache write: one launch
        # (kvq_paged_decode_attn_mq_append) and the two-launch form (kvq_cache_write,
        # then kvq_paged_decode_attn_mq)
        rows = torch.tensor([s0 + n - ql + i for s0, n in zip(w.seq_starts, w.seq_lens) for i in range(ql)],
                            device="cuda")
        k_new = w.k[rows].reshape(w.B, ql, w.Hkv, w.D).contiguous()
        v_new = w.v[rows].reshape(w.B, ql, w.Hkv, w.D).contiguous()
        slots = w.slot_mapping.to("cuda")[rows].reshape(w.B, ql).contiguous()
        one = timed(prepared(lambda kc, vc, q=q, out=out, ws=ws: K.kvq_paged_decode_attn_mq_append(
            k_new, v_new, slots, q, kc, vc, K.KVQ_KV_FP8_E4M3, L.bt, L.sl, w.max_seq_len, w.Hkv, L.ks, L.vs, L.sm,
            out, ws, prepare=True)))
        k_flat, v_flat, s_flat = k_new.view(-1, w.Hkv, w.D), v_new.view(-1, w.Hkv, w.D), slots.view(-1)

        def two_launch(kc, vc, q=q, out=out, ws=ws):
            write = K.kvq_cache_write(k_flat, v_flat, s_flat, kc, vc, K.KVQ_KV_FP8_E4M3, L.ks, L.vs, prepare=True)
            attend = K.kvq_paged_decode_attn_mq(q, kc, vc, K.KVQ_KV_FP8_E4M3, L.bt, L.sl, w.max_seq_len, w.Hkv,
                                                L.ks, L.vs, L.sm, out, ws, prepare=True)
            return lambda: (write(), attend())

        two = timed(prepared(two_launch))
        rec[f"q_len_{ql}"].update({"step_one_call_us": round(one, 2), "step_two_launch_us": round(two, 2)})
    # FP8 Q and P variant: both products on FP8 MFMA, q_scale calibrated on the queries
    amax = torch.zeros(1, dtype=torch.float32, device="cuda")
    for ql in (1, 4, 8):
        q = workloads.mq_queries(w, ql, seed=0).cuda()
        amax.zero_()
        K.kvq_amax_bf16(q, amax)
        qs = K.kvq_calibrate([float(amax.item())])[0]
        out = torch.empty(w.B, ql, w.Hq, w.D, dtype=torch.bfloat16, device="cuda")
        ws = K.new_workspace_mq(w.B, ql, w.Hq, w.Hkv, w.D, w.max_seq_len)

        us = timed(prepared(lambda kc, vc, q=q, out=out, ws=ws, qs=qs: K.kvq_paged_decode_attn_fp8qp(
            q, kc, vc, L.bt, L.sl, w.max_seq_len, w.Hkv, qs, L.ks, L.vs, L.sm, out, ws, prepare=True)))
        byts = attn_b1 + (ql - 1) * 2 * w.B * w.Hq * w.D * 2
        base = t1 if ql == 1 else rec.get(f"q_len_{ql}", {}).get("attn_us")
        rec[f"fp8qp_q_len_{ql}"] = {"attn_us": round(us, 2), "attn_gbps": round(byts / (us * 1e-6) / 1e9, 1),
                                    "over_fp8_path": round(us / base, 3) if base else None}
    del L, w
    return rec


def measure_workload(torch, K, name, steps, warmup, with_nvfp4=False):
    """FP8 and BF16 attention-call time for one workload (compact record)."""
    from quantized_decode_attention_calibrate_amd import workloads
    w = workloads.make(name, device="cuda", seed=0)
    rec = {"B": w.B, "max_seq_len": w.max_seq_len, "kv_tokens": sum(w.seq_lens), "Hq": w.Hq, "Hkv": w.Hkv,
           "D": w.D, "split_tokens": K.kvq_decode_plan_split_tokens(w.B, w.Hkv, w.max_seq_len)}
    fmts = [(K.KVQ_KV_FP8_E4M3, "fp8", 1), (K.KVQ_KV_BF16, "bf16", 2)]
    if with_nvfp4:
        fmts.append((NVFP4, "nvfp4", NVFP4_BYTES))
    for kv, tag, eb in fmts:
        L = Layers(K, w, kv, layers_for(w, eb), "cuda")
        step_ms, attn_ms = time_steps(torch, L, steps, warmup)
        attn_b, write_b = step_bytes(w.B, w.Hq, w.Hkv, w.D, w.seq_lens, eb, w.B)
        rec[tag] = {"attn_us": round(attn_ms * 1e3, 2), "attn_gbps": round(attn_b / (attn_ms * 1e-3) / 1e9, 1),
                    "pct_of_hbm_peak": round(100 * attn_b / (attn_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 1),
                    "step_us": round(step_ms * 1e3, 2), "layers_rotated": L.R,
                    # the one-token-per-sequence write's share of the two-launch step
                    "write_us_step_minus_attn": round((step_ms - attn_ms) * 1e3, 2)}
        fstep, _ = time_steps(torch, L, steps, warmup, fused=True)   # the step as one call
        rec[tag]["step_one_call_us"] = round(fstep * 1e3, 2)
        del L
    rec["fp8_over_bf16_attn_time"] = round(rec["fp8"]["attn_us"] / rec["bf16"]["attn_us"], 3)
    if with_nvfp4:
        rec["nvfp4_over_fp8_attn_time"] = round(rec["nvfp4"]["attn_us"] / rec["fp8"]["attn_us"], 3)
    rec["fp8_kv_tokens_per_s"] = round(rec["kv_tokens"] / (rec["fp8"]["attn_us"] * 1e-6), 1)
    del w
    return rec


def attn_only(torch, K, name, fmt, steps, warmup, impl=0, contiguous=False):
    """Back-to-back attention calls of one workload in one KV format over
    rotated layer caches (no step loop, no other workloads): the run that
    kernel traces and counter passes profile.  contiguous: physical blocks in
    logical order instead of the workload's random permutation."""
    from quantized_decode_attention_calibrate_amd import workloads
    kv, eb = {"fp8": (K.KVQ_KV_FP8_E4M3, 1), "bf16": (K.KVQ_KV_BF16, 2), "nvfp4": (NVFP4, NVFP4_BYTES)}[fmt]
    w = workloads.make(name, device="cuda", seed=0, contiguous=contiguous)
    L = Layers(K, w, kv, layers_for(w, eb), "cuda")
    L.prepare_all(impl)
    for i in range(warmup):
        L.run("attend", i, impl)
    torch.cuda.synchronize()
    st = torch.cuda.current_stream()
    a0, a1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a0.record(st)
    for i in range(steps):
        L.run("attend", i, impl)
    a1.record(st)
    torch.cuda.synchronize()
    us = a0.elapsed_time(a1) / steps * 1e3
    attn_b, _ = step_bytes(w.B, w.Hq, w.Hkv, w.D, w.seq_lens, eb, w.B)
    return {"workload": name, "kv": fmt, "impl": {0: "auto", 1: "valu", 2: "mfma"}[impl],
            "blocks": "contiguous" if contiguous else "permuted", "steps": steps,
            "warmup": warmup, "attn_us": round(us, 2), "attn_gbps": round(attn_b / (us * 1e-6) / 1e9, 1),
            "pct_of_hbm_peak": round(100 * attn_b / (us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 1),
            "attn_bytes": attn_b, "layers_rotated": L.R,
            "split_tokens": K.kvq_decode_plan_split_tokens(w.B, w.Hkv, w.max_seq_len)}


TRACE_LIB = os.path.join(ROOT, "quantized_decode_attention_calibrate_amd", "libkvq_trace.so")


def phase_summary(raw, decode_words, merge_words):
    """Phase breakdown of one traced call from the stamps libkvq_trace.so
    stores (kvq_trace_set layout, 100 MHz clock), in microseconds:
    distributions over waves of each decode phase, the merge kernel's start
    after the last decode wave ended and its own phases, per-XCC loop times
    (the same work lands on every XCC), and the spread of loop times between
    the waves of one work-group."""
    import numpy as np
    us = 0.01

    def q(x):
        x = np.asarray(x, dtype=np.float64)
        if x.size == 0:
            return None
        return {"med": round(float(np.median(x)), 2), "p10": round(float(np.percentile(x, 10)), 2),
                "p90": round(float(np.percentile(x, 90)), 2), "max": round(float(x.max()), 2)}

    dec = raw[:decode_words].reshape(-1, 8)
    d = dec[(dec[:, 7] & np.uint64(0xFF)) == 1]
    t = d[:, :6].astype(np.int64)
    info, ids = d[:, 6], d[:, 7]
    chunks = (info & np.uint64(0xFFFFF)).astype(np.int64)
    wg = (info >> np.uint64(20)).astype(np.int64)          # (sequence, head, split) of the wave's work-group
    xcc = ((ids >> np.uint64(8)) & np.uint64(15)).astype(np.int64)
    t00 = t[:, 0].min()
    loop = (t[:, 4] - t[:, 2]) * us
    first = t[:, 3] > 0
    out = {
        "waves": int(len(t)), "chunks_per_wave": q(chunks),
        "start_skew": q((t[:, 0] - t00) * us),
        "seq_len": q((t[:, 1] - t[:, 0]) * us),
        "block_id_staging": q((t[:, 2] - t[:, 1]) * us),
        "first_chunk": q((t[first, 3] - t[first, 2]) * us),
        "chunk_loop": q(loop),
        "epilogue": q((t[:, 5] - t[:, 4]) * us),
        "decode_end": q((t[:, 5] - t00) * us),
    }
    keys, inv = np.unique(wg, return_inverse=True)
    lo = np.full(len(keys), np.inf)
    hi = np.full(len(keys), -np.inf)
    np.minimum.at(lo, inv, loop)
    np.maximum.at(hi, inv, loop)
    out["work_groups"] = int(len(keys))
    out["intra_wg_loop_spread"] = q(hi - lo)
    out["wg_slowest_wave_loop"] = q(hi)
    out["per_xcc_loop_med"] = {int(x): round(float(np.median(loop[xcc == x])), 2) for x in np.unique(xcc)}
    out["per_xcc_decode_end_max"] = {int(x): round(float((t[xcc == x, 5] - t00).max() * us), 2)
                                     for x in np.unique(xcc)}
    mer = raw[decode_words:decode_words + merge_words].reshape(-1, 4)
    m = mer[mer[:, 3] == 1][:, :3].astype(np.int64)
    if len(m):
        out["merge_rows"] = int(len(m))
        out["merge_start_after_decode_end"] = q((m[:, 0] - t[:, 5].max()) * us)
        out["merge_split_weights"] = q((m[:, 1] - m[:, 0]) * us)
        out["merge_rest"] = q((m[:, 2] - m[:, 1]) * us)
        out["call_end"] = round(float((m[:, 2].max() - t00) * us), 2)
    else:
        out["call_end"] = round(float((t[:, 5].max() - t00) * us), 2)
    return out


def phases(torch, K, name, fmt, steps, warmup, contiguous=False):
    """Back-to-back attention calls of one workload through libkvq_trace.so;
    the phase breakdown of the last call."""
    import numpy as np
    from quantized_decode_attention_calibrate_amd import workloads
    kv, eb = {"fp8": (K.KVQ_KV_FP8_E4M3, 1), "bf16": (K.KVQ_KV_BF16, 2), "nvfp4": (NVFP4, NVFP4_BYTES)}[fmt]
    w = workloads.make(name, device="cuda", seed=0, contiguous=contiguous)
    L = Layers(K, w, kv, layers_for(w, eb), "cuda")
    split = K.kvq_decode_plan_split_tokens(w.B, w.Hkv, w.max_seq_len)
    grid = -(-w.max_seq_len // split) * w.Hkv * w.B
    decode_words, merge_words = grid * 8 * 8, w.B * w.Hq * 4    # room for 8 waves per work-group
    buf = torch.zeros(decode_words + merge_words, dtype=torch.int64, device="cuda")
    st = K.lib().kvq_trace_set(buf.data_ptr(), decode_words, merge_words)
    if st != K.KVQ_OK:
        raise RuntimeError(f"kvq_trace_set: {K.kvq_strerror(st)} (is {K.LIB_PATH} the trace build?)")
    try:
        for i in range(warmup):
            L.run("attend", i)
        torch.cuda.synchronize()
        a0, a1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a0.record()
        for i in range(steps):
            L.run("attend", i)
        a1.record()
        torch.cuda.synchronize()
        raw = buf.cpu().numpy().view(np.uint64)
    finally:
        K.lib().kvq_trace_set(None, 0, 0)
    return {"workload": name, "kv": fmt, "blocks": "contiguous" if contiguous else "permuted",
            "split_tokens": split, "traced_calls": steps,
            "traced_call_us": round(a0.elapsed_time(a1) / steps * 1e3, 2),
            "phases_us": phase_summary(raw, decode_words, merge_words)}


def measure_quality(torch, K, name):
    """The comparison the FP8 calibration guide asks for: BF16 KV, FP8 with the
    default scale 1.0, and FP8 with calibrated scales.  Reports the
    reconstruction cosine of the whole K and V tensors (fp64 over
    value(E4M3(x / scale)) * scale, codes from the library's encoder and
    decoder) and the FP8 attention output's distance from the BF16-KV output
    on the same queries, with non-finite outputs counted.  Reported, not
    gated."""
    from quantized_decode_attention_calibrate_amd import workloads
    w = workloads.make(name, device="cuda", seed=0)
    amax = torch.zeros(2, dtype=torch.float32, device="cuda")   # calibrated as the workload says (sample or data)
    K.kvq_amax_bf16(w.calib_k if w.calib_k is not None else w.k, amax[0:1])
    K.kvq_amax_bf16(w.calib_v if w.calib_v is not None else w.v, amax[1:2])
    ks, vs = K.kvq_calibrate(amax.cpu().tolist())

    def recon_cos(x, scale):
        y = (x.float() / scale).reshape(-1).contiguous()
        codes = torch.empty(y.numel(), dtype=torch.uint8, device="cuda")
        K.kvq_e4m3_encode_f32(y, codes)
        r = torch.empty(y.numel(), dtype=torch.float32, device="cuda")
        K.kvq_e4m3_decode(codes, r)
        r = r.double() * scale
        x64 = x.double().reshape(-1)
        return round(float((x64 @ r) / (x64.norm() * r.norm())), 7)

    sl = torch.tensor(w.seq_lens, dtype=torch.int32, device="cuda")
    ws = K.new_workspace(w.B, w.Hq, w.Hkv, w.D, w.max_seq_len)
    sm = float(1.0 / math.sqrt(w.D))

    def attend(kv, k_s, v_s):
        kc, vc = K.new_caches(kv, w.num_blocks, w.Hkv, w.D)
        K.kvq_cache_write(w.k, w.v, w.slot_mapping, kc, vc, kv, k_s, v_s)
        out = torch.empty(w.B, w.Hq, w.D, dtype=torch.float32, device="cuda")
        K.kvq_paged_decode_attn(w.q, kc, vc, kv, w.block_tables, sl, w.max_seq_len, w.Hkv, k_s, v_s, sm, out, ws)
        torch.cuda.synchronize()
        return out.double()

    ref = attend(K.KVQ_KV_BF16, 1.0, 1.0)
    rec = {"workload": name, "k_scale": ks, "v_scale": vs}
    for tag, (k_s, v_s) in (("fp8_calibrated", (ks, vs)), ("fp8_scale_1", (1.0, 1.0))):
        out = attend(K.KVQ_KV_FP8_E4M3, k_s, v_s)
        fin = torch.isfinite(out)
        d = (out - ref)[fin]
        rec[tag] = {"k_cos": recon_cos(w.k, k_s), "v_cos": recon_cos(w.v, v_s),
                    "saturated": int(((w.k.float() / k_s).abs() > 448).sum() + ((w.v.float() / v_s).abs() > 448).sum()),
                    "attn_rel_l2_vs_bf16": round(float(d.norm() / ref[fin].norm()), 6),
                    "attn_max_abs_vs_bf16": round(float(d.abs().max()), 6),
                    "nonfinite_outputs": int((~fin).sum())}
    del w
    return rec


def env_info(torch):
    """The run's software and device: HIP version torch was built with, the
    ROCm release, the GPU, its compute units and current clocks, and a
    diagnostic streaming rate (a 1 GiB device-to-device copy, read + write
    bytes over its time)."""
    p = torch.cuda.get_device_properties(0)
    # the ROCm release from its version file (no child process: under a
    # profiler that preloads its library, a child would initialise the GPU
    # and then exec)
    try:
        with open("/opt/rocm/.info/version") as f:
            rocm = f.read().strip()
    except OSError:
        rocm = None
    src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    st = torch.cuda.current_stream()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(st)
    for _ in range(10):
        dst.copy_(src)
    b.record(st)
    torch.cuda.synchronize()
    copy_gbps = 2 * (1 << 30) * 10 / (a.elapsed_time(b) * 1e-3) / 1e9
    del src, dst
    return {"torch": torch.__version__, "torch_hip": torch.version.hip, "rocm": rocm, "device": p.name,
            "arch": getattr(p, "gcnArchName", None), "compute_units": p.multi_processor_count,
            "copy_1gib_gbps": round(copy_gbps, 1), "clocks": read_clocks()}


def read_clocks():
    """The current shader and memory clock levels from the driver's sysfs
    tables (the line marked '*'), if readable; None otherwise."""
    import glob
    out = {}
    for key, name in (("sclk", "pp_dpm_sclk"), ("mclk", "pp_dpm_mclk")):
        for path in sorted(glob.glob(f"/sys/class/drm/card*/device/{name}")):
            try:
                with open(path) as f:
                    cur = [ln.split(":", 1)[1].strip().rstrip("*").strip() for ln in f if ln.rstrip().endswith("*")]
            except OSError:
                continue
            if cur:
                out[key] = cur[0]
                break
    return out or None


def cpu_baseline(name):
    """The oracle (fp64 C, brute-force codecs) timed on this host's cores on one
    workload's decode attention in its KV format (FP8; NVFP4 for nvfp4_131k),
    on bounded samples scaled to the whole step:
    - N threads, N = the affinity core count: every sequence's units (all G
      query heads) of the first n KV heads, n just large enough for 4 units per
      thread; KV heads are independent and cost the same, so the step takes
      Hkv / n times as long;
    - one thread: the G query heads of KV head 0 of the longest sequence,
      scaled by the step's (query head x token) pairs over the sample's.
    The oracle's cache write of the sample (threaded, untimed) supplies its
    cache.  Inputs are generated on the GPU and only the sample is copied."""
    import numpy as np
    import oracle
    import torch
    from quantized_decode_attention_calibrate_amd import workloads
    w = workloads.make(name, device="cuda", seed=0)
    nv = name == "nvfp4_131k"
    kvd, eb = (oracle.KV_NVFP4, NVFP4_BYTES) if nv else (oracle.KV_FP8, 1)
    cores = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
    G = w.G
    n = min(w.Hkv, -(-4 * cores // (w.B * G)))
    k = w.k[:, :n, :].cpu().contiguous()
    v = w.v[:, :n, :].cpu().contiguous()
    q = w.q[:, :n * G, :].cpu().contiguous()
    slots, bt = w.slot_mapping.cpu(), w.block_tables.cpu()
    lens = list(w.seq_lens)
    B, Hq, Hkv, D = w.B, w.Hq, w.Hkv, w.D
    del w
    cal = oracle.nvfp4_calibrate if nv else oracle.calibrate
    ks, vs = (float(x) for x in cal([oracle.amax_bf16(k), oracle.amax_bf16(v)]))
    nb = int(bt.max()) + 1
    kc, vc = oracle.new_caches(kvd, nb, n, k.shape[2], 16)
    if nv:
        oracle.nvfp4_cache_write(k, v, slots, kc, vc, 16, ks, vs, nthreads=cores)
    else:
        oracle.cache_write(k, v, slots, kc, vc, kvd, ks, vs, nthreads=cores)
    sm = float(np.float32(1.0 / math.sqrt(k.shape[2])))
    t = time.perf_counter()
    oracle.decode_attn(q, kc, vc, kvd, bt, lens, n, 16, ks, vs, sm, nthreads=cores)
    dt_n = time.perf_counter() - t
    b1 = int(np.argmax(lens))
    t = time.perf_counter()
    oracle.decode_attn(q, kc, vc, kvd, bt, lens, n, 16, ks, vs, sm, units=[(b1, h) for h in range(G)], nthreads=1)
    dt_1 = time.perf_counter() - t
    step_n = dt_n * Hkv / n
    step_1 = dt_1 * (Hq * sum(lens)) / (G * lens[b1])
    attn_b, _ = step_bytes(B, Hq, Hkv, D, lens, eb, B)
    fmt = "NVFP4" if nv else "FP8"
    return {"value": round(attn_b / step_n / 1e9, 4), "unit": "GB/s", "cores": cores, "kind": "oracle",
            "kv_tokens_per_s": round(sum(lens) / step_n, 1),
            "sample": f"oracle {fmt} decode attention (fp64 C) of {name} on {cores} threads: KV heads 0..{n - 1} of "
                      f"all {B} sequences ({n * G * B} of {Hq * B} (sequence, query head) units), {dt_n:.2f} s wall, "
                      f"scaled by {Hkv}/{n} to the step ({step_n:.2f} s); the cache write is excluded",
            "single_thread": {"value": round(attn_b / step_1 / 1e9, 5), "unit": "GB/s",
                              "sample": f"{G} query heads of KV head 0 of sequence {b1} ({lens[b1]} tokens) on one "
                                        f"thread: {dt_1:.2f} s wall, scaled by the step's (query head, token) pairs "
                                        f"over the sample's to {step_1:.1f} s"}}


def read_traffic(kernel_hash):
    """HBM traffic per launch from the committed PMC summary, if it was taken on this kernel source."""
    path = os.path.join(PROFILES, "decode_fp8_gptoss65k_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        d = json.load(f)
    if d.get("kernel_source_hash") != kernel_hash:
        return None
    return d.get("hbm_bytes_per_launch")


PMC_REF_CODES = 32 << 20


def pmc_reference(torch, K):
    """One dispatch of known HBM traffic for scaling PMC byte counters:
    kvq_e4m3_decode of 32 MiB of codes into 64 MiB of f16 (plain coalesced
    16-byte loads and stores).  Runs once at set-up, outside every timed region."""
    codes = torch.full((PMC_REF_CODES,), 0x38, dtype=torch.uint8, device="cuda")
    out = torch.empty(PMC_REF_CODES, dtype=torch.float16, device="cuda")
    K.kvq_e4m3_decode(codes, out)
    torch.cuda.synchronize()
    del codes, out


def _pmc_per_kernel(path, counter):
    """{kernel short name: [per-dispatch values]} of one rocprofv3 --pmc CSV."""
    import csv
    out = {}
    with open(path) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] != counter or "kvq::" not in r["Kernel_Name"]:
                continue
            name = r["Kernel_Name"].split("(")[0].replace("void ", "").replace("kvq::", "").replace(" ", "")
            out.setdefault(name, []).append(float(r["Counter_Value"]))
    return out


def pmc_summary(fetch_csv, write_csv, workload="gptoss65k"):
    """HBM traffic of one decode-attention call from two rocprofv3 --pmc runs
    of this benchmark (FETCH_SIZE, then WRITE_SIZE; KiB per dispatch).  Each
    counter is scaled by what it reads for the reference dispatch of the same
    run (pmc_reference: a coalesced kernel of known read and write bytes)."""
    from quantized_decode_attention_calibrate_amd import workloads
    w = workloads.make(workload, device="cpu", seed=0)
    fetch = _pmc_per_kernel(fetch_csv, "FETCH_SIZE")
    write = _pmc_per_kernel(write_csv, "WRITE_SIZE")
    med = lambda v: sorted(v)[len(v) // 2]
    ref = next(k for k in fetch if k.startswith("e4m3_decode_kernel"))
    fscale = PMC_REF_CODES / (med(fetch[ref]) * 1024)
    wscale = 2 * PMC_REF_CODES / (med(write[ref]) * 1024)
    # the step's call: the one-token append instantiation of the decode kernel (fifth
    # template argument, the append mode, 1) and the merge; the plain call (mode 0) beside it
    def append_mode(k):
        return int(k[k.index("<") + 1:k.rindex(">")].split(",")[4])
    fused = [k for k in fetch if k.startswith("decode_mfma_kernel") and append_mode(k) == 1]
    plain = [k for k in fetch if k.startswith("decode_mfma_kernel") and append_mode(k) == 0]
    mrg = [k for k in fetch if k.startswith("merge_")]
    f_kib = {k: med(fetch[k]) for k in fused + plain + mrg}
    w_kib = {k: med(write[k]) for k in fused + plain + mrg}
    hbm = sum(f_kib[k] for k in fused + mrg) * 1024 * fscale + sum(w_kib[k] for k in fused + mrg) * 1024 * wscale
    hbm_plain = (sum(f_kib[k] for k in plain + mrg) * 1024 * fscale +
                 sum(w_kib[k] for k in plain + mrg) * 1024 * wscale)
    attn_b, write_b = step_bytes(w.B, w.Hq, w.Hkv, w.D, w.seq_lens, 1, w.B)
    return {
        "about": "HBM traffic of one kvq_paged_decode_attn_append call (the decode step: fused cache write + "
                 f"split kernel, then the merge kernel) on the {workload} FP8 workload: medians of rocprofv3 "
                 "--pmc FETCH_SIZE and WRITE_SIZE (KiB per dispatch), each scaled by the same counter on a plain "
                 "streaming kernel of known bytes in the same run (kvq_e4m3_decode: reads "
                 f"{PMC_REF_CODES} B of codes, writes {2 * PMC_REF_CODES} B of f16).  The plain "
                 "kvq_paged_decode_attn call is listed beside it.",
        "kernel_source_hash": kernel_source_hash(),
        "fetch_size_kib_per_dispatch": f_kib,
        "write_size_kib_per_dispatch": w_kib,
        "fetch_scale_factor": round(fscale, 5),
        "write_scale_factor": round(wscale, 5),
        "hbm_bytes_per_launch": int(round(hbm)),
        "algorithmic_bytes_per_launch": attn_b + write_b,
        "traffic_over_algorithmic": round(hbm / (attn_b + write_b), 4),
        "plain_call_hbm_bytes": int(round(hbm_plain)),
        "plain_call_algorithmic_bytes": attn_b,
    }


def main():
    if len(sys.argv) >= 2 and sys.argv[1] == "--pmc-summary":
        # python bench.py --pmc-summary FETCH_CSV WRITE_CSV [OUT_JSON]
        d = pmc_summary(sys.argv[2], sys.argv[3])
        text = json.dumps(d, indent=1)
        if len(sys.argv) > 4:
            with open(sys.argv[4], "w") as f:
                f.write(text + "\n")
        print(text)
        return
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=600)
    ap.add_argument("--warmup", type=int, default=60)
    ap.add_argument("--workload", default="gptoss65k")
    ap.add_argument("--layers", type=int, default=12)
    ap.add_argument("--impl", type=int, default=0, help="0 auto, 1 VALU, 2 MFMA")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-compare", action="store_true", help="skip the BF16 comparator")
    ap.add_argument("--no-other-workloads", action="store_true",
                    help="skip the per-workload table (agents126k, mixed64, nvfp4_131k)")
    ap.add_argument("--attn-only", choices=("fp8", "bf16", "nvfp4"), default=None,
                    help="time only the attention call of --workload in this KV format (for profiling runs)")
    ap.add_argument("--phases", choices=("fp8", "bf16", "nvfp4"), default=None,
                    help="phase breakdown of the attention call of --workload in this KV format, from the "
                         "timestamps of the trace build (libkvq_trace.so)")
    ap.add_argument("--contiguous-blocks", action="store_true",
                    help="with --attn-only / --phases: physical blocks in logical order instead of the "
                         "workload's random permutation (what the scattered placement costs)")
    args = ap.parse_args()
    if args.phases:   # every library call of this process goes to the trace build
        os.environ["KVQ_LIBRARY"] = TRACE_LIB
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); this path has no multi-GPU "
              "mode: the decode kernel shards by KV head or by sequence with no exchange.", file=sys.stderr)
        sys.exit(2)

    import torch
    from quantized_decode_attention_calibrate_amd import kvq as K
    from quantized_decode_attention_calibrate_amd import workloads

    dev = "cuda"
    if args.phases:
        print(json.dumps(phases(torch, K, args.workload, args.phases, args.steps, args.warmup,
                                args.contiguous_blocks)), flush=True)
        return
    if args.attn_only:
        print(json.dumps(attn_only(torch, K, args.workload, args.attn_only, args.steps, args.warmup, args.impl,
                                   args.contiguous_blocks)), flush=True)
        return
    print(f"[bench] building {args.workload} on {torch.cuda.get_device_name(0)}", file=sys.stderr, flush=True)
    w = workloads.make(args.workload, device=dev, seed=0)
    pmc_reference(torch, K)
    fp8 = Layers(K, w, K.KVQ_KV_FP8_E4M3, args.layers, dev)
    print("[bench] timing FP8", file=sys.stderr, flush=True)
    fused = args.impl != 1      # the fused append runs on the MFMA family
    step_ms, attn_ms = time_steps(torch, fp8, args.steps, args.warmup, args.impl, fused=fused)
    fused_spread = fp8.spread
    two_step_ms, _ = time_steps(torch, fp8, args.steps, args.warmup, args.impl, fused=False)
    attn_b, write_b = step_bytes(w.B, w.Hq, w.Hkv, w.D, w.seq_lens, 1, w.B)
    tokens = sum(w.seq_lens)
    gbps = (attn_b + write_b) / (step_ms * 1e-3) / 1e9
    # dominant kernel: the step's one call (fused append: decode with the write, then the merge),
    # timed back to back by the step loop itself; without fusion the attention call alone
    roof_bytes, roof_ms = (attn_b + write_b, step_ms) if fused else (attn_b, attn_ms)
    achieved = roof_bytes / (roof_ms * 1e-3) / 1e9
    khash = kernel_source_hash()
    traffic = read_traffic(khash)
    result = {
        "metric": METRIC,
        "value": round(gbps, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8_e4m3 KV, f32 accumulate",
        "data": "synthetic (seeded N(0,1), 0.5% of K/V x10)",
        "config": {"workload": f"{args.workload}: B={w.B} x L={w.max_seq_len}, Hq={w.Hq}/Hkv={w.Hkv}, D={w.D}, "
                               f"block 16, FP8 E4M3 paged KV, {args.layers} layer caches rotated; step = "
                               "cache write of the new token + decode attention"
                               + (" (one kvq_paged_decode_attn_append call)" if fused else ""),
                   "B": w.B, "seq_len": w.max_seq_len, "Hq": w.Hq, "Hkv": w.Hkv, "head_dim": w.D,
                   "kv_dtype": "fp8_e4m3", "layers_rotated": args.layers,
                   "split_tokens": K.kvq_decode_plan_split_tokens(w.B, w.Hkv, w.max_seq_len)},
        "pct_of_hbm_peak": round(100 * gbps / HBM_PEAK_GBPS, 2),
        "kv_tokens_per_s": round(tokens / (step_ms * 1e-3), 1),
        "step_bytes": attn_b + write_b,
        "two_launch_ms_per_step": round(two_step_ms, 6),
        "ms_per_step_blocks": {"blocks": len(fused_spread), "min": round(fused_spread[0], 6),
                               "median": round(fused_spread[len(fused_spread) // 2], 6),
                               "max": round(fused_spread[-1], 6)},
        "env": env_info(torch),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": traffic,
                     "kernel": ("kvq_paged_decode_attn_append (split-K decode with the fused cache write + merge)"
                                if fused else "kvq_paged_decode_attn (split-K decode + merge)")
                               + f", bytes per launch = {roof_bytes}", "launch_ms_mean": round(roof_ms, 6),
                     "attn_ms_mean": round(attn_ms, 6),
                     "kernel_source_hash": khash},
    }
    if not args.no_compare:
        print("[bench] timing BF16 comparator", file=sys.stderr, flush=True)
        fp8_caches = fp8.caches
        del fp8
        bf = Layers(K, w, K.KVQ_KV_BF16, args.layers, dev)
        b_step, b_attn = time_steps(torch, bf, args.steps, args.warmup, args.impl, fused=fused)
        b_attn_b, _ = step_bytes(w.B, w.Hq, w.Hkv, w.D, w.seq_lens, 2, w.B)
        result["bf16_kv"] = {"ms_per_step": round(b_step, 6), "attn_ms_mean": round(b_attn, 6),
                             "attn_gbps": round(b_attn_b / (b_attn * 1e-3) / 1e9, 2)}
        result["fp8_over_bf16_attn_time"] = round(attn_ms / b_attn, 4)
        del bf, fp8_caches
    del w
    if not args.no_other_workloads:
        result["workloads"] = {}
        for name in ("agents126k", "mixed64", "nvfp4_131k"):
            print(f"[bench] workload {name}", file=sys.stderr, flush=True)
            result["workloads"][name] = measure_workload(torch, K, name, 60, 10, with_nvfp4=name == "nvfp4_131k")
        print("[bench] prefill cache writes", file=sys.stderr, flush=True)
        result["prefill_write"] = {n: measure_prefill_write(torch, K, n) for n in ("nvfp4_131k", "mixed64")}
        print("[bench] host-tier offload", file=sys.stderr, flush=True)
        result["offload"] = measure_offload(torch, K, "gptoss65k")
        print("[bench] multi-query decode", file=sys.stderr, flush=True)
        result["multiquery"] = measure_multiquery(torch, K, "gptoss65k", (2, 4, 8), 200, 20)
        print("[bench] quantization quality", file=sys.stderr, flush=True)
        result["quality"] = [measure_quality(torch, K, n) for n in ("gptoss65k", "agents126k")]
    if not args.no_cpu_baseline:
        # the oracle on the host's cores, once per workload: the headline workload's
        # figure is cpu_baseline, every workload's is in cpu_baseline["per_workload"]
        result["cpu_baseline"] = None
        per = {}
        for name in (args.workload, "agents126k", "mixed64", "nvfp4_131k"):
            if name in per:
                continue
            print(f"[bench] timing the CPU oracle on a sample of {name}", file=sys.stderr, flush=True)
            per[name] = cpu_baseline(name)
            if args.no_other_workloads:
                break
        result["cpu_baseline"] = dict(per[args.workload], per_workload=per)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
