"""bench.Layers and bench.time_steps on the CPU with a stand-in for the
library (no GPU, no compute): the set-up writes every sequence's newest token
into each layer cache before any attention call reads it, and a timed loop
marshals no call inside its timed region, however few warmup steps it has."""
import pytest
import torch

import bench
from quantized_decode_attention_calibrate_amd import workloads


class FakeLib:
    """Records which cache slots each call writes and which ones each
    attention call reads (every token of every sequence)."""
    KVQ_KV_BF16 = 0
    KVQ_KV_FP8_E4M3 = 1

    def __init__(self, w):
        self.w = w
        self.written = {}          # cache id -> set of slots written
        self.unwritten_reads = []  # (cache id, missing slots) per attention call
        self.prepared = 0          # calls marshalled (prepare=True)
        self.runs = []             # (kind, cache id) per run of a prepared call
        self.needed = set(int(s) for s in w.slot_mapping.tolist() if s >= 0)

    def kvq_amax_bf16(self, x, out):
        out.fill_(1.0)

    def kvq_calibrate(self, amax):
        return [0.01 for _ in amax]

    def new_caches(self, kv, num_blocks, Hkv, D, device="cpu"):
        return torch.empty(1), torch.empty(1)

    def new_workspace(self, *args, **kw):
        return torch.empty(1)

    def _write(self, kc, slots):
        self.written.setdefault(id(kc), set()).update(int(s) for s in slots.tolist() if s >= 0)

    def _attend(self, kc):
        missing = self.needed - self.written.get(id(kc), set())
        if missing:
            self.unwritten_reads.append((id(kc), len(missing)))

    def _call(self, kind, kc, fn, prepare):
        if not prepare:
            fn()
            return None
        self.prepared += 1

        def run():
            self.runs.append((kind, id(kc)))
            fn()
            return 0
        return run

    def kvq_cache_write(self, k, v, slots, kc, vc, kv, ks, vs, prepare=False):
        return self._call("write", kc, lambda: self._write(kc, slots), prepare)

    def kvq_paged_decode_attn_append(self, k_new, v_new, slots, q, kc, vc, kv, bt, sl, max_seq_len, Hkv, ks, vs,
                                     sm, out, ws, prepare=False):
        def fn():
            self._write(kc, slots)
            self._attend(kc)
        return self._call("append", kc, fn, prepare)

    def kvq_paged_decode_attn(self, q, kc, vc, kv, bt, sl, max_seq_len, Hkv, ks, vs, sm, out, ws, impl=0,
                              prepare=False):
        return self._call("attend", kc, lambda: self._attend(kc), prepare)


class FakeEvent:
    log = []

    def __init__(self, enable_timing=False):
        pass

    def record(self, stream=None):
        FakeEvent.log.append(FakeEvent.lib.prepared)

    def elapsed_time(self, other):
        return 1.0


@pytest.fixture
def setup(monkeypatch):
    w = workloads.make("mixed64", device="cpu", seed=3, seq_lens=[40, 17, 1, 0, 33],
                       shape=dict(Hq=8, Hkv=2, D=64, calib_tokens=32))
    lib = FakeLib(w)
    FakeEvent.lib, FakeEvent.log = lib, []
    monkeypatch.setattr(torch.cuda, "synchronize", lambda *a, **k: None)
    monkeypatch.setattr(torch.cuda, "current_stream", lambda *a, **k: None)
    monkeypatch.setattr(torch.cuda, "Event", FakeEvent)
    return w, lib


def test_setup_writes_newest_token_before_any_attention_call(setup):
    w, lib = setup
    L = bench.Layers(lib, w, lib.KVQ_KV_FP8_E4M3, 5, "cpu")
    assert lib.unwritten_reads == []
    # every cache was written once and then read by the attention call at
    # set-up (the set-up then keeps reading them for a while: settle)
    for kc, _ in L.caches:
        kinds = [kind for kind, c in lib.runs if c == id(kc)]
        assert kinds[0] == "write" and kinds.count("write") == 1 and kinds[1] == "attend", kinds[:4]
        assert set(kinds[1:]) == {"attend"}
    # later attention calls on their own read written slots only
    for i in range(2 * L.R):
        L.run("attend", i)
    assert lib.unwritten_reads == []


def test_prefill_alone_leaves_the_newest_tokens_unwritten(setup):
    # the case the set-up write exists for: without it an attention call
    # would read each sequence's newest slot unwritten
    w, lib = setup
    kc = torch.empty(1)
    lib._write(kc, w.prefill_slots())
    lib._attend(kc)
    n_seqs = sum(1 for n in w.seq_lens if n > 0)
    assert lib.unwritten_reads == [(id(kc), n_seqs)]


@pytest.mark.parametrize("fused", [True, False])
def test_timed_region_marshals_nothing(setup, fused):
    w, lib = setup
    L = bench.Layers(lib, w, lib.KVQ_KV_FP8_E4M3, 6, "cpu")
    FakeEvent.log = []
    step_ms, attn_ms = bench.time_steps(torch, L, steps=10, warmup=1, fused=fused)   # warmup < layer caches
    assert FakeEvent.log, "no events recorded"
    # the events bracket the step loop (6 marks) and the attention loop (2):
    # no call was marshalled after the first of them
    assert len(set(FakeEvent.log)) == 1, FakeEvent.log
    assert lib.unwritten_reads == []
