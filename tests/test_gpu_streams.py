"""The library enqueues every device call on the caller's stream: the whole
decode step (amax, cache write, split decode and merge, the fused append)
run on a second stream gives the same bytes and outputs as on the default
stream, bit for bit.  The second stream keeps the default priority."""
import numpy as np
import pytest
import torch

from quantized_decode_attention_calibrate_amd import workloads

from gpu_common import bits_u8, gpu_or_skip, kvq

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def K():
    gpu_or_skip()
    return kvq()


def step(K, w, kv, stream):
    """Calibrate, write the prefill, then one decode step as one fused call and
    as two launches, all enqueued on `stream` (None: the current stream)."""
    dev = "cuda"
    amax = torch.zeros(2, dtype=torch.float32, device=dev)
    K.kvq_amax_bf16(w.k, amax[0:1], stream=stream)
    K.kvq_amax_bf16(w.v, amax[1:2], stream=stream)
    (stream or torch.cuda.current_stream()).synchronize()
    ks, vs = K.kvq_calibrate(amax.cpu().tolist()) if kv == K.KVQ_KV_FP8_E4M3 else (1.0, 1.0)
    kc, vc = K.new_caches(kv, w.num_blocks, w.Hkv, w.D, device=dev)
    kc.view(torch.uint8).fill_(0xFF)
    vc.view(torch.uint8).fill_(0xFF)
    torch.cuda.synchronize()
    K.kvq_cache_write(w.k, w.v, w.prefill_slots().to(dev), kc, vc, kv, ks, vs, stream=stream)
    rows = w.last_token_rows().to(dev)
    safe = rows.clamp(min=0)
    k_new, v_new = w.k[safe].contiguous(), w.v[safe].contiguous()
    slots = torch.where(rows >= 0, w.slot_mapping.to(dev)[safe], torch.full_like(rows, -1)).contiguous()
    sl = torch.tensor(w.seq_lens, dtype=torch.int32, device=dev)
    bt = w.block_tables.to(dev)
    sm = float(np.float32(1.0 / np.sqrt(w.D)))
    ws = K.new_workspace(w.B, w.Hq, w.Hkv, w.D, w.max_seq_len, 256)
    out1 = torch.empty(w.B, w.Hq, w.D, dtype=torch.float32, device=dev)
    K.kvq_paged_decode_attn_append(k_new, v_new, slots, w.q.to(dev), kc, vc, kv, bt, sl, w.max_seq_len, w.Hkv, ks,
                                   vs, sm, out1, ws, split_tokens=256, stream=stream)
    out2 = torch.empty_like(out1)
    K.kvq_paged_decode_attn(w.q.to(dev), kc, vc, kv, bt, sl, w.max_seq_len, w.Hkv, ks, vs, sm, out2, ws,
                            split_tokens=256, stream=stream)
    (stream or torch.cuda.current_stream()).synchronize()
    return bits_u8(kc).copy(), bits_u8(vc).copy(), out1.cpu().numpy(), out2.cpu().numpy()


@pytest.mark.parametrize("kv", [1, 0], ids=["fp8", "bf16"])
def test_second_stream_matches_default_stream(K, kv):
    w = workloads.make("gptoss65k", seed=98, seq_lens=[3000, 700, 0, 129], shape=dict(Hq=16, Hkv=2), device="cuda")
    ref = step(K, w, kv, None)
    side = torch.cuda.Stream()            # default priority
    with torch.cuda.stream(side):         # the binding's default is the current stream ...
        got_ctx = step(K, w, kv, None)
    got_arg = step(K, w, kv, side)        # ... or the stream passed explicitly
    for got in (got_ctx, got_arg):
        for a, b in zip(ref, got):
            assert np.array_equal(a.view(np.uint8), b.view(np.uint8))
    # the fused call and the two-launch call agree too
    assert np.array_equal(ref[2].view(np.uint32), ref[3].view(np.uint32))
