"""The decode entry point that allocates nothing (kvq_paged_decode_attn_scratch),
for callers that cannot allocate.  Called through the C ABI, it must equal
kvq_paged_decode_attn with a caller workspace (same kernels, same split plan)
bit for bit, and the oracle within the path's tolerance, on two calls in a
row, the second with a smaller input (the scratch still holds the first
call's partials), for FP8 and BF16 caches; a call that needs more than the
scratch holds is refused before any launch."""
import numpy as np
import pytest
import torch

from quantized_decode_attention_calibrate_amd import workloads

from gpu_common import Setup, assert_attention_close, gpu_or_skip, kvq, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def K():
    gpu_or_skip()
    return kvq()


def scratch_call(K, s, out):
    """kvq_paged_decode_attn_scratch straight through the C ABI."""
    w = s.w
    st = torch.cuda.current_stream().cuda_stream
    return K.lib().kvq_paged_decode_attn_scratch(
        s.q.data_ptr(), s.kc.data_ptr(), s.vc.data_ptr(), s.kv_dtype, s.bt.data_ptr(), s.bt.shape[1],
        s.sl.data_ptr(), w.max_seq_len, w.B, w.Hq, w.Hkv, w.D, 16, s.kc.shape[0], s.ks, s.vs, s.sm_scale,
        out.data_ptr(), K.KVQ_OUT_F32 if out.dtype == torch.float32 else K.KVQ_OUT_BF16, st)


@pytest.mark.parametrize("kv", [1, 0], ids=["fp8", "bf16"])
def test_scratch_entry_equals_the_workspace_entry(K, kv):
    # a larger call (two sequences over many splits), then a smaller one
    shapes = [("gptoss65k", 171, [9000, 3000], dict(Hq=16, Hkv=2)),
              ("mixed64", 172, [700], dict(Hq=8, Hkv=2, D=128))]
    for name, seed, lens, shape in shapes:
        w = workloads.make(name, seed=seed, seq_lens=lens, shape=shape)
        s = Setup(w, kv)
        need = K.kvq_decode_workspace_bytes(w.B, w.Hq, w.Hkv, w.D, w.max_seq_len)
        say(f"scratch entry: {name} lens={lens} D={w.D} kv={kv} partials {need} B "
            f"(scratch {K.KVQ_SCRATCH_MAX_BYTES} B)")
        ref_ws = s.attend(torch.float32)                       # caller workspace
        for dt in (torch.float32, torch.bfloat16):
            out = torch.full((w.B, w.Hq, w.D), float("nan"), dtype=dt, device="cuda")
            assert scratch_call(K, s, out) == K.KVQ_OK
            torch.cuda.synchronize()
            want = ref_ws if dt == torch.float32 else s.attend(torch.bfloat16)
            assert torch.equal(out.view(torch.int16) if dt == torch.bfloat16 else out,
                               want.view(torch.int16) if dt == torch.bfloat16 else want)
        kc, vc = s.oracle_caches()
        assert_attention_close(ref_ws.cpu().numpy(), s.oracle_attention(kc, vc), f"scratch {name} kv={kv}")


def test_scratch_entry_refuses_a_call_larger_than_the_scratch(K):
    # 64 sequences x 32 heads x 256 dims over 16 splits need 32 MiB + of partials:
    # refused before any launch, so small stand-in buffers are never read
    B, Hq, Hkv, D, L = 64, 32, 8, 256, 16 * 8192
    need = K.kvq_decode_workspace_bytes(B, Hq, Hkv, D, L)
    assert need > K.KVQ_SCRATCH_MAX_BYTES
    buf = torch.zeros(1 << 16, dtype=torch.uint8, device="cuda")
    p = buf.data_ptr()
    st = K.lib().kvq_paged_decode_attn_scratch(p, p, p, K.KVQ_KV_FP8_E4M3, p, L // 16, p, L, B, Hq, Hkv, D, 16,
                                               1, 0.1, 0.1, 0.0625, p, K.KVQ_OUT_F32, None)
    assert st == K.KVQ_EWORKSPACE
    torch.cuda.synchronize()
    assert int(buf.sum()) == 0
