"""The Python binding rejects, before any launch, caches and tensors that do
not match what the call's kernels assume: a cache of the wrong dtype or
layout for the call's format (an FP8 uint8 cache passed as BF16 would make a
kernel run twice past the allocation), K and V caches of different block
counts or not contiguous, non-contiguous seq_lens or block tables, and
tensors that are not on one GPU.  These run on the CPU: every check fires
before a kernel could see the pointers."""
import pytest
import torch

from quantized_decode_attention_calibrate_amd import kvq as K

B, Hq, Hkv, D, NB = 2, 8, 2, 64, 10


def caches(fmt, nb=NB):
    if fmt == K.KVQ_FORMAT_NVFP4:
        r = K.kvq_nvfp4_region_bytes(D)
        return torch.zeros(nb, Hkv, r, dtype=torch.uint8), torch.zeros(nb, Hkv, r, dtype=torch.uint8)
    return K.new_caches(fmt, nb, Hkv, D, device="cpu")


def decode_args(fmt=K.KVQ_KV_FP8_E4M3, **over):
    kc, vc = caches(fmt)
    a = dict(q=torch.zeros(B, Hq, D, dtype=torch.bfloat16), k_cache=kc, v_cache=vc,
             block_tables=torch.zeros(B, 4, dtype=torch.int32), seq_lens=torch.zeros(B, dtype=torch.int32),
             out=torch.zeros(B, Hq, D, dtype=torch.float32), workspace=torch.zeros(4096, dtype=torch.uint8))
    a.update(over)
    return a


def call_decode(fmt, a):
    if fmt == K.KVQ_FORMAT_NVFP4:
        return K.kvq_nvfp4_paged_decode_attn(a["q"], a["k_cache"], a["v_cache"], a["block_tables"], a["seq_lens"],
                                             64, Hkv, 0.1, 0.1, 0.125, a["out"], a["workspace"])
    return K.kvq_paged_decode_attn(a["q"], a["k_cache"], a["v_cache"], fmt, a["block_tables"], a["seq_lens"], 64,
                                   Hkv, 0.1, 0.1, 0.125, a["out"], a["workspace"])


@pytest.mark.parametrize("fmt,other", [(K.KVQ_KV_FP8_E4M3, K.KVQ_KV_BF16), (K.KVQ_KV_BF16, K.KVQ_KV_FP8_E4M3),
                                       (K.KVQ_FORMAT_NVFP4, K.KVQ_KV_FP8_E4M3)])
def test_cache_of_another_format_is_rejected(fmt, other):
    kc, vc = caches(other)
    with pytest.raises(ValueError, match="cache is"):
        call_decode(fmt, decode_args(fmt, k_cache=kc, v_cache=vc))


def test_cache_layouts_are_checked():
    kc, vc = caches(K.KVQ_KV_FP8_E4M3)
    # V in K's token-major layout (the transposed block)
    with pytest.raises(ValueError, match="v_cache"):
        call_decode(1, decode_args(k_cache=kc, v_cache=vc.transpose(2, 3).contiguous()))
    # another head count or head dim
    kc3, vc3 = K.new_caches(1, NB, Hkv + 1, D, device="cpu")
    with pytest.raises(ValueError, match="k_cache"):
        call_decode(1, decode_args(k_cache=kc3, v_cache=vc3))
    # K and V of different block counts
    kc2, _ = caches(1, NB + 3)
    with pytest.raises(ValueError, match="numbers of blocks"):
        call_decode(1, decode_args(k_cache=kc2, v_cache=vc))
    # a non-contiguous cache (every other block)
    big_k, big_v = caches(1, 2 * NB)
    with pytest.raises(ValueError, match="contiguous"):
        call_decode(1, decode_args(k_cache=big_k[::2], v_cache=big_v[::2]))


def test_tables_and_devices_are_checked():
    with pytest.raises(ValueError, match="seq_lens"):
        call_decode(1, decode_args(seq_lens=torch.zeros(2 * B, dtype=torch.int32)[::2]))
    with pytest.raises(ValueError, match="block_tables"):
        call_decode(1, decode_args(block_tables=torch.zeros(4, B, dtype=torch.int32).t()))
    with pytest.raises(ValueError, match="seq_lens"):
        call_decode(1, decode_args(seq_lens=torch.zeros(B, dtype=torch.int64)))
    # everything well formed, but in host memory: no kernel may receive these pointers
    for fmt in (K.KVQ_KV_FP8_E4M3, K.KVQ_KV_BF16, K.KVQ_FORMAT_NVFP4):
        with pytest.raises(ValueError, match="GPU"):
            call_decode(fmt, decode_args(fmt))


def test_cache_writes_check_caches():
    k = torch.zeros(5, Hkv, D, dtype=torch.bfloat16)
    slots = torch.arange(5, dtype=torch.int64)
    kc, vc = caches(K.KVQ_KV_FP8_E4M3)
    with pytest.raises(ValueError, match="cache is"):        # FP8 bytes written as BF16
        K.kvq_cache_write(k, k, slots, kc, vc, K.KVQ_KV_BF16)
    with pytest.raises(ValueError, match="kv_dtype"):
        K.kvq_cache_write(k, k, slots, kc, vc, 7)
    with pytest.raises(ValueError, match="cache is"):        # an FP8 cache is not an NVFP4 region
        K.kvq_nvfp4_cache_write(k, k, slots, kc, vc, 0.1, 0.1)
    nk, nv = caches(K.KVQ_FORMAT_NVFP4)
    with pytest.raises(ValueError, match="GPU"):
        K.kvq_nvfp4_cache_write(k, k, slots, nk, nv, 0.1, 0.1)
    with pytest.raises(ValueError, match="GPU"):
        K.kvq_cache_write(k, k, slots, kc, vc, K.KVQ_KV_FP8_E4M3, 0.1, 0.1)


def test_multiquery_and_fp8qp_check_caches():
    q = torch.zeros(B, 2, Hq, D, dtype=torch.bfloat16)
    out = torch.zeros(B, 2, Hq, D, dtype=torch.float32)
    a = decode_args()
    bf_k, bf_v = caches(K.KVQ_KV_BF16)
    with pytest.raises(ValueError, match="cache is"):         # FP8 Q/P reads FP8 caches only
        K.kvq_paged_decode_attn_fp8qp(q, bf_k, bf_v, a["block_tables"], a["seq_lens"], 64, Hkv, 0.1, 0.1, 0.1,
                                      0.125, out, a["workspace"])
    with pytest.raises(ValueError, match="cache is"):
        K.kvq_paged_decode_attn_mq(q, a["k_cache"], a["v_cache"], K.KVQ_KV_BF16, a["block_tables"], a["seq_lens"],
                                   64, Hkv, 0.1, 0.1, 0.125, out, a["workspace"])
    with pytest.raises(ValueError, match="cache is"):
        K.kvq_nvfp4_paged_decode_attn_mq(q, a["k_cache"], a["v_cache"], a["block_tables"], a["seq_lens"], 64, Hkv,
                                         0.1, 0.1, 0.125, out, a["workspace"])
    with pytest.raises(ValueError, match="GPU"):
        K.kvq_paged_decode_attn_mq(q, a["k_cache"], a["v_cache"], K.KVQ_KV_FP8_E4M3, a["block_tables"],
                                   a["seq_lens"], 64, Hkv, 0.1, 0.1, 0.125, out, a["workspace"])


def test_block_copies_check_caches():
    kc, vc = caches(K.KVQ_KV_FP8_E4M3)
    bb = K.kvq_cache_block_bytes(K.KVQ_KV_FP8_E4M3, Hkv, D)
    ids = torch.zeros(2, dtype=torch.int32)
    dst = torch.zeros(2 * bb, dtype=torch.uint8)
    with pytest.raises(ValueError, match="whole blocks"):
        K.kvq_gather_blocks(kc, bb + 16, ids, torch.zeros(2 * (bb + 16), dtype=torch.uint8))
    with pytest.raises(ValueError, match="GPU"):
        K.kvq_gather_blocks(kc, bb, ids, dst)
