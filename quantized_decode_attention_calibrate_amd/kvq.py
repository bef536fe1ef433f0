"""ctypes binding of libkvq.so (include/kvq.h): same names, argument
marshalling only.  Every computation runs in the library's HIP kernels; torch
supplies device memory and the current stream.  There is no fallback: if the
library is missing or fails to load, importing this module raises.
"""
from __future__ import annotations

import ctypes
import os

import torch  # must be loaded first: libkvq binds to the HIP runtime torch ships

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("KVQ_LIBRARY") or os.path.join(_PKG, "libkvq.so")
# the same library with device-side checks of the caller's data (kvq_check_flags)
CHECK_LIB_PATH = os.path.join(_PKG, "libkvq_check.so")
TRACE_LIB_PATH = os.path.join(_PKG, "libkvq_trace.so")
KVQ_CHECK_BLOCK_ID, KVQ_CHECK_SEQ_LEN, KVQ_CHECK_SLOT = 1, 2, 4

KVQ_OK, KVQ_EINVAL, KVQ_EUNSUPPORTED, KVQ_EWORKSPACE, KVQ_EHIP = 0, -1, -2, -3, -4
KVQ_KV_BF16, KVQ_KV_FP8_E4M3 = 0, 1
KVQ_OUT_BF16, KVQ_OUT_F32 = 0, 1
KVQ_IMPL_AUTO, KVQ_IMPL_VALU, KVQ_IMPL_MFMA = 0, 1, 2
KVQ_FORMAT_NVFP4 = 2   # cache-format tag of kvq_cache_block_bytes (the C ABI has separate NVFP4 calls)
BLOCK_SIZE = 16


class KvqError(RuntimeError):
    def __init__(self, fn: str, status: int):
        msg = f"{fn}: {kvq_strerror(status)} ({status})"
        if status == KVQ_EHIP:
            msg += f", hipError {_lib.kvq_last_hip_error()}"
        super().__init__(msg)
        self.status = status


def _load(path: str) -> ctypes.CDLL:
    if not os.path.exists(path):
        raise ImportError(f"{path} is not built; run `python -m quantized_decode_attention_calibrate_amd.build`")
    L = ctypes.CDLL(path)
    P, I, I64, F, SZ = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
    sig = {
        "kvq_strerror": (ctypes.c_char_p, [I]),
        "kvq_last_hip_error": (I, []),
        "kvq_abi_version": (I, []),
        "kvq_check_flags": (I, [P, I]),
        "kvq_trace_set": (I, [P, I64, I64]),
        "kvq_e4m3_encode_f32": (I, [P, P, I64, P]),
        "kvq_e4m3_decode": (I, [P, P, I, I64, P]),
        "kvq_amax_bf16": (I, [P, I64, I64, I64, P, P]),
        "kvq_calibrate": (I, [P, P, I]),
        "kvq_cache_write": (I, [P, P, I64, P, I, I, I, P, P, I, I, I, F, F, P]),
        "kvq_decode_workspace_bytes": (SZ, [I, I, I, I, I, I]),
        "kvq_decode_workspace_bytes_ex": (SZ, [I, I, I, I, I, I, I]),
        "kvq_decode_plan_split_tokens": (I, [I, I, I, I]),
        "kvq_paged_decode_attn": (I, [P, P, P, I, P, I, P, I, I, I, I, I, I, I, F, F, F, P, I, P, SZ, P]),
        "kvq_paged_decode_attn_ex": (I, [P, P, P, I, P, I, P, I, I, I, I, I, I, I, F, F, F, P, I, P, SZ, P,
                                         I, I]),
        "kvq_nvfp4_calibrate": (I, [P, P, I]),
        "kvq_paged_decode_attn_scratch": (I, [P, P, P, I, P, I, P, I, I, I, I, I, I, I, F, F, F, P, I, P]),
        "kvq_nvfp4_region_bytes": (SZ, [I, I]),
        "kvq_nvfp4_cache_bytes_per_block": (SZ, [I, I, I]),
        "kvq_nvfp4_cache_write": (I, [P, P, I64, P, I, I, I, P, P, I, I, F, F, P]),
        "kvq_nvfp4_paged_decode_attn": (I, [P, P, P, P, I, P, I, I, I, I, I, I, I, F, F, F, P, I, P, SZ, P]),
        "kvq_nvfp4_paged_decode_attn_ex": (I, [P, P, P, P, I, P, I, I, I, I, I, I, I, F, F, F, P, I, P, SZ, P,
                                               I]),
        "kvq_e2m1_decode": (I, [P, ctypes.c_uint8, P, I64, P]),
        "kvq_paged_decode_attn_fp8qp": (I, [P, I, I, P, P, P, I, P, I, I, I, I, I, I, I, F, F, F, F, P, I, P, SZ,
                                            P, I]),
        "kvq_paged_decode_attn_append": (I, [P, P, I64, P, P, P, P, I, P, I, P, I, I, I, I, I, I, I, F, F, F, P, I,
                                             P, SZ, P, I]),
        "kvq_nvfp4_paged_decode_attn_append": (I, [P, P, I64, P, P, P, P, P, I, P, I, I, I, I, I, I, I, F, F, F, P,
                                                   I, P, SZ, P, I]),
        "kvq_cache_block_bytes": (SZ, [I, I, I, I]),
        "kvq_gather_blocks": (I, [P, SZ, P, I, P, P]),
        "kvq_scatter_blocks": (I, [P, SZ, P, I, P, P]),
        "kvq_offload_blocks": (I, [P, P, SZ, P, I, P, P, P]),
        "kvq_restore_blocks": (I, [P, P, SZ, P, I, P, P, P]),
        "kvq_decode_workspace_bytes_mq": (SZ, [I, I, I, I, I, I, I, I, I]),
        "kvq_paged_decode_attn_mq": (I, [P, I, I, P, P, I, P, I, P, I, I, I, I, I, I, I, F, F, F, P, I, P, SZ, P,
                                         I]),
        "kvq_nvfp4_paged_decode_attn_mq": (I, [P, I, I, P, P, P, I, P, I, I, I, I, I, I, I, F, F, F, P, I, P, SZ,
                                               P, I]),
        "kvq_paged_decode_attn_mq_append": (I, [P, P, I64, P, P, I, I, P, P, I, P, I, P, I, I, I, I, I, I, I, F, F,
                                                F, P, I, P, SZ, P, I]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(L, name)
        fn.restype = res
        fn.argtypes = args
    return L


_lib = _load(LIB_PATH)


def lib() -> ctypes.CDLL:
    return _lib


def open_library(path: str = CHECK_LIB_PATH) -> ctypes.CDLL:
    """Another handle with the same signatures, e.g. the checked build (its
    calls take raw pointers, as lib()'s do)."""
    return _load(path)


def kvq_check_flags(clear: bool = True, L: ctypes.CDLL = None) -> int:
    """Contract-violation bits of a checked library (synchronous)."""
    flags = ctypes.c_uint(0)
    _check("kvq_check_flags", (L or _lib).kvq_check_flags(ctypes.byref(flags), 1 if clear else 0))
    return flags.value


def _stream(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _check(fn: str, status: int) -> None:
    if status != KVQ_OK:
        raise KvqError(fn, status)


class PreparedCall:
    """One library call with its arguments marshalled and checked once.
    Calling it enqueues the same work again, on the stream it was prepared
    for, without the Python-side checks: for launch-bound loops such as one
    decode step per layer cache.  It keeps its tensors alive; their contents
    may change between calls, their storage may not."""
    __slots__ = ("_name", "_fn", "_args", "_keep")

    def __init__(self, name: str, fn, args: tuple, keep: tuple):
        self._name, self._fn, self._args, self._keep = name, fn, args, keep

    def __call__(self) -> None:
        status = self._fn(*self._args)
        if status != KVQ_OK:
            raise KvqError(self._name, status)


def _run(name: str, fn, args: tuple, prepare: bool, keep: tuple):
    """Call now, or (prepare=True) return the call as a PreparedCall."""
    if prepare:
        return PreparedCall(name, fn, args, keep)
    _check(name, fn(*args))
    return None


def _ptr(t) -> int:
    return 0 if t is None else t.data_ptr()


def _require(cond: bool, msg: str) -> None:
    if not cond:
        raise ValueError(msg)


_FMT_NAME = {0: "BF16", 1: "FP8 E4M3", 2: "NVFP4"}


def _caches(k_cache: torch.Tensor, v_cache: torch.Tensor, fmt: int, Hkv: int, D: int) -> int:
    """Checks that K and V caches have the dtype and layout the call's format
    assumes (so no kernel can index past them): FP8 uint8 and BF16 bfloat16
    [num_blocks][Hkv][16][D] (K) and [num_blocks][Hkv][D][16] (V); NVFP4
    uint8 [num_blocks][Hkv][kvq_nvfp4_region_bytes(D)] both; contiguous, on
    one GPU.  Returns num_blocks."""
    name = _FMT_NAME.get(fmt, str(fmt))
    _require(fmt in _FMT_NAME, f"unknown cache format {fmt}")
    want = torch.bfloat16 if fmt == KVQ_KV_BF16 else torch.uint8
    for t, which in ((k_cache, "k_cache"), (v_cache, "v_cache")):
        _require(isinstance(t, torch.Tensor) and t.dtype == want,
                 f"{which}: a {name} cache is {want}, got {getattr(t, 'dtype', type(t))}")
    if fmt == KVQ_FORMAT_NVFP4:
        r = kvq_nvfp4_region_bytes(D)
        shape_k = shape_v = (Hkv, r)
    else:
        shape_k, shape_v = (Hkv, BLOCK_SIZE, D), (Hkv, D, BLOCK_SIZE)
    _require(k_cache.dim() == 1 + len(shape_k) and tuple(k_cache.shape[1:]) == shape_k,
             f"k_cache: a {name} cache is [num_blocks]{list(shape_k)}, got {list(k_cache.shape)}")
    _require(v_cache.dim() == 1 + len(shape_v) and tuple(v_cache.shape[1:]) == shape_v,
             f"v_cache: a {name} cache is [num_blocks]{list(shape_v)}, got {list(v_cache.shape)}")
    _require(k_cache.shape[0] == v_cache.shape[0], "k_cache and v_cache hold different numbers of blocks")
    _require(k_cache.is_contiguous() and v_cache.is_contiguous(), "caches must be contiguous")
    return int(k_cache.shape[0])


def _same_gpu(*tensors) -> None:
    """Every tensor (None skipped) on one CUDA device."""
    ts = [t for t in tensors if t is not None]
    dev = ts[0].device
    _require(dev.type == "cuda", f"tensors must be on a GPU, got {dev}")
    for t in ts[1:]:
        _require(t.device == dev, f"tensors on different devices: {dev} and {t.device}")


def _tables(block_tables: torch.Tensor, seq_lens: torch.Tensor, B: int) -> None:
    _require(block_tables.dtype == torch.int32 and block_tables.dim() == 2 and block_tables.is_contiguous()
             and block_tables.shape[0] == B, "block_tables: contiguous int32 [B][max_blocks]")
    _require(seq_lens.dtype == torch.int32 and tuple(seq_lens.shape) == (B,) and seq_lens.is_contiguous(),
             "seq_lens: contiguous int32 [B]")


def kvq_strerror(status: int) -> str:
    return _lib.kvq_strerror(status).decode()


def kvq_abi_version() -> int:
    return _lib.kvq_abi_version()


def kvq_e4m3_encode_f32(y: torch.Tensor, codes: torch.Tensor, stream=None) -> None:
    assert y.dtype == torch.float32 and codes.dtype == torch.uint8 and y.is_contiguous() and codes.is_contiguous()
    assert codes.numel() >= y.numel()
    _check("kvq_e4m3_encode_f32", _lib.kvq_e4m3_encode_f32(_ptr(y), _ptr(codes), y.numel(), _stream(stream)))


def kvq_e4m3_decode(codes: torch.Tensor, out: torch.Tensor, stream=None) -> None:
    kind = {torch.float32: 0, torch.float16: 1, torch.bfloat16: 2}[out.dtype]
    assert codes.dtype == torch.uint8 and codes.is_contiguous() and out.is_contiguous()
    assert out.numel() >= codes.numel()
    _check("kvq_e4m3_decode", _lib.kvq_e4m3_decode(_ptr(codes), _ptr(out), kind, codes.numel(), _stream(stream)))


def kvq_amax_bf16(x: torch.Tensor, amax: torch.Tensor, stream=None) -> None:
    """Running max |x| into amax (fp32 device scalar, caller-initialised).
    x: bf16, viewed as rows of its last-but-flattened layout: a 2-D or 3-D
    tensor whose last dims are contiguous and whose first dim may be strided."""
    assert x.dtype == torch.bfloat16 and amax.dtype == torch.float32
    x2 = x.reshape(x.shape[0], -1) if x.dim() > 2 else x
    assert x2.stride(1) == 1
    _check("kvq_amax_bf16", _lib.kvq_amax_bf16(_ptr(x2), x2.shape[0], x2.shape[1], x2.stride(0), _ptr(amax),
                                                _stream(stream)))


def _host_scales(fn_name: str, amax) -> list:
    vals = [float(a) for a in amax]
    n = len(vals)
    src = (ctypes.c_float * n)(*vals)
    dst = (ctypes.c_float * n)()
    _check(fn_name, getattr(_lib, fn_name)(ctypes.addressof(src), ctypes.addressof(dst), n))
    return list(dst)


def kvq_nvfp4_calibrate(amax) -> list:
    """Host-only: per-tensor NVFP4 global scales from observed maxima."""
    return _host_scales("kvq_nvfp4_calibrate", amax)


def kvq_nvfp4_region_bytes(D: int) -> int:
    return _lib.kvq_nvfp4_region_bytes(D, BLOCK_SIZE)


def kvq_nvfp4_cache_bytes_per_block(Hkv: int, D: int) -> int:
    return _lib.kvq_nvfp4_cache_bytes_per_block(Hkv, D, BLOCK_SIZE)


def new_nvfp4_caches(num_blocks: int, Hkv: int, D: int, device="cuda"):
    """Uninitialised NVFP4 K and V caches [num_blocks][Hkv][region] bytes."""
    r = kvq_nvfp4_region_bytes(D)
    return (torch.empty((num_blocks, Hkv, r), dtype=torch.uint8, device=device),
            torch.empty((num_blocks, Hkv, r), dtype=torch.uint8, device=device))


def kvq_nvfp4_cache_write(k: torch.Tensor, v: torch.Tensor, slot_mapping: torch.Tensor, k_cache: torch.Tensor,
                          v_cache: torch.Tensor, k_gscale: float, v_gscale: float, stream=None, prepare: bool = False):
    assert k.dtype == torch.bfloat16 and v.dtype == torch.bfloat16 and slot_mapping.dtype == torch.int64
    T, Hkv, D = k.shape
    assert v.shape == k.shape and k.stride(0) == v.stride(0) and k.stride(2) == 1 and k.stride(1) == D
    assert slot_mapping.shape == (T,) and slot_mapping.is_contiguous()
    num_blocks = _caches(k_cache, v_cache, KVQ_FORMAT_NVFP4, Hkv, D)
    _same_gpu(k, v, slot_mapping, k_cache, v_cache)
    return _run("kvq_nvfp4_cache_write", _lib.kvq_nvfp4_cache_write, (
        _ptr(k), _ptr(v), k.stride(0), _ptr(slot_mapping), T, Hkv, D, _ptr(k_cache), _ptr(v_cache),
        num_blocks, BLOCK_SIZE, k_gscale, v_gscale, _stream(stream)),
        prepare, (k, v, slot_mapping, k_cache, v_cache))


def kvq_nvfp4_paged_decode_attn(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                                block_tables: torch.Tensor, seq_lens: torch.Tensor, max_seq_len: int, Hkv: int,
                                k_gscale: float, v_gscale: float, sm_scale: float, out: torch.Tensor,
                                workspace: torch.Tensor, split_tokens: int = 0, stream=None, prepare: bool = False):
    B, Hq, D = q.shape
    assert q.dtype == torch.bfloat16 and q.is_contiguous() and out.is_contiguous() and out.shape == q.shape
    _tables(block_tables, seq_lens, B)
    _caches(k_cache, v_cache, KVQ_FORMAT_NVFP4, Hkv, D)
    _same_gpu(q, k_cache, v_cache, block_tables, seq_lens, out, workspace)
    out_dtype = {torch.bfloat16: KVQ_OUT_BF16, torch.float32: KVQ_OUT_F32}[out.dtype]
    return _run("kvq_nvfp4_paged_decode_attn", _lib.kvq_nvfp4_paged_decode_attn_ex, (
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables), block_tables.shape[1], _ptr(seq_lens),
        max_seq_len, B, Hq, Hkv, D, BLOCK_SIZE, k_cache.shape[0], k_gscale, v_gscale, sm_scale, _ptr(out),
        out_dtype, _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream), split_tokens),
        prepare, (q, k_cache, v_cache, block_tables, seq_lens, out, workspace))


def kvq_nvfp4_paged_decode_attn_append(k_new: torch.Tensor, v_new: torch.Tensor, slot_mapping: torch.Tensor,
                                       q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                                       block_tables: torch.Tensor, seq_lens: torch.Tensor, max_seq_len: int,
                                       Hkv: int, k_gscale: float, v_gscale: float, sm_scale: float,
                                       out: torch.Tensor, workspace: torch.Tensor, split_tokens: int = 0,
                                       stream=None, prepare: bool = False):
    """kvq_nvfp4_cache_write of each sequence's newest token followed by
    kvq_nvfp4_paged_decode_attn, in one launch (arguments as
    kvq_paged_decode_attn_append, with the global scales)."""
    B, Hq, D = q.shape
    assert q.dtype == torch.bfloat16 and q.is_contiguous() and out.is_contiguous() and out.shape == q.shape
    assert k_new.dtype == torch.bfloat16 and v_new.dtype == torch.bfloat16 and slot_mapping.dtype == torch.int64
    assert k_new.shape == (B, Hkv, D) and v_new.shape == k_new.shape and k_new.stride(0) == v_new.stride(0)
    assert k_new.stride(2) == 1 and k_new.stride(1) == D and v_new.stride(2) == 1 and v_new.stride(1) == D
    assert slot_mapping.shape == (B,) and slot_mapping.is_contiguous()
    _tables(block_tables, seq_lens, B)
    _caches(k_cache, v_cache, KVQ_FORMAT_NVFP4, Hkv, D)
    _same_gpu(k_new, v_new, slot_mapping, q, k_cache, v_cache, block_tables, seq_lens, out, workspace)
    out_dtype = {torch.bfloat16: KVQ_OUT_BF16, torch.float32: KVQ_OUT_F32}[out.dtype]
    return _run("kvq_nvfp4_paged_decode_attn_append", _lib.kvq_nvfp4_paged_decode_attn_append, (
        _ptr(k_new), _ptr(v_new), k_new.stride(0), _ptr(slot_mapping), _ptr(q), _ptr(k_cache), _ptr(v_cache),
        _ptr(block_tables), block_tables.shape[1], _ptr(seq_lens), max_seq_len, B, Hq, Hkv, D, BLOCK_SIZE,
        k_cache.shape[0], k_gscale, v_gscale, sm_scale, _ptr(out), out_dtype, _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream), split_tokens),
        prepare, (k_new, v_new, slot_mapping, q, k_cache, v_cache, block_tables, seq_lens, out, workspace))


def kvq_e2m1_decode(codes: torch.Tensor, scale_code: int, out: torch.Tensor, stream=None) -> None:
    """out (f16, 2 per byte) = E2M1 codes times the E4M3 value of scale_code."""
    assert codes.dtype == torch.uint8 and codes.is_contiguous() and out.is_contiguous()
    assert out.dtype == torch.float16 and out.numel() >= 2 * codes.numel()
    _check("kvq_e2m1_decode", _lib.kvq_e2m1_decode(_ptr(codes), scale_code, _ptr(out), codes.numel(),
                                                    _stream(stream)))


def kvq_calibrate(amax) -> list:
    """Host-only: per-layer scales from observed maxima (list of floats)."""
    return _host_scales("kvq_calibrate", amax)


def new_caches(kv_dtype: int, num_blocks: int, Hkv: int, D: int, device="cuda"):
    """Uninitialised K and V caches in the library's layouts."""
    dt = torch.uint8 if kv_dtype == KVQ_KV_FP8_E4M3 else torch.bfloat16
    k = torch.empty((num_blocks, Hkv, BLOCK_SIZE, D), dtype=dt, device=device)
    v = torch.empty((num_blocks, Hkv, D, BLOCK_SIZE), dtype=dt, device=device)
    return k, v


def kvq_cache_write(k: torch.Tensor, v: torch.Tensor, slot_mapping: torch.Tensor, k_cache: torch.Tensor,
                    v_cache: torch.Tensor, kv_dtype: int, k_scale: float = 1.0, v_scale: float = 1.0,
                    stream=None, prepare: bool = False):
    """k, v: bf16 [T][Hkv][D] (token dim may be strided); slot_mapping int64 [T]."""
    assert k.dtype == torch.bfloat16 and v.dtype == torch.bfloat16 and slot_mapping.dtype == torch.int64
    T, Hkv, D = k.shape
    assert v.shape == k.shape and k.stride(0) == v.stride(0) and k.stride(2) == 1 and k.stride(1) == D
    assert slot_mapping.shape == (T,) and slot_mapping.is_contiguous()
    _require(kv_dtype in (KVQ_KV_BF16, KVQ_KV_FP8_E4M3), f"kv_dtype {kv_dtype}: BF16 or FP8 E4M3")
    num_blocks = _caches(k_cache, v_cache, kv_dtype, Hkv, D)
    _same_gpu(k, v, slot_mapping, k_cache, v_cache)
    return _run("kvq_cache_write", _lib.kvq_cache_write, (
        _ptr(k), _ptr(v), k.stride(0), _ptr(slot_mapping), T, Hkv, D, _ptr(k_cache), _ptr(v_cache),
        num_blocks, BLOCK_SIZE, kv_dtype, k_scale, v_scale, _stream(stream)),
        prepare, (k, v, slot_mapping, k_cache, v_cache))


def kvq_decode_workspace_bytes(B: int, Hq: int, Hkv: int, D: int, max_seq_len: int, split_tokens: int = 0) -> int:
    return _lib.kvq_decode_workspace_bytes_ex(B, Hq, Hkv, D, max_seq_len, BLOCK_SIZE, split_tokens)


def kvq_decode_plan_split_tokens(B: int, Hkv: int, max_seq_len: int) -> int:
    return _lib.kvq_decode_plan_split_tokens(B, Hkv, max_seq_len, BLOCK_SIZE)


def new_workspace(B: int, Hq: int, Hkv: int, D: int, max_seq_len: int, split_tokens: int = 0, device="cuda"):
    """Workspace for kvq_paged_decode_attn."""
    n = kvq_decode_workspace_bytes(B, Hq, Hkv, D, max_seq_len, split_tokens)
    return torch.empty(max(n, 256), dtype=torch.uint8, device=device)


def kvq_paged_decode_attn(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, kv_dtype: int,
                          block_tables: torch.Tensor, seq_lens: torch.Tensor, max_seq_len: int, Hkv: int,
                          k_scale: float, v_scale: float, sm_scale: float, out: torch.Tensor,
                          workspace: torch.Tensor, impl: int = KVQ_IMPL_AUTO, split_tokens: int = 0,
                          stream=None, prepare: bool = False):
    """q bf16 [B][Hq][D]; out bf16 or fp32 [B][Hq][D]; block_tables int32 [B][max_blocks]; seq_lens int32 [B]."""
    B, Hq, D = q.shape
    assert q.dtype == torch.bfloat16 and q.is_contiguous() and out.is_contiguous() and out.shape == q.shape
    _tables(block_tables, seq_lens, B)
    _require(kv_dtype in (KVQ_KV_BF16, KVQ_KV_FP8_E4M3), f"kv_dtype {kv_dtype}: BF16 or FP8 E4M3")
    _caches(k_cache, v_cache, kv_dtype, Hkv, D)
    _same_gpu(q, k_cache, v_cache, block_tables, seq_lens, out, workspace)
    out_dtype = {torch.bfloat16: KVQ_OUT_BF16, torch.float32: KVQ_OUT_F32}[out.dtype]
    return _run("kvq_paged_decode_attn", _lib.kvq_paged_decode_attn_ex, (
        _ptr(q), _ptr(k_cache), _ptr(v_cache), kv_dtype, _ptr(block_tables), block_tables.shape[1],
        _ptr(seq_lens), max_seq_len, B, Hq, Hkv, D, BLOCK_SIZE, k_cache.shape[0], k_scale, v_scale, sm_scale,
        _ptr(out), out_dtype, _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream),
        impl, split_tokens),
        prepare, (q, k_cache, v_cache, block_tables, seq_lens, out, workspace))


KVQ_SCRATCH_MAX_BYTES = 32 * 1024 * 1024


def kvq_paged_decode_attn_scratch(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, kv_dtype: int,
                                  block_tables: torch.Tensor, seq_lens: torch.Tensor, max_seq_len: int, Hkv: int,
                                  k_scale: float, v_scale: float, sm_scale: float, out: torch.Tensor, stream=None,
                                  prepare: bool = False):
    """kvq_paged_decode_attn without a workspace: the split partials go to the
    library's own per-GPU scratch (KVQ_SCRATCH_MAX_BYTES); the call allocates
    nothing.  Calls that overlap on one GPU race."""
    B, Hq, D = q.shape
    assert q.dtype == torch.bfloat16 and q.is_contiguous() and out.is_contiguous() and out.shape == q.shape
    _tables(block_tables, seq_lens, B)
    _require(kv_dtype in (KVQ_KV_BF16, KVQ_KV_FP8_E4M3), f"kv_dtype {kv_dtype}: BF16 or FP8 E4M3")
    _caches(k_cache, v_cache, kv_dtype, Hkv, D)
    _same_gpu(q, k_cache, v_cache, block_tables, seq_lens, out)
    out_dtype = {torch.bfloat16: KVQ_OUT_BF16, torch.float32: KVQ_OUT_F32}[out.dtype]
    return _run("kvq_paged_decode_attn_scratch", _lib.kvq_paged_decode_attn_scratch, (
        _ptr(q), _ptr(k_cache), _ptr(v_cache), kv_dtype, _ptr(block_tables), block_tables.shape[1],
        _ptr(seq_lens), max_seq_len, B, Hq, Hkv, D, BLOCK_SIZE, k_cache.shape[0], k_scale, v_scale, sm_scale,
        _ptr(out), out_dtype, _stream(stream)),
        prepare, (q, k_cache, v_cache, block_tables, seq_lens, out))


def kvq_paged_decode_attn_append(k_new: torch.Tensor, v_new: torch.Tensor, slot_mapping: torch.Tensor,
                                 q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, kv_dtype: int,
                                 block_tables: torch.Tensor, seq_lens: torch.Tensor, max_seq_len: int, Hkv: int,
                                 k_scale: float, v_scale: float, sm_scale: float, out: torch.Tensor,
                                 workspace: torch.Tensor, split_tokens: int = 0, stream=None, prepare: bool = False):
    """kvq_cache_write of each sequence's newest token followed by
    kvq_paged_decode_attn, in one launch.  k_new, v_new bf16 [B][Hkv][D] (token
    dim may be strided); slot_mapping int64 [B], the slot of position
    seq_lens[b] - 1 (or < 0: not written); the rest as kvq_paged_decode_attn."""
    B, Hq, D = q.shape
    assert q.dtype == torch.bfloat16 and q.is_contiguous() and out.is_contiguous() and out.shape == q.shape
    assert k_new.dtype == torch.bfloat16 and v_new.dtype == torch.bfloat16 and slot_mapping.dtype == torch.int64
    assert k_new.shape == (B, Hkv, D) and v_new.shape == k_new.shape and k_new.stride(0) == v_new.stride(0)
    assert k_new.stride(2) == 1 and k_new.stride(1) == D and v_new.stride(2) == 1 and v_new.stride(1) == D
    assert slot_mapping.shape == (B,) and slot_mapping.is_contiguous()
    _tables(block_tables, seq_lens, B)
    _require(kv_dtype in (KVQ_KV_BF16, KVQ_KV_FP8_E4M3), f"kv_dtype {kv_dtype}: BF16 or FP8 E4M3")
    _caches(k_cache, v_cache, kv_dtype, Hkv, D)
    _same_gpu(k_new, v_new, slot_mapping, q, k_cache, v_cache, block_tables, seq_lens, out, workspace)
    out_dtype = {torch.bfloat16: KVQ_OUT_BF16, torch.float32: KVQ_OUT_F32}[out.dtype]
    return _run("kvq_paged_decode_attn_append", _lib.kvq_paged_decode_attn_append, (
        _ptr(k_new), _ptr(v_new), k_new.stride(0), _ptr(slot_mapping), _ptr(q), _ptr(k_cache), _ptr(v_cache),
        kv_dtype, _ptr(block_tables), block_tables.shape[1], _ptr(seq_lens), max_seq_len, B, Hq, Hkv, D, BLOCK_SIZE,
        k_cache.shape[0], k_scale, v_scale, sm_scale, _ptr(out), out_dtype, _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream), split_tokens),
        prepare, (k_new, v_new, slot_mapping, q, k_cache, v_cache, block_tables, seq_lens, out, workspace))


# ---- multi-query decode -------------------------------------------------------

def kvq_decode_workspace_bytes_mq(B: int, q_len: int, Hq: int, Hkv: int, D: int, max_seq_len: int,
                                  split_tokens: int = 0, window: int = 0) -> int:
    return _lib.kvq_decode_workspace_bytes_mq(B, q_len, window, Hq, Hkv, D, max_seq_len, BLOCK_SIZE, split_tokens)


def new_workspace_mq(B: int, q_len: int, Hq: int, Hkv: int, D: int, max_seq_len: int, split_tokens: int = 0,
                     device="cuda", window: int = 0):
    """Workspace for kvq_paged_decode_attn_mq / kvq_nvfp4_paged_decode_attn_mq."""
    n = kvq_decode_workspace_bytes_mq(B, q_len, Hq, Hkv, D, max_seq_len, split_tokens, window)
    return torch.empty(max(n, 256), dtype=torch.uint8, device=device)


def _mq_args(q, block_tables, seq_lens, out, k_cache, v_cache, fmt, Hkv, workspace, *more):
    B, q_len, Hq, D = q.shape
    assert q.dtype == torch.bfloat16 and q.is_contiguous() and out.is_contiguous() and out.shape == q.shape
    _tables(block_tables, seq_lens, B)
    _caches(k_cache, v_cache, fmt, Hkv, D)
    _same_gpu(q, k_cache, v_cache, block_tables, seq_lens, out, workspace, *more)
    out_dtype = {torch.bfloat16: KVQ_OUT_BF16, torch.float32: KVQ_OUT_F32}[out.dtype]
    return B, q_len, Hq, D, out_dtype


def kvq_paged_decode_attn_mq(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, kv_dtype: int,
                             block_tables: torch.Tensor, seq_lens: torch.Tensor, max_seq_len: int, Hkv: int,
                             k_scale: float, v_scale: float, sm_scale: float, out: torch.Tensor,
                             workspace: torch.Tensor, split_tokens: int = 0, window: int = 0, stream=None,
                             prepare: bool = False):
    """q bf16 [B][q_len][Hq][D] (the q_len newest tokens, already in the cache);
    out bf16 or fp32 [B][q_len][Hq][D]; window > 0: sliding-window attention."""
    _require(kv_dtype in (KVQ_KV_BF16, KVQ_KV_FP8_E4M3), f"kv_dtype {kv_dtype}: BF16 or FP8 E4M3")
    B, q_len, Hq, D, out_dtype = _mq_args(q, block_tables, seq_lens, out, k_cache, v_cache, kv_dtype, Hkv, workspace)
    return _run("kvq_paged_decode_attn_mq", _lib.kvq_paged_decode_attn_mq, (
        _ptr(q), q_len, window, _ptr(k_cache), _ptr(v_cache), kv_dtype, _ptr(block_tables), block_tables.shape[1],
        _ptr(seq_lens), max_seq_len, B, Hq, Hkv, D, BLOCK_SIZE, k_cache.shape[0], k_scale, v_scale, sm_scale,
        _ptr(out), out_dtype, _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream),
        split_tokens),
        prepare, (q, k_cache, v_cache, block_tables, seq_lens, out, workspace))


def kvq_paged_decode_attn_mq_append(k_new: torch.Tensor, v_new: torch.Tensor, slot_mapping: torch.Tensor,
                                    q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, kv_dtype: int,
                                    block_tables: torch.Tensor, seq_lens: torch.Tensor, max_seq_len: int, Hkv: int,
                                    k_scale: float, v_scale: float, sm_scale: float, out: torch.Tensor,
                                    workspace: torch.Tensor, split_tokens: int = 0, window: int = 0, stream=None,
                                    prepare: bool = False):
    """kvq_cache_write of the q_len new tokens of every sequence followed by
    kvq_paged_decode_attn_mq, in one launch.  k_new, v_new bf16 [B][q_len][Hkv][D]
    (token rows may be strided); slot_mapping int64 [B][q_len], the slots of
    positions seq_lens[b] - q_len + i (or < 0: not written); the rest as
    kvq_paged_decode_attn_mq."""
    _require(kv_dtype in (KVQ_KV_BF16, KVQ_KV_FP8_E4M3), f"kv_dtype {kv_dtype}: BF16 or FP8 E4M3")
    B, q_len, Hq, D, out_dtype = _mq_args(q, block_tables, seq_lens, out, k_cache, v_cache, kv_dtype, Hkv, workspace,
                                          k_new, v_new, slot_mapping)
    assert k_new.dtype == torch.bfloat16 and v_new.dtype == torch.bfloat16 and slot_mapping.dtype == torch.int64
    assert k_new.shape == (B, q_len, Hkv, D) and v_new.shape == k_new.shape
    assert k_new.stride(0) == q_len * k_new.stride(1) and k_new.stride(1) == v_new.stride(1)
    assert v_new.stride(0) == q_len * v_new.stride(1)
    for t in (k_new, v_new):
        assert t.stride(3) == 1 and t.stride(2) == D
    assert slot_mapping.shape == (B, q_len) and slot_mapping.is_contiguous()
    return _run("kvq_paged_decode_attn_mq_append", _lib.kvq_paged_decode_attn_mq_append, (
        _ptr(k_new), _ptr(v_new), k_new.stride(1), _ptr(slot_mapping), _ptr(q), q_len, window, _ptr(k_cache),
        _ptr(v_cache), kv_dtype, _ptr(block_tables), block_tables.shape[1], _ptr(seq_lens), max_seq_len, B, Hq, Hkv,
        D, BLOCK_SIZE, k_cache.shape[0], k_scale, v_scale, sm_scale, _ptr(out), out_dtype, _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream), split_tokens),
        prepare, (k_new, v_new, slot_mapping, q, k_cache, v_cache, block_tables, seq_lens, out, workspace))


def kvq_nvfp4_paged_decode_attn_mq(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                                   block_tables: torch.Tensor, seq_lens: torch.Tensor, max_seq_len: int, Hkv: int,
                                   k_gscale: float, v_gscale: float, sm_scale: float, out: torch.Tensor,
                                   workspace: torch.Tensor, split_tokens: int = 0, window: int = 0,
                                   stream=None, prepare: bool = False):
    """NVFP4 caches; otherwise as kvq_paged_decode_attn_mq."""
    B, q_len, Hq, D, out_dtype = _mq_args(q, block_tables, seq_lens, out, k_cache, v_cache, KVQ_FORMAT_NVFP4, Hkv,
                                          workspace)
    return _run("kvq_nvfp4_paged_decode_attn_mq", _lib.kvq_nvfp4_paged_decode_attn_mq, (
        _ptr(q), q_len, window, _ptr(k_cache), _ptr(v_cache), _ptr(block_tables), block_tables.shape[1],
        _ptr(seq_lens), max_seq_len, B, Hq, Hkv, D, BLOCK_SIZE, k_cache.shape[0], k_gscale, v_gscale, sm_scale,
        _ptr(out), out_dtype, _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream),
        split_tokens),
        prepare, (q, k_cache, v_cache, block_tables, seq_lens, out, workspace))


# ---- block copies for a host-memory KV tier ----------------------------------------


def kvq_cache_block_bytes(kv_format: int, Hkv: int, D: int) -> int:
    return _lib.kvq_cache_block_bytes(kv_format, Hkv, D, BLOCK_SIZE)


def _nbytes(t: torch.Tensor) -> int:
    return t.numel() * t.element_size()


def _block_cache(cache: torch.Tensor, block_bytes: int) -> None:
    _require(cache.is_contiguous() and block_bytes > 0 and _nbytes(cache) % block_bytes == 0,
             "a cache for block copies is contiguous and holds whole blocks of block_bytes")


def kvq_gather_blocks(cache: torch.Tensor, block_bytes: int, ids: torch.Tensor, dst: torch.Tensor, stream=None):
    assert ids.dtype == torch.int32 and ids.is_contiguous() and _nbytes(dst) >= ids.numel() * block_bytes
    _block_cache(cache, block_bytes)
    _require(dst.is_contiguous(), "dst must be contiguous")
    _same_gpu(cache, ids, dst)
    _check("kvq_gather_blocks", _lib.kvq_gather_blocks(_ptr(cache), block_bytes, _ptr(ids), ids.numel(), _ptr(dst),
                                                       _stream(stream)))


def kvq_scatter_blocks(src: torch.Tensor, block_bytes: int, ids: torch.Tensor, cache: torch.Tensor, stream=None):
    assert ids.dtype == torch.int32 and ids.is_contiguous() and _nbytes(src) >= ids.numel() * block_bytes
    _block_cache(cache, block_bytes)
    _require(src.is_contiguous(), "src must be contiguous")
    _same_gpu(cache, ids, src)
    _check("kvq_scatter_blocks", _lib.kvq_scatter_blocks(_ptr(src), block_bytes, _ptr(ids), ids.numel(),
                                                         _ptr(cache), _stream(stream)))


def kvq_offload_blocks(k_cache: torch.Tensor, v_cache: torch.Tensor, block_bytes: int, ids: torch.Tensor,
                       staging: torch.Tensor, host_dst: torch.Tensor, stream=None):
    """K blocks then V blocks of `ids` into host_dst (pinned, >= 2 * n * block_bytes bytes)."""
    n = ids.numel()
    assert ids.dtype == torch.int32 and ids.is_contiguous()
    assert _nbytes(staging) >= 2 * n * block_bytes and _nbytes(host_dst) >= 2 * n * block_bytes
    assert host_dst.device.type == "cpu" and host_dst.is_contiguous()
    _block_cache(k_cache, block_bytes)
    _block_cache(v_cache, block_bytes)
    _require(staging.is_contiguous(), "staging must be contiguous")
    _same_gpu(k_cache, v_cache, ids, staging)
    _check("kvq_offload_blocks", _lib.kvq_offload_blocks(_ptr(k_cache), _ptr(v_cache), block_bytes, _ptr(ids), n,
                                                         _ptr(staging), _ptr(host_dst), _stream(stream)))


def kvq_restore_blocks(host_src: torch.Tensor, staging: torch.Tensor, block_bytes: int, ids: torch.Tensor,
                       k_cache: torch.Tensor, v_cache: torch.Tensor, stream=None):
    n = ids.numel()
    assert ids.dtype == torch.int32 and ids.is_contiguous()
    assert _nbytes(staging) >= 2 * n * block_bytes and _nbytes(host_src) >= 2 * n * block_bytes
    assert host_src.device.type == "cpu" and host_src.is_contiguous()
    _block_cache(k_cache, block_bytes)
    _block_cache(v_cache, block_bytes)
    _require(staging.is_contiguous(), "staging must be contiguous")
    _same_gpu(k_cache, v_cache, ids, staging)
    _check("kvq_restore_blocks", _lib.kvq_restore_blocks(_ptr(host_src), _ptr(staging), block_bytes, _ptr(ids), n,
                                                         _ptr(k_cache), _ptr(v_cache), _stream(stream)))


# ---- FP8 Q and P variant ---------------------------------------------------------------

def kvq_paged_decode_attn_fp8qp(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                                block_tables: torch.Tensor, seq_lens: torch.Tensor, max_seq_len: int, Hkv: int,
                                q_scale: float, k_scale: float, v_scale: float, sm_scale: float, out: torch.Tensor,
                                workspace: torch.Tensor, split_tokens: int = 0, window: int = 0, stream=None,
                                prepare: bool = False):
    """FP8 cache, FP8 Q (q_scale) and FP8 P on FP8 MFMA; q [B][q_len][Hq][D] as kvq_paged_decode_attn_mq."""
    B, q_len, Hq, D, out_dtype = _mq_args(q, block_tables, seq_lens, out, k_cache, v_cache, KVQ_KV_FP8_E4M3, Hkv,
                                          workspace)
    return _run("kvq_paged_decode_attn_fp8qp", _lib.kvq_paged_decode_attn_fp8qp, (
        _ptr(q), q_len, window, _ptr(k_cache), _ptr(v_cache), _ptr(block_tables), block_tables.shape[1],
        _ptr(seq_lens), max_seq_len, B, Hq, Hkv, D, BLOCK_SIZE, k_cache.shape[0], q_scale, k_scale, v_scale,
        sm_scale, _ptr(out), out_dtype, _ptr(workspace), workspace.numel() * workspace.element_size(),
        _stream(stream), split_tokens),
        prepare, (q, k_cache, v_cache, block_tables, seq_lens, out, workspace))
