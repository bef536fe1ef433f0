"""CPU oracle for the FP8 / NVFP4 paged decode-attention path.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, by ``__graft_entry__.smoke()``
and by the ``cpu_baseline`` leg of ``bench.py``; never by the product package.
It shares no code with the GPU path (``kvq_oracle.c`` is plain C, fp64,
brute-force codecs) and this wrapper does nothing but marshal numpy arrays.

The definitions and their sources are documented in ``kvq_oracle.h``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kvq_oracle.c")
# KVQ_ORACLE_SANITIZE=1 selects the AddressSanitizer + UndefinedBehaviorSanitizer
# build (its process must preload gcc's libasan; tests/test_oracle_sanitizers.py)
SANITIZED = os.environ.get("KVQ_ORACLE_SANITIZE") == "1"
_PLAIN_LIB = os.path.join(_HERE, "libkvq_oracle.so")
_SAN_LIB = os.path.join(_HERE, "libkvq_oracle_san.so")
_LIB_PATH = _SAN_LIB if SANITIZED else _PLAIN_LIB
_SAN_FLAGS = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
              "-fno-sanitize-recover=all"]

KV_BF16, KV_FP8, KV_NVFP4 = 0, 1, 2


def build(force: bool = False, sanitize: bool = SANITIZED) -> str:
    """Compile the oracle with gcc (no fast-math, no fp contraction); with
    sanitize, the instrumented variant."""
    path = _SAN_LIB if sanitize else _PLAIN_LIB
    if force or not os.path.exists(path) or (
        os.path.getmtime(path) < max(os.path.getmtime(_SRC), os.path.getmtime(os.path.join(_HERE, "kvq_oracle.h")))):
        tmp = path + ".tmp%d" % os.getpid()
        opt = _SAN_FLAGS if sanitize else ["-O2"]
        subprocess.check_call(["gcc", *opt, "-std=c99", "-fPIC", "-shared", "-ffp-contract=off",
                               "-fno-fast-math", "-Wall", "-o", tmp, _SRC, "-lm", "-lpthread"])
        os.replace(tmp, path)
    return path


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        build()
        L = ctypes.CDLL(_LIB_PATH)
        P, I, I64, F, D = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float, ctypes.c_double
        U8, U16 = ctypes.c_uint8, ctypes.c_uint16
        sig = {
            "kvqo_e4m3_value": (D, [U8]),
            "kvqo_e4m3_encode": (U8, [F]),
            "kvqo_e4m3_encode_array": (None, [P, P, I64]),
            "kvqo_bf16_to_float": (F, [U16]),
            "kvqo_e4m3_quantize": (U8, [U16, F]),
            "kvqo_e2m1_value": (D, [U8]),
            "kvqo_e2m1_encode": (U8, [F]),
            "kvqo_calibrate": (I, [P, P, I]),
            "kvqo_nvfp4_calibrate": (I, [P, P, I]),
            "kvqo_amax_bf16": (F, [P, I64, I64, I64]),
            "kvqo_nvfp4_region_bytes": (I64, [I, I]),
            "kvqo_cache_write": (None, [P, P, I64, P, I, I, I, P, P, I, I, F, F, I]),
            "kvqo_nvfp4_cache_write": (None, [P, P, I64, P, I, I, I, P, P, I, F, F, I]),
            "kvqo_nvfp4_k_value": (D, [P, I64, I, I, I, I, I, F]),
            "kvqo_nvfp4_v_value": (D, [P, I64, I, I, I, I, I, F]),
            "kvqo_decode_attn": (None, [P, P, P, I, P, I, P, I, I, I, I, I, F, F, F, P, I]),
            "kvqo_decode_attn_units": (None, [P, P, P, I, P, I, P, I, I, I, I, I, F, F, F, P, I, P, I]),
            "kvqo_block_bytes": (ctypes.c_size_t, [I, I, I, I]),
            "kvqo_gather_blocks": (None, [P, ctypes.c_size_t, P, I, P]),
            "kvqo_scatter_blocks": (None, [P, ctypes.c_size_t, P, I, P]),
            "kvqo_decode_attn_fp8qp": (None, [P, I, I, P, P, P, I, P, I, I, I, I, I, F, F, F, F, P, I]),
            "kvqo_decode_attn_fp8qp_tol": (None, [P, I, I, P, P, P, I, P, I, I, I, I, I, F, F, F, F,
                                                  ctypes.c_double, P, P, P, P]),
            "kvqo_decode_attn_mq": (None, [P, I, I, P, P, I, P, I, P, I, I, I, I, I, F, F, F, P, I]),
            "kvqo_fp8_cos_sim": (D, [P, I64, F]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _ptr(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"], "oracle inputs must be C-contiguous"
    return a.ctypes.data


def _bits16(a) -> np.ndarray:
    """bf16 data as uint16 bit patterns (accepts uint16 arrays or torch bf16 tensors)."""
    if isinstance(a, np.ndarray):
        assert a.dtype == np.uint16
        return np.ascontiguousarray(a)
    import torch  # local: the oracle itself needs only numpy
    assert a.dtype == torch.bfloat16
    return np.ascontiguousarray(a.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16))


# ---- codecs ---------------------------------------------------------------

def e4m3_value(code: int) -> float:
    return lib().kvqo_e4m3_value(code)


def e4m3_table() -> np.ndarray:
    return np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)


def e4m3_encode(y: float) -> int:
    return lib().kvqo_e4m3_encode(y)


def e4m3_encode_array(y) -> np.ndarray:
    """Brute-force encode of every element of a float32 array."""
    a = np.ascontiguousarray(np.asarray(y, dtype=np.float32).reshape(-1))
    out = np.zeros(a.size, dtype=np.uint8)
    lib().kvqo_e4m3_encode_array(_ptr(a), _ptr(out), a.size)
    return out


def e4m3_quantize(x_bf16_bits: int, scale: float) -> int:
    return lib().kvqo_e4m3_quantize(x_bf16_bits, scale)


def e2m1_value(nib: int) -> float:
    return lib().kvqo_e2m1_value(nib)


def e2m1_encode(y: float) -> int:
    return lib().kvqo_e2m1_encode(y)


# ---- calibration ----------------------------------------------------------

def calibrate(amax) -> np.ndarray:
    a = np.ascontiguousarray(np.asarray(amax, dtype=np.float32).reshape(-1))
    out = np.zeros_like(a)
    rc = lib().kvqo_calibrate(_ptr(a), _ptr(out), a.size)
    if rc != 0:
        raise ValueError("amax must be finite and non-negative")
    return out


def nvfp4_calibrate(amax) -> np.ndarray:
    a = np.ascontiguousarray(np.asarray(amax, dtype=np.float32).reshape(-1))
    out = np.zeros_like(a)
    rc = lib().kvqo_nvfp4_calibrate(_ptr(a), _ptr(out), a.size)
    if rc != 0:
        raise ValueError("amax must be finite and non-negative")
    return out


def amax_bf16(x) -> float:
    """max |x| over a bf16 array of any shape (flattened rows of the last dim)."""
    b = _bits16(x)
    cols = b.shape[-1] if b.ndim else 1
    rows = b.size // max(cols, 1)
    return lib().kvqo_amax_bf16(_ptr(b), rows, cols, cols)


# ---- cache ----------------------------------------------------------------

def nvfp4_region_bytes(D: int, block_size: int) -> int:
    return lib().kvqo_nvfp4_region_bytes(D, block_size)


def new_caches(kv_dtype: int, num_blocks: int, Hkv: int, D: int, block_size: int, fill: int = 0):
    """Zero- (or `fill`-) initialised K and V caches in the documented layouts."""
    if kv_dtype == KV_BF16:
        shp_k, shp_v, dt = (num_blocks, Hkv, block_size, D), (num_blocks, Hkv, D, block_size), np.uint16
    elif kv_dtype == KV_FP8:
        shp_k, shp_v, dt = (num_blocks, Hkv, block_size, D), (num_blocks, Hkv, D, block_size), np.uint8
    else:
        r = nvfp4_region_bytes(D, block_size)
        shp_k = shp_v = (num_blocks, Hkv, r)
        dt = np.uint8
    return np.full(shp_k, fill, dtype=dt), np.full(shp_v, fill, dtype=dt)


def cache_write(k, v, slot_mapping, k_cache: np.ndarray, v_cache: np.ndarray, kv_dtype: int,
                k_scale: float = 1.0, v_scale: float = 1.0, nthreads: int = 1) -> None:
    """k, v: bf16 [T][Hkv][D]; writes in place (nthreads: see kvq_oracle.h)."""
    kb, vb = _bits16(k), _bits16(v)
    T, Hkv, D = kb.shape
    sm = np.ascontiguousarray(np.asarray(slot_mapping, dtype=np.int64))
    assert sm.shape == (T,)
    bs = k_cache.shape[2] if kv_dtype != KV_NVFP4 else None
    assert kv_dtype in (KV_BF16, KV_FP8)
    lib().kvqo_cache_write(_ptr(kb), _ptr(vb), Hkv * D, _ptr(sm), T, Hkv, D,
                           _ptr(k_cache), _ptr(v_cache), bs, kv_dtype, k_scale, v_scale, nthreads)


def nvfp4_cache_write(k, v, slot_mapping, k_cache: np.ndarray, v_cache: np.ndarray, block_size: int,
                      k_gscale: float, v_gscale: float, nthreads: int = 1) -> None:
    kb, vb = _bits16(k), _bits16(v)
    T, Hkv, D = kb.shape
    sm = np.ascontiguousarray(np.asarray(slot_mapping, dtype=np.int64))
    lib().kvqo_nvfp4_cache_write(_ptr(kb), _ptr(vb), Hkv * D, _ptr(sm), T, Hkv, D,
                                 _ptr(k_cache), _ptr(v_cache), block_size, k_gscale, v_gscale, nthreads)


def nvfp4_values(cache: np.ndarray, which: str, slots, Hkv: int, D: int, block_size: int,
                 gscale: float) -> np.ndarray:
    """Dequantized [len(slots)][Hkv][D] values of an NVFP4 K ('k') or V ('v') cache."""
    fn = lib().kvqo_nvfp4_k_value if which == "k" else lib().kvqo_nvfp4_v_value
    out = np.zeros((len(slots), Hkv, D))
    for i, s in enumerate(slots):
        for g in range(Hkv):
            for d in range(D):
                out[i, g, d] = fn(_ptr(cache), int(s), g, d, Hkv, D, block_size, gscale)
    return out


# ---- attention ------------------------------------------------------------

def decode_attn(q, k_cache: np.ndarray, v_cache: np.ndarray, kv_dtype: int, block_tables, seq_lens,
                Hkv: int, block_size: int, k_scale: float, v_scale: float, sm_scale: float,
                units=None, nthreads: int = 1) -> np.ndarray:
    """fp64 attention output [B][Hq][D] (or [n_units][D] for a list of (b, h) units)."""
    qb = _bits16(q)
    B, Hq, D = qb.shape
    bt = np.ascontiguousarray(np.asarray(block_tables, dtype=np.int32))
    sl = np.ascontiguousarray(np.asarray(seq_lens, dtype=np.int32))
    assert bt.shape[0] == B and sl.shape == (B,)
    kc, vc = np.ascontiguousarray(k_cache), np.ascontiguousarray(v_cache)
    if units is None:
        out = np.zeros((B, Hq, D), dtype=np.float64)
        lib().kvqo_decode_attn(_ptr(qb), _ptr(kc), _ptr(vc), kv_dtype, _ptr(bt), bt.shape[1], _ptr(sl),
                               B, Hq, Hkv, D, block_size, k_scale, v_scale, sm_scale, _ptr(out), nthreads)
    else:
        u = np.ascontiguousarray(np.asarray(units, dtype=np.int32).reshape(-1, 2))
        out = np.zeros((u.shape[0], D), dtype=np.float64)
        lib().kvqo_decode_attn_units(_ptr(qb), _ptr(kc), _ptr(vc), kv_dtype, _ptr(bt), bt.shape[1],
                                     _ptr(sl), B, Hq, Hkv, D, block_size, k_scale, v_scale, sm_scale,
                                     _ptr(u), u.shape[0], _ptr(out), nthreads)
    return out


def decode_attn_mq(q, k_cache: np.ndarray, v_cache: np.ndarray, kv_dtype: int, block_tables, seq_lens,
                   Hkv: int, block_size: int, k_scale: float, v_scale: float, sm_scale: float,
                   nthreads: int = 1, window: int = 0) -> np.ndarray:
    """fp64 multi-query attention output [B][q_len][Hq][D] for q [B][q_len][Hq][D]
    (query i of sequence b, at position p = seq_len - q_len + i, attends causally
    to tokens 0 .. p, or to its `window` newest tokens when window > 0)."""
    qb = _bits16(q)
    B, q_len, Hq, D = qb.shape
    bt = np.ascontiguousarray(np.asarray(block_tables, dtype=np.int32))
    sl = np.ascontiguousarray(np.asarray(seq_lens, dtype=np.int32))
    assert bt.shape[0] == B and sl.shape == (B,)
    kc, vc = np.ascontiguousarray(k_cache), np.ascontiguousarray(v_cache)
    out = np.zeros((B, q_len, Hq, D), dtype=np.float64)
    lib().kvqo_decode_attn_mq(_ptr(qb), q_len, window, _ptr(kc), _ptr(vc), kv_dtype, _ptr(bt), bt.shape[1], _ptr(sl),
                              B, Hq, Hkv, D, block_size, k_scale, v_scale, sm_scale, _ptr(out), nthreads)
    return out


def decode_attn_fp8qp(q, k_cache: np.ndarray, v_cache: np.ndarray, block_tables, seq_lens, Hkv: int,
                      block_size: int, q_scale: float, k_scale: float, v_scale: float, sm_scale: float,
                      nthreads: int = 1, window: int = 0) -> np.ndarray:
    """FP8 Q and P attention [B][q_len][Hq][D] over an FP8 cache (see kvq_oracle.h)."""
    qb = _bits16(q)
    B, q_len, Hq, D = qb.shape
    bt = np.ascontiguousarray(np.asarray(block_tables, dtype=np.int32))
    sl = np.ascontiguousarray(np.asarray(seq_lens, dtype=np.int32))
    kc, vc = np.ascontiguousarray(k_cache), np.ascontiguousarray(v_cache)
    out = np.zeros((B, q_len, Hq, D), dtype=np.float64)
    lib().kvqo_decode_attn_fp8qp(_ptr(qb), q_len, window, _ptr(kc), _ptr(vc), _ptr(bt), bt.shape[1], _ptr(sl),
                                 B, Hq, Hkv, D, block_size, q_scale, k_scale, v_scale, sm_scale, _ptr(out),
                                 nthreads)
    return out


def decode_attn_fp8qp_tol(q, k_cache: np.ndarray, v_cache: np.ndarray, block_tables, seq_lens, Hkv: int,
                          block_size: int, q_scale: float, k_scale: float, v_scale: float, sm_scale: float,
                          eps: float, window: int = 0, weights: bool = False):
    """(tol, n_open): per-element tolerance [B][q_len][Hq][D] of
    decode_attn_fp8qp for an implementation meeting assumptions A1-A3 of
    kvq_oracle.h with accuracy eps.  weights=True appends the definition's
    weights w_t and their bounds delta_t, [B][q_len][Hq][max seq_len]."""
    qb = _bits16(q)
    B, q_len, Hq, D = qb.shape
    bt = np.ascontiguousarray(np.asarray(block_tables, dtype=np.int32))
    sl = np.ascontiguousarray(np.asarray(seq_lens, dtype=np.int32))
    kc, vc = np.ascontiguousarray(k_cache), np.ascontiguousarray(v_cache)
    tol = np.zeros((B, q_len, Hq, D), dtype=np.float64)
    n = np.zeros(1, dtype=np.int64)
    max_l = max(1, int(sl.max())) if sl.size else 1
    wt = np.zeros((B, q_len, Hq, max_l)) if weights else None
    dt = np.zeros_like(wt) if weights else None
    lib().kvqo_decode_attn_fp8qp_tol(_ptr(qb), q_len, window, _ptr(kc), _ptr(vc), _ptr(bt), bt.shape[1], _ptr(sl),
                                     B, Hq, Hkv, D, block_size, q_scale, k_scale, v_scale, sm_scale, eps,
                                     _ptr(tol), _ptr(n), _ptr(wt) if weights else None,
                                     _ptr(dt) if weights else None)
    if weights:
        return tol, int(n[0]), wt, dt
    return tol, int(n[0])


def fp8_cos_sim(x, scale: float) -> float:
    b = _bits16(x).reshape(-1)
    return lib().kvqo_fp8_cos_sim(_ptr(b), b.size, scale)


# ---- block copies for a host-memory tier ---------------------------------------

def block_bytes(kv_dtype: int, Hkv: int, D: int, block_size: int = 16) -> int:
    return lib().kvqo_block_bytes(kv_dtype, Hkv, D, block_size)


def gather_blocks(cache: np.ndarray, ids, block_bytes_: int) -> np.ndarray:
    """Blocks ids[i] of a cache (any dtype, blocks of block_bytes_ bytes) as [n][block_bytes_] uint8."""
    c = np.ascontiguousarray(cache).view(np.uint8).reshape(-1)
    i = np.ascontiguousarray(np.asarray(ids, dtype=np.int32))
    out = np.zeros((i.size, block_bytes_), dtype=np.uint8)
    lib().kvqo_gather_blocks(_ptr(c), block_bytes_, _ptr(i), i.size, _ptr(out))
    return out


def scatter_blocks(src: np.ndarray, ids, block_bytes_: int, cache: np.ndarray) -> None:
    """Writes src[i] (uint8 [n][block_bytes_]) to block ids[i] of cache, in place."""
    assert cache.flags["C_CONTIGUOUS"]
    c = cache.view(np.uint8).reshape(-1)   # a view: writes land in cache
    i = np.ascontiguousarray(np.asarray(ids, dtype=np.int32))
    s = np.ascontiguousarray(src, dtype=np.uint8)
    lib().kvqo_scatter_blocks(_ptr(s), block_bytes_, _ptr(i), i.size, _ptr(c))
