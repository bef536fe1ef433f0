"""Calls every entry point of the oracle library on small seeded numpy inputs
(no torch), for tests/test_oracle_sanitizers.py, which runs it with the
AddressSanitizer + UndefinedBehaviorSanitizer build of the oracle
(KVQ_ORACLE_SANITIZE=1, gcc's libasan preloaded).  A sanitizer report aborts
the process; on success the last line is "oracle sanitize driver: ok".
The values are not checked here (the oracle's pins do that); the point is
that every code path runs under the sanitizers: the codecs over all codes,
the cache writes (skipped and in-range slots), every attention definition
(single- and multi-query, window, FP8 Q/P with its tolerance, units, threads) and
the block copies."""
import os
import sys

import numpy as np

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
import oracle  # noqa: E402


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns, round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def paging(lens, bs, rng):
    nblk = [(L + bs - 1) // bs for L in lens]
    nb = max(sum(nblk), 1)
    perm = rng.permutation(nb).astype(np.int32)
    bt = np.zeros((len(lens), max(max(nblk), 1)), dtype=np.int32)
    slots, cur = [], 0
    for b, L in enumerate(lens):
        ids = perm[cur:cur + nblk[b]]
        bt[b, :nblk[b]] = ids
        pos = np.arange(L)
        slots.append(ids[pos // bs].astype(np.int64) * bs + pos % bs)
        cur += nblk[b]
    return bt, np.concatenate(slots), nb


def main():
    rng = np.random.default_rng(7)
    # codecs and calibration
    assert oracle.e4m3_table().shape == (256,)
    oracle.e4m3_encode_array(rng.standard_normal(4096).astype(np.float32) * 300)
    oracle.e4m3_encode_array(np.array([np.inf, -np.inf, np.nan, 0.0, -0.0, 1e-30, 500.0], dtype=np.float32))
    for n in range(16):
        oracle.e2m1_value(n)
    for y in (0.25, 0.75, 2.5, 7.0, -5.0):
        oracle.e2m1_encode(y)
    oracle.e4m3_quantize(0x3F80, 0.5)
    oracle.calibrate([0.0, 1.0, 448.0 / 1.05])
    oracle.nvfp4_calibrate([0.0, 3.0])
    try:
        oracle.calibrate([float("nan")])
    except ValueError:
        pass

    lens = [70, 33, 0, 130]
    B, Hq, Hkv, D, bs = len(lens), 8, 2, 64, 16
    bt, slots, nb = paging(lens, bs, rng)
    T = int(sum(lens))
    k = bf16_bits(rng.standard_normal((T, Hkv, D)))
    v = bf16_bits(rng.standard_normal((T, Hkv, D)))
    q = bf16_bits(rng.standard_normal((B, Hq, D)))
    oracle.amax_bf16(k)
    ks, vs = (float(s) for s in oracle.calibrate([oracle.amax_bf16(k), oracle.amax_bf16(v)]))
    sm = 1.0 / np.sqrt(D)
    slots_skip = slots.copy()
    slots_skip[::5] = -1
    for kvd in (oracle.KV_FP8, oracle.KV_BF16):
        kc, vc = oracle.new_caches(kvd, nb, Hkv, D, bs, fill=0)
        oracle.cache_write(k, v, slots_skip, kc, vc, kvd, ks, vs)
        oracle.cache_write(k, v, slots, kc, vc, kvd, ks, vs)
        oracle.decode_attn(q, kc, vc, kvd, bt, lens, Hkv, bs, ks, vs, sm, nthreads=2)
        oracle.decode_attn(q, kc, vc, kvd, bt, lens, Hkv, bs, ks, vs, sm, units=[(0, 1), (3, 7), (2, 0)])
        qm = bf16_bits(rng.standard_normal((B, 3, Hq, D)))
        oracle.decode_attn_mq(qm, kc, vc, kvd, bt, lens, Hkv, bs, ks, vs, sm, nthreads=2)
        oracle.decode_attn_mq(qm, kc, vc, kvd, bt, lens, Hkv, bs, ks, vs, sm, window=20)
        bb = oracle.block_bytes(kvd, Hkv, D, bs)
        ids = [0, nb - 1, 1]
        got = oracle.gather_blocks(kc, ids, bb)
        oracle.scatter_blocks(got, ids, bb, kc)
        oracle.fp8_cos_sim(k, ks)
        if kvd == oracle.KV_FP8:
            qs = float(oracle.calibrate([oracle.amax_bf16(q)])[0])
            qm1 = bf16_bits(rng.standard_normal((B, 2, Hq, D)))
            oracle.decode_attn_fp8qp(qm1, kc, vc, bt, lens, Hkv, bs, qs, ks, vs, sm, nthreads=2, window=40)
            oracle.decode_attn_fp8qp_tol(qm1, kc, vc, bt, lens, Hkv, bs, qs, ks, vs, sm, 2.0 ** -10)
            oracle.decode_attn_fp8qp_tol(qm1, kc, vc, bt, lens, Hkv, bs, qs, ks, vs, sm, 2.0 ** -10, window=40,
                                         weights=True)
    # NVFP4
    gk, gv = (float(s) for s in oracle.nvfp4_calibrate([oracle.amax_bf16(k), oracle.amax_bf16(v)]))
    kc, vc = oracle.new_caches(oracle.KV_NVFP4, nb, Hkv, D, bs, fill=0)
    oracle.nvfp4_cache_write(k, v, slots_skip, kc, vc, bs, gk, gv)
    oracle.nvfp4_cache_write(k, v, slots, kc, vc, bs, gk, gv)
    oracle.nvfp4_values(kc, "k", slots[:5], Hkv, D, bs, gk)
    oracle.nvfp4_values(vc, "v", slots[:5], Hkv, D, bs, gv)
    oracle.decode_attn(q, kc, vc, oracle.KV_NVFP4, bt, lens, Hkv, bs, gk, gv, sm, nthreads=2)
    print("oracle sanitize driver: ok", flush=True)


if __name__ == "__main__":
    main()
