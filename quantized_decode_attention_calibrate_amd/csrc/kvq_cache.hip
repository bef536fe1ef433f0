// kvq_cache.hip -- calibration observation (amax), E4M3 codec utilities and
// the paged KV-cache write (quantize + scatter by slot mapping).
//
// The calibration guide for the Radiance R9700 fork (calibrator paragraph)
// defines what is observed (BF16 K/V absolute maxima, combined by maximum)
// and the OCP E4M3 format with maximum 448; its storage paragraph fixes FP8
// at one byte per element.  These kernels are HBM/latency bound: one pass
// over the input, 16-byte loads, no LDS.
#include <type_traits>

#include "kvq_device.h"
#include "kvq_internal.h"

namespace kvq {

// ---- amax ------------------------------------------------------------------
// |bf16| ordered as an unsigned 15-bit magnitude equals the order of the
// values (NaN patterns above Inf), so the running max is an integer max on
// the fp32 bit pattern of the magnitude.  Each thread walks 16-byte vectors
// (row, column) with a carry instead of a per-element 64-bit division, keeps
// kAmaxUnroll loads in flight, and the work-group reduces through LDS to one
// atomicMax (skipped when the running value is already larger).
constexpr int kAmaxThreads = 256;
constexpr int kAmaxUnroll = 4;

__device__ __forceinline__ uint32_t absmax8(const u32x4& w) {
    uint32_t m = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) m = max(m, max(w[j] & 0x7FFFu, (w[j] >> 16) & 0x7FFFu));
    return m;
}

__global__ void __launch_bounds__(kAmaxThreads) amax_bf16_kernel(const uint16_t* __restrict__ x, int64_t rows,
                                                                 int64_t cols, int64_t stride,
                                                                 uint32_t* __restrict__ amax_bits) {
    __shared__ uint32_t red[kAmaxThreads / 64];
    uint32_t m = 0;
    const int64_t nthreads = (int64_t)gridDim.x * blockDim.x;
    const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if ((cols & 7) == 0 && (stride & 7) == 0) {
        // vector i = (r, c): element offset r * stride + 8c; thread i, i + nthreads, ...
        const int64_t vpr = cols >> 3;
        int64_t r = tid / vpr, c = tid - r * vpr;
        const int64_t dr = nthreads / vpr, dc = nthreads - dr * vpr;
        while (r < rows) {
            u32x4 w[kAmaxUnroll];
#pragma unroll
            for (int u = 0; u < kAmaxUnroll; ++u) {
                if (r < rows) {
                    w[u] = *reinterpret_cast<const u32x4*>(x + r * stride + (c << 3));
                    c += dc;
                    r += dr;
                    if (c >= vpr) {
                        c -= vpr;
                        ++r;
                    }
                } else {
                    w[u] = u32x4{0u, 0u, 0u, 0u};
                }
            }
#pragma unroll
            for (int u = 0; u < kAmaxUnroll; ++u) m = max(m, absmax8(w[u]));
        }
    } else {
        const int64_t n = rows * cols;
        int64_t r = tid / cols, c = tid - r * cols;
        const int64_t dr = nthreads / cols, dc = nthreads - dr * cols;
        for (int64_t i = tid; i < n; i += nthreads) {
            m = max(m, (uint32_t)(x[r * stride + c] & 0x7FFFu));
            c += dc;
            r += dr;
            if (c >= cols) {
                c -= cols;
                ++r;
            }
        }
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1)
        m = max(m, (uint32_t)__builtin_amdgcn_ds_bpermute((__lane_id() ^ o) << 2, (int)m));
    if (__lane_id() == 0) red[threadIdx.x >> 6] = m;
    __syncthreads();
    if (threadIdx.x == 0) {
#pragma unroll
        for (int w = 1; w < kAmaxThreads / 64; ++w) m = max(m, red[w]);
        const uint32_t bits = m << 16;
        if (m != 0 && bits > __hip_atomic_load(amax_bits, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT))
            atomicMax(amax_bits, bits);
    }
}

hipError_t launch_amax_bf16(const void* x, int64_t rows, int64_t cols, int64_t stride, float* amax,
                            hipStream_t st) {
    const int64_t work = ((cols & 7) == 0 && (stride & 7) == 0) ? rows * (cols >> 3) : rows * cols;
    // about 16 vectors per thread, at most 4 work-groups per CU
    int64_t blocks = (work + kAmaxThreads * 16 - 1) / (kAmaxThreads * 16);
    if (blocks > 1024) blocks = 1024;
    if (blocks < 1) blocks = 1;
    hipLaunchKernelGGL(amax_bf16_kernel, dim3((unsigned)blocks), dim3(kAmaxThreads), 0, st,
                       (const uint16_t*)x, rows, cols, stride, (uint32_t*)amax);
    return hipGetLastError();
}

// ---- codec utilities -------------------------------------------------------
__global__ void __launch_bounds__(256) e4m3_encode_kernel(const float* __restrict__ y,
                                                          uint8_t* __restrict__ codes, int64_t n) {
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (; i < n; i += stride) codes[i] = (uint8_t)e4m3_encode(y[i]);
}

__global__ void __launch_bounds__(256) e4m3_decode_kernel(const uint8_t* __restrict__ codes, void* out,
                                                          int kind, int64_t n) {
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (; i < n; i += stride) {
        uint32_t w = codes[i];
        if (kind == 0) {
            ((float*)out)[i] = e4m3x2_to_f32(w, false)[0];
        } else if (kind == 1) {
            ((_Float16*)out)[i] = e4m3x2_to_f16(w, false)[0];
        } else {
            ((__bf16*)out)[i] = e4m3x2_to_bf16(w, false)[0];
        }
    }
}

static unsigned grid_for(int64_t n) {
    int64_t b = (n + 255) / 256;
    return (unsigned)(b < 1 ? 1 : (b > 8192 ? 8192 : b));
}

hipError_t launch_e4m3_encode(const float* y, uint8_t* codes, int64_t n, hipStream_t st) {
    hipLaunchKernelGGL(e4m3_encode_kernel, dim3(grid_for(n)), dim3(256), 0, st, y, codes, n);
    return hipGetLastError();
}

hipError_t launch_e4m3_decode(const uint8_t* codes, void* out, int kind, int64_t n, hipStream_t st) {
    hipLaunchKernelGGL(e4m3_decode_kernel, dim3(grid_for(n)), dim3(256), 0, st, codes, out, kind, n);
    return hipGetLastError();
}

// ---- cache write -----------------------------------------------------------
// One work-group per (window of 16 consecutive input tokens, KV head).
// Phase 1, lane order (token, 8-dim chunk) with the chunk fastest: coalesced
// 16-byte loads of 8 bf16 of K and of V; K codes go straight to their
// token-major row [blk][g][off][D]; V codes go to an LDS tile [D][16].
// Phase 2, lane order (dim, token) with the token fastest: V elements leave
// the tile one per lane to [blk][g][D][16], so lanes holding consecutive
// slots write consecutive bytes of one cache row and their stores coalesce,
// whatever the slot mapping.  The quantize step is an IEEE fp32 division (the
// scale multiplies code values), so this translation unit must not be built
// with fast-math.
constexpr int kWriteTokens = 16;     // tokens per work-group window
constexpr int kWriteThreads = 256;

template <bool FP8>
__global__ void __launch_bounds__(kWriteThreads) cache_write_kernel(
    const uint16_t* __restrict__ k, const uint16_t* __restrict__ v, int64_t src_stride,
    const int64_t* __restrict__ slot_mapping, int T, int Hkv, int D, uint8_t* __restrict__ k_cache,
    uint8_t* __restrict__ v_cache, float k_scale, float v_scale, int64_t n_slots) {
    using Elem = typename std::conditional<FP8, uint8_t, uint16_t>::type;
    extern __shared__ uint32_t lds_w[];
    Elem* vt = reinterpret_cast<Elem*>(lds_w);   // [D][16] V elements of the window
    __shared__ int64_t s_slot[kWriteTokens];
    const int t0 = blockIdx.x * kWriteTokens, g = blockIdx.y;
    const int chunks = D >> 3;
    // each lane reads its token's slot itself, alongside the K/V loads (the
    // source address does not depend on it), so phase 1 is one round trip
    for (int i = threadIdx.x; i < kWriteTokens * chunks; i += kWriteThreads) {
        const int tw = i / chunks, c = i - tw * chunks, d0 = c << 3;
        const int t = t0 + tw;
        if (t >= T) {
            if (c == 0) s_slot[tw] = -1;
            continue;
        }
        const int64_t src = (int64_t)t * src_stride + (int64_t)g * D + d0;
        int64_t slot = slot_mapping[t];
        if (KVQ_CHECK && slot >= n_slots) {
            check_fail(kCheckSlot);
            slot = -1;
        }
        const u32x4 kw = *reinterpret_cast<const u32x4*>(k + src);
        const u32x4 vw = *reinterpret_cast<const u32x4*>(v + src);
        if (c == 0) s_slot[tw] = slot;
        if (slot < 0) continue;
        const int64_t blk = slot / kBlockSize;   // block_size is validated to be kBlockSize
        const int off = (int)(slot - blk * kBlockSize);
        const int64_t kdst = ((blk * Hkv + g) * kBlockSize + off) * D + d0;   // [blk][g][off][d]
        if constexpr (FP8) {
#pragma clang fp contract(off)
            float kf[8], vf[8];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                kf[2 * j] = bf16_lo(kw[j]) / k_scale;
                kf[2 * j + 1] = bf16_hi(kw[j]) / k_scale;
                vf[2 * j] = bf16_lo(vw[j]) / v_scale;
                vf[2 * j + 1] = bf16_hi(vw[j]) / v_scale;
            }
            u32x2 kc;
            kc[0] = e4m3_encode4(kf[0], kf[1], kf[2], kf[3]);
            kc[1] = e4m3_encode4(kf[4], kf[5], kf[6], kf[7]);
            *reinterpret_cast<u32x2*>(k_cache + kdst) = kc;
#pragma unroll
            for (int j = 0; j < 8; ++j) vt[(d0 + j) * kWriteTokens + tw] = (uint8_t)e4m3_encode(vf[j]);
        } else {
            *reinterpret_cast<u32x4*>(reinterpret_cast<uint16_t*>(k_cache) + kdst) = kw;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                vt[(d0 + 2 * j) * kWriteTokens + tw] = (uint16_t)(vw[j] & 0xFFFFu);
                vt[(d0 + 2 * j + 1) * kWriteTokens + tw] = (uint16_t)(vw[j] >> 16);
            }
        }
    }
    __syncthreads();
    Elem* vc = reinterpret_cast<Elem*>(v_cache);
    for (int i = threadIdx.x; i < kWriteTokens * D; i += kWriteThreads) {
        const int d = i / kWriteTokens, tw = i - d * kWriteTokens;
        const int64_t slot = s_slot[tw];
        if (slot < 0) continue;
        const int64_t blk = slot / kBlockSize;   // block_size is validated to be kBlockSize
        const int off = (int)(slot - blk * kBlockSize);
        vc[((blk * Hkv + g) * (int64_t)D + d) * kBlockSize + off] = vt[d * kWriteTokens + tw];   // [blk][g][d][off]
    }
}

hipError_t launch_cache_write(const void* k, const void* v, int64_t src_stride, const int64_t* slots, int T,
                              int Hkv, int D, void* k_cache, void* v_cache, int bs, int kv_dtype,
                              float k_scale, float v_scale, int64_t n_slots, hipStream_t st) {
    (void)bs;   // validated to be kBlockSize
    const dim3 grid((unsigned)((T + kWriteTokens - 1) / kWriteTokens), (unsigned)Hkv);
    const size_t lds = (size_t)kWriteTokens * D * (kv_dtype == 1 ? 1 : 2);
    if (kv_dtype == 1)
        hipLaunchKernelGGL(cache_write_kernel<true>, grid, dim3(kWriteThreads), lds, st, (const uint16_t*)k,
                           (const uint16_t*)v, src_stride, slots, T, Hkv, D, (uint8_t*)k_cache,
                           (uint8_t*)v_cache, k_scale, v_scale, n_slots);
    else
        hipLaunchKernelGGL(cache_write_kernel<false>, grid, dim3(kWriteThreads), lds, st, (const uint16_t*)k,
                           (const uint16_t*)v, src_stride, slots, T, Hkv, D, (uint8_t*)k_cache,
                           (uint8_t*)v_cache, k_scale, v_scale, n_slots);
    return hipGetLastError();
}

// ---- NVFP4 (block-scaled E2M1) cache write --------------------------------
// The Run 26 video description names the format: a block-scaled 4-bit float
// with FP8 scale factors, 4.5 bits per number.  Per (token, head) row, each
// group of 16 consecutive dims gets one E4M3 block scale:
//   bscale = E4M3(bamax / fp32(6 * gscale)), e = fp32(value(bscale) * gscale),
//   code_i = E2M1(x_i / e)  (all zero when e == 0).
// Region per (block, head): K codes [16][D/2], K scales [16][D/16];
// V codes [D][8] (token 2j in the low nibble), V scales [D/16][16].
// Same windows as the FP8 write.  Phase 1, one lane per (token, group) with
// the token fastest: block scales and codes; K codes and both scale bytes are
// stored directly, V codes go to an LDS tile [D][16].  Phase 2, one lane per
// (dim, token): a V code byte holds the nibbles of slots 2j and 2j+1, so the
// lane of the even slot stores the whole byte when the odd slot's token is in
// the same window (the usual case for a prefill); a nibble whose partner is
// not is merged into its 32-bit word with atomicAnd / atomicOr on its own bits.
__global__ void __launch_bounds__(kWriteThreads) nvfp4_cache_write_kernel(
    const uint16_t* __restrict__ k, const uint16_t* __restrict__ v, int64_t src_stride,
    const int64_t* __restrict__ slot_mapping, int T, int Hkv, int D, uint8_t* __restrict__ k_cache,
    uint8_t* __restrict__ v_cache, float k_gscale, float v_gscale, int64_t n_slots) {
    extern __shared__ uint32_t lds_w[];
    uint8_t* vt = reinterpret_cast<uint8_t*>(lds_w);   // [D][16] V codes of the window, one per byte
    __shared__ int64_t s_slot[kWriteTokens];
    const int t0 = blockIdx.x * kWriteTokens, g = blockIdx.y;
    const int groups = D >> 4;
    const int64_t region = (int64_t)kBlockSize * D / 2 + (int64_t)kBlockSize * D / 16;
    const int64_t codes_bytes = (int64_t)kBlockSize * D / 2;
    for (int i = threadIdx.x; i < kWriteTokens * groups; i += kWriteThreads) {
        const int grp = i / kWriteTokens, tw = i - grp * kWriteTokens;
        const int t = t0 + tw;
        if (t >= T) {
            if (grp == 0) s_slot[tw] = -1;
            continue;
        }
        // the lane reads its token's slot itself, alongside the K/V loads (the
        // source address does not depend on it): one round trip
        const int64_t src = (int64_t)t * src_stride + (int64_t)g * D + grp * 16;
        int64_t slot = slot_mapping[t];
        if (KVQ_CHECK && slot >= n_slots) {
            check_fail(kCheckSlot);
            slot = -1;
        }
        const u32x4 k0 = *reinterpret_cast<const u32x4*>(k + src), k1 = *reinterpret_cast<const u32x4*>(k + src + 8);
        const u32x4 v0 = *reinterpret_cast<const u32x4*>(v + src), v1 = *reinterpret_cast<const u32x4*>(v + src + 8);
        if (grp == 0) s_slot[tw] = slot;
        if (slot < 0) continue;
        const int64_t blk = slot / kBlockSize;
        const int off = (int)(slot - blk * kBlockSize);
        uint32_t codes[16], bcode;
        nvfp4_quantize_group(k0, k1, k_gscale, codes, &bcode);
        uint8_t* kr = k_cache + (blk * Hkv + g) * region;
        u32x2 packed = {0u, 0u};
#pragma unroll
        for (int j = 0; j < 16; ++j) packed[j >> 3] |= codes[j] << (4 * (j & 7));
        *reinterpret_cast<u32x2*>(kr + (int64_t)off * (D / 2) + grp * 8) = packed;
        kr[codes_bytes + (int64_t)off * groups + grp] = (uint8_t)bcode;
        nvfp4_quantize_group(v0, v1, v_gscale, codes, &bcode);
        v_cache[(blk * Hkv + g) * region + codes_bytes + (int64_t)grp * kBlockSize + off] = (uint8_t)bcode;
#pragma unroll
        for (int j = 0; j < 16; ++j) vt[(grp * 16 + j) * kWriteTokens + tw] = (uint8_t)codes[j];
    }
    __syncthreads();
    for (int i = threadIdx.x; i < kWriteTokens * D; i += kWriteThreads) {
        const int d = i / kWriteTokens, tw = i - d * kWriteTokens;
        const int64_t slot = s_slot[tw];
        if (slot < 0) continue;
        const int64_t blk = slot / kBlockSize;
        const int off = (int)(slot - blk * kBlockSize);
        uint8_t* vr = v_cache + (blk * Hkv + g) * region;
        const int64_t byte = (int64_t)d * (kBlockSize / 2) + (off >> 1);
        const uint32_t code = vt[d * kWriteTokens + tw];
        // the token of the other nibble of this byte, if it is in the window
        const int pw = (off & 1) ? tw - 1 : tw + 1;
        const bool paired = pw >= 0 && pw < kWriteTokens && s_slot[pw] == (slot ^ 1);
        if (paired) {
            if ((off & 1) == 0) vr[byte] = (uint8_t)(code | (uint32_t)vt[d * kWriteTokens + pw] << 4);
        } else {
            const unsigned shift = 8u * (unsigned)(byte & 3) + 4u * (unsigned)(off & 1);
            unsigned* word = reinterpret_cast<unsigned*>(vr + (byte & ~(int64_t)3));
            atomicAnd(word, ~(0xFu << shift));
            atomicOr(word, code << shift);
        }
    }
}

hipError_t launch_nvfp4_cache_write(const void* k, const void* v, int64_t src_stride, const int64_t* slots, int T,
                                    int Hkv, int D, void* k_cache, void* v_cache, float k_gscale, float v_gscale,
                                    int64_t n_slots, hipStream_t st) {
    const dim3 grid((unsigned)((T + kWriteTokens - 1) / kWriteTokens), (unsigned)Hkv);
    hipLaunchKernelGGL(nvfp4_cache_write_kernel, grid, dim3(kWriteThreads), (size_t)kWriteTokens * D, st,
                       (const uint16_t*)k, (const uint16_t*)v, src_stride, slots, T, Hkv, D, (uint8_t*)k_cache,
                       (uint8_t*)v_cache, k_gscale, v_gscale, n_slots);
    return hipGetLastError();
}

// ---- block copies for a host-memory tier ---------------------------------------
// A physical block of a K or V cache is one contiguous run of block_bytes
// (all heads).  One work-group per listed block (grid-stride over blocks),
// 16-byte words: gather copies block ids[i] to row i of a dense buffer,
// scatter copies row i back to block ids[i].
__global__ void __launch_bounds__(256) block_copy_kernel(const u32x4* __restrict__ src, u32x4* __restrict__ dst,
                                                         const int32_t* __restrict__ ids, int n,
                                                         int64_t words, int gather) {
    for (int i = blockIdx.x; i < n; i += gridDim.x) {
        const int64_t blk = ids[i];
        if (KVQ_CHECK && blk < 0) {   // (the copy calls take no block count: only the sign is checked)
            if (threadIdx.x == 0) check_fail(kCheckBlockId);
            continue;
        }
        const u32x4* s = src + (gather ? blk : (int64_t)i) * words;
        u32x4* d = dst + (gather ? (int64_t)i : blk) * words;
        for (int64_t w = threadIdx.x; w < words; w += blockDim.x) d[w] = s[w];
    }
}

hipError_t launch_block_copy(const void* src, void* dst, const int32_t* ids, int n, size_t block_bytes, int gather,
                             hipStream_t st) {
    const unsigned grid = (unsigned)(n < 65536 ? n : 65536);
    hipLaunchKernelGGL(block_copy_kernel, dim3(grid), dim3(256), 0, st, (const u32x4*)src, (u32x4*)dst, ids, n,
                       (int64_t)(block_bytes / 16), gather);
    return hipGetLastError();
}

// ---- E2M1 decode utility: out[2i], out[2i+1] = the two codes of byte i times
// the E4M3 value of scale_code, computed as the NVFP4 decode kernel does (f16).
__global__ void __launch_bounds__(256) e2m1_decode_kernel(const uint8_t* __restrict__ codes, uint32_t scale_code,
                                                          f16x2* __restrict__ out, int64_t n) {
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    int64_t stride = (int64_t)gridDim.x * blockDim.x;
    const _Float16 sc = e4m3x2_to_f16(scale_code, false)[0];
    for (; i < n; i += stride) out[i] = e2m1x2_to_f16<0>(codes[i]) * f16x2{sc, sc};
}

hipError_t launch_e2m1_decode(const uint8_t* codes, uint32_t scale_code, void* out, int64_t n, hipStream_t st) {
    hipLaunchKernelGGL(e2m1_decode_kernel, dim3(grid_for(n)), dim3(256), 0, st, codes, scale_code, (f16x2*)out, n);
    return hipGetLastError();
}

unsigned check_flags_cache(bool clear) {
#if KVQ_CHECK
    unsigned v = 0;
    if (hipMemcpyFromSymbol(&v, HIP_SYMBOL(g_check_flags), sizeof(v)) != hipSuccess) return ~0u;
    if (clear) {
        const unsigned z = 0;
        if (hipMemcpyToSymbol(HIP_SYMBOL(g_check_flags), &z, sizeof(z)) != hipSuccess) return ~0u;
    }
    return v;
#else
    (void)clear;
    return 0;
#endif
}

}  // namespace kvq
