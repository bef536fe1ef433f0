// kvq_cache.hip -- calibration observation (amax), E4M3 codec utilities and
// the paged KV-cache write (quantize + scatter by slot mapping).
//
// The calibration guide for the Radiance R9700 fork (calibrator paragraph)
// defines what is observed (BF16 K/V absolute maxima, combined by maximum)
// and the OCP E4M3 format with maximum 448; its storage paragraph fixes FP8
// at one byte per element.  These kernels are HBM/latency bound: one pass
// over the input, 16-byte loads, no LDS.
#include "kvq_device.h"
#include "kvq_internal.h"

namespace kvq {

// ---- amax ------------------------------------------------------------------
// |bf16| ordered as an unsigned 15-bit magnitude equals the order of the
// values (NaN patterns above Inf), so the running max is an integer max on
// the fp32 bit pattern of the magnitude; one atomicMax per wave.
__global__ void __launch_bounds__(256) amax_bf16_kernel(const uint16_t* __restrict__ x, int64_t rows,
                                                        int64_t cols, int64_t stride,
                                                        uint32_t* __restrict__ amax_bits) {
    uint32_t m = 0;
    const int64_t nthreads = (int64_t)gridDim.x * blockDim.x;
    const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if ((cols & 7) == 0 && (stride & 7) == 0) {
        const int64_t vec_per_row = cols >> 3;
        const int64_t nvec = rows * vec_per_row;
        for (int64_t i = tid; i < nvec; i += nthreads) {
            int64_t r = i / vec_per_row, c = (i - r * vec_per_row) << 3;
            u32x4 w = *reinterpret_cast<const u32x4*>(x + r * stride + c);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                uint32_t lo = w[j] & 0x7FFFu, hi = (w[j] >> 16) & 0x7FFFu;
                m = max(m, max(lo, hi));
            }
        }
    } else {
        const int64_t n = rows * cols;
        for (int64_t i = tid; i < n; i += nthreads) {
            int64_t r = i / cols, c = i - r * cols;
            m = max(m, (uint32_t)(x[r * stride + c] & 0x7FFFu));
        }
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1)
        m = max(m, (uint32_t)__builtin_amdgcn_ds_bpermute((__lane_id() ^ o) << 2, (int)m));
    if (__lane_id() == 0 && m != 0) atomicMax(amax_bits, m << 16);
}

hipError_t launch_amax_bf16(const void* x, int64_t rows, int64_t cols, int64_t stride, float* amax,
                            hipStream_t st) {
    int64_t work = ((cols & 7) == 0 && (stride & 7) == 0) ? rows * (cols >> 3) : rows * cols;
    int64_t blocks = (work + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    if (blocks < 1) blocks = 1;
    hipLaunchKernelGGL(amax_bf16_kernel, dim3((unsigned)blocks), dim3(256), 0, st,
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
// One thread per (token, head, 8-element chunk of D): a 16-byte load of 8 bf16
// for K and for V.  K goes to [blk][g][off][D] (one 8-byte store of codes);
// V goes to [blk][g][D][bs] (8 single-byte stores, stride bs).  The quantize
// step is an IEEE fp32 division (the scale multiplies code values), so this
// translation unit must not be built with fast-math.
template <bool FP8>
__global__ void __launch_bounds__(256) cache_write_kernel(
    const uint16_t* __restrict__ k, const uint16_t* __restrict__ v, int64_t src_stride,
    const int64_t* __restrict__ slot_mapping, int T, int Hkv, int D, uint8_t* __restrict__ k_cache,
    uint8_t* __restrict__ v_cache, int bs, float k_scale, float v_scale) {
    const int chunks = D >> 3;
    const int64_t per_tok = (int64_t)Hkv * chunks;
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= (int64_t)T * per_tok) return;
    const int t = (int)(i / per_tok);
    const int rem = (int)(i - (int64_t)t * per_tok);
    const int g = rem / chunks;
    const int d0 = (rem - g * chunks) << 3;
    const int64_t slot = slot_mapping[t];
    if (slot < 0) return;
    const int64_t blk = slot / bs;
    const int off = (int)(slot - blk * bs);
    const int64_t src = (int64_t)t * src_stride + (int64_t)g * D + d0;
    const u32x4 kw = *reinterpret_cast<const u32x4*>(k + src);
    const u32x4 vw = *reinterpret_cast<const u32x4*>(v + src);
    const int64_t kdst = ((blk * Hkv + g) * bs + off) * D + d0;             // [blk][g][off][d]
    const int64_t vdst = ((blk * Hkv + g) * (int64_t)D + d0) * bs + off;    // [blk][g][d][off]
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
        for (int j = 0; j < 8; ++j) v_cache[vdst + (int64_t)j * bs] = (uint8_t)e4m3_encode(vf[j]);
    } else {
        uint16_t* kc = reinterpret_cast<uint16_t*>(k_cache);
        uint16_t* vc = reinterpret_cast<uint16_t*>(v_cache);
        *reinterpret_cast<u32x4*>(kc + kdst) = kw;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            vc[vdst + (int64_t)(2 * j) * bs] = (uint16_t)(vw[j] & 0xFFFFu);
            vc[vdst + (int64_t)(2 * j + 1) * bs] = (uint16_t)(vw[j] >> 16);
        }
    }
}

hipError_t launch_cache_write(const void* k, const void* v, int64_t src_stride, const int64_t* slots, int T,
                              int Hkv, int D, void* k_cache, void* v_cache, int bs, int kv_dtype,
                              float k_scale, float v_scale, hipStream_t st) {
    const int64_t threads = (int64_t)T * Hkv * (D >> 3);
    const unsigned blocks = (unsigned)((threads + 255) / 256);
    if (kv_dtype == 1)
        hipLaunchKernelGGL(cache_write_kernel<true>, dim3(blocks), dim3(256), 0, st, (const uint16_t*)k,
                           (const uint16_t*)v, src_stride, slots, T, Hkv, D, (uint8_t*)k_cache,
                           (uint8_t*)v_cache, bs, k_scale, v_scale);
    else
        hipLaunchKernelGGL(cache_write_kernel<false>, dim3(blocks), dim3(256), 0, st, (const uint16_t*)k,
                           (const uint16_t*)v, src_stride, slots, T, Hkv, D, (uint8_t*)k_cache,
                           (uint8_t*)v_cache, bs, k_scale, v_scale);
    return hipGetLastError();
}

}  // namespace kvq
