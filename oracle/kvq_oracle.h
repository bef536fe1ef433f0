/*
 * kvq_oracle.h -- plain, slow, obviously-correct CPU definition of the FP8 /
 * 4-bit KV-cache quantization and paged decode-attention path.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, includes
 * or calls this code; only the tests, the smoke check and the CPU-baseline leg
 * of the benchmark do.  It shares no source with the GPU path.
 *
 * Every routine is written as the definition of its result: fp64 arithmetic
 * except where a step is defined to happen in fp32 (the quantize division and
 * the NVFP4 scale products), brute-force nearest-value search for the codecs,
 * and a direct loop over logical tokens for attention.  No blocking, no
 * fusion, no reordering.
 *
 * Sources (web pages; cited by title and the part of the page):
 *   [CAL]  "FP8 KV calibration" operator guide for the Radiance vLLM fork on
 *          Radeon AI PRO R9700 (thetechpanda.github.io, FP8-KV-CALIBRATION):
 *          the calibrator paragraph (per-layer scale formula, OCP E4M3,
 *          maximum 448, 5% headroom, 1e-12 floor, combine across ranks) and
 *          the storage paragraph (FP8 is one byte per element, half of BF16).
 *   [RUN26] "I Tested NVFP4 vs FP8 KV Cache on Blackwell" video description
 *          (Skildcore Run 26: KV Cache Precision), "WHAT YOU'LL LEARN" list:
 *          24,576 B/token in BF16; E4M3 one byte per number; block-scaled
 *          4-bit float with FP8 scale factors at 4.5 bits per number; every
 *          decode token reads the whole cache; chapter "The Missing Fused
 *          Dequant Kernel"; "two-level FP32 accumulation".
 *
 * Readings where the pages are silent (the OCP E4M3 / E2M1 bit layouts, the
 * cache layout, the NVFP4 global-scale formula, block axis and nibble order)
 * are stated at each function.
 */
#ifndef KVQ_ORACLE_H
#define KVQ_ORACLE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- codecs ------------------------------------------------------------ */

/* OCP E4M3 value of a code ([CAL] calibrator paragraph names OCP E4M3 with
 * maximum 448).  Layout (OCP 8-bit FP spec): 1 sign, 4 exponent (bias 7),
 * 3 mantissa bits; exponent 0 is subnormal; S.1111.111 is NaN; no Inf. */
double kvqo_e4m3_value(uint8_t code);

/* Saturating round-to-nearest-even fp32 -> E4M3 by brute-force search over
 * the 127 non-negative finite codes; ties go to the even code; |y| > 448 and
 * +-Inf saturate to +-448; NaN -> 0x7F with the NaN's sign; the sign of y is
 * kept, so negative values that round to zero give 0x80. */
uint8_t kvqo_e4m3_encode(float y);

/* kvqo_e4m3_encode over an array. */
void kvqo_e4m3_encode_array(const float* y, uint8_t* codes, int64_t n);

/* bf16 bit pattern -> fp32 (exact). */
float kvqo_bf16_to_float(uint16_t bits);

/* Quantize one bf16 element with a per-layer scale: the scale multiplies the
 * code value to give the real value ([CAL] scale formula), so quantizing
 * divides: y = fp32(x) / scale in IEEE fp32 (one rounding), then E4M3. */
uint8_t kvqo_e4m3_quantize(uint16_t x_bf16, float scale);

/* E2M1 value of a 4-bit code: bit 3 sign, 2 exponent bits (bias 1), 1
 * mantissa bit: {0, 0.5, 1, 1.5, 2, 3, 4, 6}. */
double kvqo_e2m1_value(uint8_t nibble);

/* Saturating RNE fp32 -> E2M1 by brute force over the 8 non-negative values,
 * ties to the even code, |y| > 6 and Inf -> 6, NaN -> 6 with its sign. */
uint8_t kvqo_e2m1_encode(float y);

/* ---- calibration ------------------------------------------------------- */

/* [CAL] calibrator paragraph: scale = max(amax * 1.05 / 448, 1e-12), per
 * layer.  Evaluated left to right in fp64, rounded once to fp32.  Returns 0,
 * or -1 (and leaves scale[i] untouched) if any amax is negative, NaN or Inf. */
int kvqo_calibrate(const float* amax, float* scale, int n);

/* Max |x| over a bf16 matrix of `rows` rows of `cols` elements, row stride
 * `row_stride` elements.  Exact.  Any NaN makes the result NaN. */
float kvqo_amax_bf16(const uint16_t* x, int64_t rows, int64_t cols, int64_t row_stride);

/* NVFP4 global scale (reading of [RUN26] "block-scaled 4-bit float with FP8
 * scale factors"; the pages print no formula): the [CAL] formula with the
 * largest representable magnitude 6 * 448 = 2688 (E2M1 max times E4M3 max):
 * gscale = fp32(max(amax * 1.05 / 2688, 1e-12)).  Same error rule. */
int kvqo_nvfp4_calibrate(const float* amax, float* gscale, int n);

/* ---- paged cache layout -------------------------------------------------
 * A cache is num_blocks physical blocks; each block holds block_size tokens
 * of Hkv heads.  Element (token t of a sequence, head g, dim d) with slot
 * s = phys_block * block_size + off:
 *   K cache (FP8 u8 or BF16 u16):  [num_blocks][Hkv][block_size][D]
 *   V cache (FP8 u8 or BF16 u16):  [num_blocks][Hkv][D][block_size]
 * (V is stored dim-major inside a block.)
 * NVFP4 cache region per (block, head), bytes:
 *   K: codes [block_size][D/2] (element 2i low nibble, 2i+1 high nibble)
 *      then block scales [block_size][D/16] (E4M3 codes)
 *   V: codes [D][block_size/2] (token 2j low nibble, 2j+1 high nibble)
 *      then block scales [D/16][block_size] (group-major: one dim group's
 *      scales for all tokens of the block are contiguous)
 *   region bytes = block_size*D/2 + block_size*D/16. */
int64_t kvqo_nvfp4_region_bytes(int D, int block_size);

/* Write T tokens of K and V (bf16, [T][Hkv][D], token stride `src_stride`
 * elements) into the caches at slot_mapping[t]; slot < 0 skips the token.
 * kv_dtype 0 = BF16 (bit copy, scales unused), 1 = FP8 E4M3 with the given
 * per-layer scales.  Bytes not addressed are left unchanged.  Tokens are
 * written in order; when one slot appears several times the last write
 * stays.  `nthreads` > 1 shares the tokens out by slot pair (slot / 2), so
 * every write to a slot happens in one thread in token order and the bytes
 * do not depend on it. */
void kvqo_cache_write(const uint16_t* k, const uint16_t* v, int64_t src_stride,
                      const int64_t* slot_mapping, int T, int Hkv, int D,
                      void* k_cache, void* v_cache, int block_size, int kv_dtype,
                      float k_scale, float v_scale, int nthreads);

/* NVFP4 write.  For each (token, head) row and each group of 16 consecutive
 * dims: bamax = max |x| (fp32); bscale = E4M3(bamax / fp32(6 * gscale));
 * e = fp32(value(bscale) * gscale); codes = E2M1(x / e) (fp32), or all zero
 * when e == 0.  Order and threads as kvqo_cache_write (a V code byte holds
 * the nibbles of a slot pair). */
void kvqo_nvfp4_cache_write(const uint16_t* k, const uint16_t* v, int64_t src_stride,
                            const int64_t* slot_mapping, int T, int Hkv, int D,
                            uint8_t* k_cache, uint8_t* v_cache, int block_size,
                            float k_gscale, float v_gscale, int nthreads);

/* Dequantized value of element (slot, head g, dim d) of an NVFP4 K or V cache. */
double kvqo_nvfp4_k_value(const uint8_t* k_cache, int64_t slot, int g, int d,
                          int Hkv, int D, int block_size, float k_gscale);
double kvqo_nvfp4_v_value(const uint8_t* v_cache, int64_t slot, int g, int d,
                          int Hkv, int D, int block_size, float v_gscale);

/* ---- attention ----------------------------------------------------------
 * Single-token decode attention over a paged cache ([RUN26]: every generated
 * token reads the whole cache).  For sequence b, query head h (KV head
 * g = h / (Hq/Hkv)), L = seq_lens[b] tokens, token t at physical block
 * block_tables[b*max_blocks + t/block_size], offset t % block_size:
 *   k_t, v_t = dequantized cache values (fp64)
 *   s_t = sm_scale * sum_d q[d] * k_t[d]
 *   out = sum_t exp(s_t - max s) v_t / sum_t exp(s_t - max s)
 * and out = 0 when L == 0.  q is bf16 [B][Hq][D]; out is fp64 [B][Hq][D].
 * kv_dtype 0 = BF16 cache, 1 = FP8 cache (scales applied), 2 = NVFP4 cache
 * (k_scale / v_scale are the global scales).  `nthreads` > 1 splits the
 * independent (b, h) units over threads; results do not depend on it. */
void kvqo_decode_attn(const uint16_t* q, const void* k_cache, const void* v_cache,
                      int kv_dtype, const int32_t* block_tables, int max_blocks,
                      const int32_t* seq_lens, int B, int Hq, int Hkv, int D,
                      int block_size, float k_scale, float v_scale, float sm_scale,
                      double* out, int nthreads);

/* Multi-query decode (the verification step of speculative decoding): the
 * q_len newest tokens of each sequence, all already in the cache, attend at
 * once, each causally.  q is bf16 [B][q_len][Hq][D]; query i of sequence b
 * is the token at position p = seq_lens[b] - q_len + i and attends to tokens
 * 0 .. p, or with a sliding window W = window > 0 to tokens
 * max(0, p - W + 1) .. p (out = 0 if there are none).  out is fp64
 * [B][q_len][Hq][D].  q_len = 1, window = 0 is kvqo_decode_attn. */
void kvqo_decode_attn_mq(const uint16_t* q, int q_len, int window, const void* k_cache, const void* v_cache,
                         int kv_dtype, const int32_t* block_tables, int max_blocks,
                         const int32_t* seq_lens, int B, int Hq, int Hkv, int D,
                         int block_size, float k_scale, float v_scale, float sm_scale,
                         double* out, int nthreads);

/* FP8 Q and P variant over an FP8 cache (a reading of the Radiance FP8
 * guide's Q maxima and prob_scale): same queries, causality and window as
 * kvqo_decode_attn_mq, with
 *   qc_d  = E4M3(fp32(q_d) / q_scale)                     (kvqo_e4m3_quantize)
 *   x_t   = c * sum_d value(qc_d) * value(kc_td),  c = fp32(sm_scale * q_scale
 *           * k_scale * log2 e) rounded once from fp64
 *   R     = ceil(max_t x_t)          (an integer: a power-of-two reference)
 *   pc_t  = E4M3(fp32(448 * 2^(x_t - R)))                  (P in (0, 448])
 *   out   = v_scale * sum_t value(pc_t) value(vc_t) / sum_t value(pc_t)
 * in fp64.  The power-of-two reference makes the P codes independent of how
 * a kernel orders or splits the tokens (rescaling by 2^k commutes with E4M3
 * rounding in the normal range). */
void kvqo_decode_attn_fp8qp(const uint16_t* q, int q_len, int window, const uint8_t* k_cache,
                            const uint8_t* v_cache, const int32_t* block_tables, int max_blocks,
                            const int32_t* seq_lens, int B, int Hq, int Hkv, int D, int block_size,
                            float q_scale, float k_scale, float v_scale, float sm_scale, double* out,
                            int nthreads);

/* Per-element tolerance of kvqo_decode_attn_fp8qp ([B][q_len][Hq][D], v_scale
 * applied), derived from the definition for any implementation that meets
 * three stated assumptions (the pages give no accuracy for this variant, and
 * the matrix-core ISA does not state the rounding inside its FP8 dot steps,
 * so eps is an assumption, not a measured property):
 *   (A1) each score sum_d value(qc_d) value(kc_td) is computed within
 *        eps * sum_d |value(qc_d) value(kc_td)|; the fp32 scale-and-shift step
 *        and exp2 add at most 2^-20 (2 + |x_t| + |x_t - R|) to x_t;
 *   (A2) sum_t p_t value(vc_td) and sum_t p_t over the weights p_t it used
 *        are computed within eps times the sum of the terms' magnitudes;
 *   (A3) each weight is value(E4M3(fp32(448 * 2^(x'_t - r)))) * 2^(r - R')
 *        for its computed score x'_t and some integer reference r with
 *        x'_t <= r <= R' = ceil(max_t x'_t): references are powers of two and
 *        may grow while the tokens are visited (one pass, splits, merges).
 * Then, in the definition's frame R, each weight differs from value(pc_t) by
 * at most delta_t: where 448 * 2^(x_t - R) * 2^(-dx_t) >= 2^-5 the argument is
 * normal in every such frame (R' <= R + 1), rounding commutes with the
 * rescale and delta_t is the distance to the codes of the extreme arguments
 * 448 * 2^(x_t - R +- dx_t); below that, delta_t bounds rounding on a grid up
 * to twice as coarse (half its spacing, plus the definition's own rounding).  With W = sum w_t, DW = sum delta_t and o the
 * definition's output in code units:
 *   tol = v_scale * ( (sum_t delta_t |v_t - o| + eps (sum_t (w_t + delta_t)
 *         |v_t| + |o| (W + DW))) / ((W - DW)(1 - eps)) + 2^-20 |o| ),
 * or +Inf when W <= DW or some dx_t >= 1/2.  n_open counts tokens in the
 * normal range whose code the score bound leaves open.  w_out / delta_out
 * (NULL to skip): [B][q_len][Hq][max seq_len] receive w_t and delta_t. */
void kvqo_decode_attn_fp8qp_tol(const uint16_t* q, int q_len, int window, const uint8_t* k_cache,
                                const uint8_t* v_cache, const int32_t* block_tables, int max_blocks,
                                const int32_t* seq_lens, int B, int Hq, int Hkv, int D, int block_size,
                                float q_scale, float k_scale, float v_scale, float sm_scale, double eps,
                                double* tol, int64_t* n_open, double* w_out, double* delta_out);

/* Same as kvqo_decode_attn, for a chosen subset of (b, h) units:
 * units[2*i] = b, units[2*i+1] = h; out is [n_units][D]. */
void kvqo_decode_attn_units(const uint16_t* q, const void* k_cache, const void* v_cache,
                            int kv_dtype, const int32_t* block_tables, int max_blocks,
                            const int32_t* seq_lens, int B, int Hq, int Hkv, int D,
                            int block_size, float k_scale, float v_scale, float sm_scale,
                            const int32_t* units, int n_units, double* out, int nthreads);

/* Reconstruction cosine similarity of n bf16 values against their FP8
 * round trip value(E4M3(x / scale)) * scale, in fp64. */
double kvqo_fp8_cos_sim(const uint16_t* x, int64_t n, float scale);

/* ---- block copies for a host-memory KV tier ------------------------------
 * The Radiance FP8 guide's operator notes count FP8 blocks as half the BF16
 * bytes for host offload, and the dual-R9700 page runs a 10 GiB CPU KV tier.
 * A physical block of a K (or V) cache is one contiguous run of
 * kvqo_block_bytes bytes (all heads): Hkv * bs * D * 2 (BF16), * 1 (FP8),
 * Hkv * (bs * D / 2 + bs * D / 16) (NVFP4). */
size_t kvqo_block_bytes(int kv_dtype, int Hkv, int D, int block_size);
/* dst[i] = block ids[i] of cache, i < n (blocks of block_bytes bytes). */
void kvqo_gather_blocks(const uint8_t* cache, size_t block_bytes, const int32_t* ids, int n, uint8_t* dst);
/* block ids[i] of cache = src[i]. */
void kvqo_scatter_blocks(const uint8_t* src, size_t block_bytes, const int32_t* ids, int n, uint8_t* cache);

#ifdef __cplusplus
}
#endif
#endif
