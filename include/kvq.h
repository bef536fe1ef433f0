/*
 * kvq.h -- C ABI of libkvq.so: FP8 (OCP E4M3) and block-scaled 4-bit KV-cache
 * quantization with calibrated per-layer scales, paged KV-cache writes, and
 * single-token split-K paged decode attention that dequantizes inside the
 * kernel, for AMD Instinct MI355X (gfx950).
 *
 * Sources (web pages, cited by title and the part of the page):
 *   [CAL]   "FP8 KV calibration" guide for the Radiance vLLM fork on Radeon AI
 *           PRO R9700: calibrator paragraph (observe BF16 K/V absolute maxima,
 *           combine across ranks, scale = max(amax * 1.05 / 448, 1e-12), OCP
 *           E4M3); storage paragraph (FP8 is one byte per element, half of BF16).
 *   [RUN26] "I Tested NVFP4 vs FP8 KV Cache on Blackwell" video description
 *           (Skildcore Run 26: KV Cache Precision), WHAT YOU'LL LEARN list and
 *           CHAPTERS: every generated token reads the whole KV cache; E4M3 one
 *           byte per number; block-scaled 4-bit float with FP8 scale factors,
 *           4.5 bits per number; chapter "The Missing Fused Dequant Kernel";
 *           "two-level FP32 accumulation".
 *
 * Conventions for every call:
 *   - Pointers named *_dev are device pointers, *_host are host pointers.  The
 *     caller owns every buffer; the library allocates nothing and keeps no
 *     per-call state.
 *   - `hip_stream` is a hipStream_t passed as void* (NULL = default stream).
 *     Device calls are asynchronous: they validate arguments on the host,
 *     enqueue kernels on the stream and return; they never synchronize.
 *   - Return value: KVQ_OK or a negative kvq_status.  Host validation happens
 *     before any HIP call, so an invalid call enqueues nothing.  A failed
 *     launch returns KVQ_EHIP; kvq_last_hip_error() then gives the hipError_t
 *     (per calling thread).  Nothing throws or aborts.
 *   - Data that lives on the device (slot mappings, block tables, sequence
 *     lengths) is the caller's contract: slots < num_blocks * block_size,
 *     block ids < num_blocks, 0 <= seq_lens[b] <= max_seq_len.  The library
 *     cannot check device data without a synchronization and does not.
 *   - All tensors are dense row-major; device pointers to caches, q, out and
 *     k/v sources must be 16-byte aligned and the k/v token stride a multiple
 *     of 8 elements (KVQ_EINVAL otherwise).
 *   - GQA: query head h reads KV head h / (Hq / Hkv).
 *
 * Paged cache layout (num_blocks physical blocks of block_size tokens):
 *   BF16 / FP8 K cache  [num_blocks][Hkv][block_size][D]    (u16 / u8)
 *   BF16 / FP8 V cache  [num_blocks][Hkv][D][block_size]    (u16 / u8, dim-major)
 *   NVFP4 K and V cache [num_blocks][Hkv][kvq_nvfp4_region_bytes(D, bs)] bytes
 *                       (layout inside a region: see the NVFP4 section)
 *   A token's slot is physical_block * block_size + offset.
 */
#ifndef KVQ_H
#define KVQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* 2: multi-query and sliding-window decode, FP8 Q/P variant, fused append,
 *    host-memory block tier
 * 3: kvq_check_flags and the checked build libkvq_check.so
 * 4: kvq_paged_decode_attn_mq_append
 * 5: kvq_nvfp4_cache_bytes_per_block
 * 6: kvq_paged_decode_attn_scratch
 * 7: kvq_trace_set and the phase-trace build libkvq_trace.so */
#define KVQ_ABI_VERSION 7

enum kvq_status {
    KVQ_OK = 0,
    KVQ_EINVAL = -1,        /* bad pointer, size, alignment or argument combination */
    KVQ_EUNSUPPORTED = -2,  /* valid but not implemented here (D, block_size, G) */
    KVQ_EWORKSPACE = -3,    /* workspace smaller than kvq_decode_workspace_bytes() */
    KVQ_EHIP = -4           /* a HIP launch failed; see kvq_last_hip_error() */
};

enum kvq_kv_dtype { KVQ_KV_BF16 = 0, KVQ_KV_FP8_E4M3 = 1 };

/* F32 writes the fp32 epilogue unrounded (same kernels; only the final store
 * differs); BF16 rounds it to nearest even. */
enum kvq_out_dtype { KVQ_OUT_BF16 = 0, KVQ_OUT_F32 = 1 };

/* Decode-attention kernel family (for comparisons; AUTO picks per shape). */
enum kvq_attn_impl { KVQ_IMPL_AUTO = 0, KVQ_IMPL_VALU = 1, KVQ_IMPL_MFMA = 2 };

/* Human-readable text of a kvq_status (static storage). */
const char* kvq_strerror(int status);

/* hipError_t of the last KVQ_EHIP returned on this thread (0 if none). */
int kvq_last_hip_error(void);

/* KVQ_ABI_VERSION of the loaded library. */
int kvq_abi_version(void);

/* ---- checked build -------------------------------------------------------
 * Device data (block tables, slot mappings, sequence lengths, block-copy ids)
 * is the caller's contract and the release library libkvq.so does not check
 * it.  libkvq_check.so is the same library built with device-side checks: a
 * block-table entry outside [0, num_blocks) reads block 0, a sequence length
 * outside [0, max_seq_len] is clamped, a slot at or past
 * num_blocks * block_size (cache writes and the fused append) is skipped,
 * and a negative block-copy id is skipped (the copy calls take no block
 * count); each case sets a bit in a device flag word.  Meant for tests and
 * debugging: results of valid calls are bit-identical to libkvq.so's.
 * kvq_check_flags copies the OR of the bits to *flags_host and, if clear is
 * non-zero, zeroes them.  It is synchronous: call it after the streams that
 * ran the checked calls have finished.  Returns KVQ_EUNSUPPORTED (and 0 in
 * *flags_host) from libkvq.so, KVQ_EINVAL if flags_host is NULL, KVQ_EHIP if
 * the copy fails. */
#define KVQ_CHECK_BLOCK_ID 1u
#define KVQ_CHECK_SEQ_LEN 2u
#define KVQ_CHECK_SLOT 4u
int kvq_check_flags(unsigned* flags_host, int clear);

/* ---- phase trace (libkvq_trace.so) -----------------------------------------
 * libkvq_trace.so is built from the same sources with -DKVQ_TRACE=1: the MFMA
 * decode kernel and the merge kernel also store timestamps of their phases
 * (the 100 MHz real-time counter, s_memrealtime), for attributing a call's
 * time to its parts.  A stamp first waits for the wave's outstanding memory
 * operations, so a traced call runs slightly slower; its results are the
 * release build's.
 * kvq_trace_set points the kernels at buf_dev, a device buffer of
 * decode_words + merge_words uint64 words owned by the caller (NULL: tracing
 * off); it is synchronous and applies to the current device.  Every call
 * overwrites what the previous one stored.  Layout:
 *   decode region, words [0, decode_words): 8 words per wave at
 *     ((x + X * (y + Y * z)) * W + wave) * 8 for work-group (x, y, z) of a
 *     grid (X, Y, Z) = (splits, KV heads, sequences) and W waves per
 *     work-group: stamps at the start, after the sequence length, after the
 *     block-id staging, after the first chunk, at the end of the chunk loop
 *     and at the end; then chunks | split << 20 | KV head << 36 |
 *     sequence << 44; then 1 | XCC id << 8 | HW_ID register << 16;
 *   merge region, words [decode_words, decode_words + merge_words): 4 words
 *     per output row (b * q_len + i) * Hq + h that has two or more splits:
 *     start, after the split weights, end, 1.
 * Waves and rows whose slots fall outside their region store nothing.
 * Returns KVQ_EUNSUPPORTED from libkvq.so and libkvq_check.so, KVQ_EINVAL for
 * negative sizes, KVQ_EHIP if setting the device pointer fails. */
int kvq_trace_set(uint64_t* buf_dev, int64_t decode_words, int64_t merge_words);

/* ---- codec utilities (device) ---------------------------------------------
 * The E4M3 codec used by every kernel, exposed for exhaustive checks.
 * Encode: saturating round-to-nearest-even fp32 -> OCP E4M3 ([CAL]: OCP E4M3,
 * maximum 448): |y| > 448 and +-Inf -> +-448 (0x7E/0xFE), NaN -> 0x7F with
 * the NaN's sign, sign kept on underflow (-tiny -> 0x80).
 * Decode: exact; out_kind 0 = fp32, 1 = fp16, 2 = bf16 (every finite E4M3
 * value is exact in all three), through the conversion the attention kernels
 * use for that type.  codes_dev: n bytes; y_dev / out_dev: n elements. */
int kvq_e4m3_encode_f32(const float* y_dev, uint8_t* codes_dev, int64_t n, void* hip_stream);
int kvq_e4m3_decode(const uint8_t* codes_dev, void* out_dev, int out_kind, int64_t n, void* hip_stream);

/* ---- calibration ---------------------------------------------------------
 * [CAL] calibrator paragraph: the calibrator observes BF16 K/V absolute
 * maxima per layer, combines observations by maximum, and writes
 * scale = max(observed_absolute_max * 1.05 / 448, 1e-12).
 *
 * kvq_amax_bf16: running maximum of |x| over a bf16 matrix of `rows` rows of
 * `cols` elements with row stride `row_stride` elements (e.g. K as
 * [T][Hkv*D]) into *amax_dev (fp32, device).  *amax_dev must be initialised by
 * the caller (0 for a fresh observation); calling it again on more data, or on
 * data from another rank, combines by maximum.  Exact.  A NaN anywhere makes
 * the result NaN (kvq_calibrate then rejects it).  rows == 0 is a no-op. */
int kvq_amax_bf16(const void* x_dev, int64_t rows, int64_t cols, int64_t row_stride,
                  float* amax_dev, void* hip_stream);

/* kvq_calibrate: host only.  scale_host[i] = fp32(max((double)amax_host[i] *
 * 1.05 / 448, 1e-12)), evaluated left to right in fp64 and rounded once.
 * KVQ_EINVAL (scale_host untouched) if any amax is negative, NaN or Inf. */
int kvq_calibrate(const float* amax_host, float* scale_host, int n);

/* ---- cache write ---------------------------------------------------------
 * [CAL] storage paragraph: FP8 stores one byte per K or V element against two
 * for BF16, so an FP8 block is half the size of a BF16 block.
 *
 * Quantize T tokens of K and V and scatter them into the paged caches.
 *   k_dev, v_dev        bf16 [T][Hkv][D]; row t starts at t * src_token_stride
 *                       elements (so K and V may be slices of a fused QKV
 *                       projection output)
 *   slot_mapping_dev    int64 [T]; slot < 0 skips the token
 *   k_cache_dev, v_cache_dev  caches in the layouts above
 *   kv_dtype            KVQ_KV_FP8_E4M3: code = E4M3(fp32(x) / scale) with an
 *                       IEEE fp32 division (the scale multiplies a code value
 *                       to give the real value, [CAL]); KVQ_KV_BF16: bit copy
 *                       (scales ignored)
 *   k_scale, v_scale    per-layer scales from kvq_calibrate (> 0, finite)
 * Bytes of slots not written are left unchanged.  T == 0 is a no-op. */
int kvq_cache_write(const void* k_dev, const void* v_dev, int64_t src_token_stride,
                    const int64_t* slot_mapping_dev, int T, int Hkv, int D,
                    void* k_cache_dev, void* v_cache_dev, int num_blocks, int block_size,
                    int kv_dtype, float k_scale, float v_scale, void* hip_stream);

/* ---- decode attention ----------------------------------------------------
 * [RUN26]: each generated token reads the whole KV cache, so decode is a scan
 * of the cache; the FP8 speed-up needs the dequantization fused into the
 * attention kernel, and accuracy needs fp32 accumulation at both levels.
 *
 * For every sequence b and query head h (KV head g = h / (Hq / Hkv)), with
 * L = seq_lens_dev[b] tokens, token t at physical block
 * block_tables_dev[b * max_blocks_per_seq + t / block_size]:
 *   s_t = sm_scale * sum_d q[b][h][d] * dequant(K[t][g][d])
 *   out[b][h][:] = sum_t exp(s_t - max s) dequant(V[t][g][:]) / sum_t exp(s_t - max s)
 * with dequant = code value * k_scale (v_scale) for FP8 and the bf16 value for
 * BF16; out = 0 when L == 0.  Accumulation is fp32 throughout: per-split
 * online softmax partials (m, l, acc[D]) and an fp32 log-sum-exp merge.
 *   q_dev              bf16 [B][Hq][D]
 *   block_tables_dev   int32 [B][max_blocks_per_seq]; entries past a sequence's
 *                      last block are not read
 *   seq_lens_dev       int32 [B]
 *   sm_scale           softmax scale, finite and > 0 (usually 1/sqrt(D))
 *   max_seq_len        host upper bound of seq_lens (sizes the grid; no
 *                      device-to-host copy happens); must be
 *                      <= max_blocks_per_seq * block_size
 *   out_dev            [B][Hq][D], bf16 or fp32 per out_dtype
 *   workspace_dev      >= kvq_decode_workspace_bytes(...) bytes, 16-B aligned;
 *                      contents on entry irrelevant.  Calls that share a
 *                      workspace must not run concurrently.
 * Launches: the split kernel (each work-group reduces its 4 waves through LDS;
 * a split that holds a whole sequence writes `out` directly) and, when any
 * sequence spans two or more splits, the merge kernel for those sequences.
 * Supported: D in {64, 128, 256}, block_size 16, 1 <= Hq / Hkv <= 16, at most
 * 16384 splits (KVQ_EUNSUPPORTED otherwise). */
size_t kvq_decode_workspace_bytes(int B, int Hq, int Hkv, int D, int max_seq_len, int block_size);

int kvq_paged_decode_attn(const void* q_dev, const void* k_cache_dev, const void* v_cache_dev,
                          int kv_dtype, const int32_t* block_tables_dev, int max_blocks_per_seq,
                          const int32_t* seq_lens_dev, int max_seq_len,
                          int B, int Hq, int Hkv, int D, int block_size, int num_blocks,
                          float k_scale, float v_scale, float sm_scale,
                          void* out_dev, int out_dtype,
                          void* workspace_dev, size_t workspace_bytes, void* hip_stream);

/* As kvq_paged_decode_attn with an explicit kernel family (kvq_attn_impl) and
 * split length in tokens (a positive multiple of 64; 0 = automatic).  Used to
 * compare kernels; results agree within fp32 summation order. */
size_t kvq_decode_workspace_bytes_ex(int B, int Hq, int Hkv, int D, int max_seq_len, int block_size,
                                     int split_tokens);
int kvq_paged_decode_attn_ex(const void* q_dev, const void* k_cache_dev, const void* v_cache_dev,
                             int kv_dtype, const int32_t* block_tables_dev, int max_blocks_per_seq,
                             const int32_t* seq_lens_dev, int max_seq_len,
                             int B, int Hq, int Hkv, int D, int block_size, int num_blocks,
                             float k_scale, float v_scale, float sm_scale,
                             void* out_dev, int out_dtype,
                             void* workspace_dev, size_t workspace_bytes, void* hip_stream,
                             int impl, int split_tokens);

/* ---- decode attention without a workspace, for callers that cannot allocate ----
 * For code that may not call hipMalloc or allocate through a framework: inside
 * HIP graph capture, in a tight serving loop, or under a harness that forbids
 * allocation.  kvq_paged_decode_attn with the same arguments, results and
 * kernels (automatic split plan, MFMA family), except that the split partials
 * go to the library's own scratch: a KVQ_SCRATCH_MAX_BYTES device array that
 * each GPU the library runs on holds until the process ends.  The call
 * allocates nothing.  Its first call on a device looks the array's address up
 * (hipGetSymbolAddress, with that device current; the caller's stream must
 * belong to the current device).
 *   Returns KVQ_EWORKSPACE, before any HIP call, when the call needs more than
 *   KVQ_SCRATCH_MAX_BYTES (kvq_decode_workspace_bytes of the same shape).
 * Every call on one GPU shares that GPU's array and leaves its partials there
 * (no call needs them cleared): calls that overlap on one GPU -- on different
 * streams, or from different threads -- race and must be ordered by the
 * caller. */
#define KVQ_SCRATCH_MAX_BYTES (32u * 1024u * 1024u)
int kvq_paged_decode_attn_scratch(const void* q_dev, const void* k_cache_dev, const void* v_cache_dev,
                                  int kv_dtype, const int32_t* block_tables_dev, int max_blocks_per_seq,
                                  const int32_t* seq_lens_dev, int max_seq_len,
                                  int B, int Hq, int Hkv, int D, int block_size, int num_blocks,
                                  float k_scale, float v_scale, float sm_scale,
                                  void* out_dev, int out_dtype, void* hip_stream);

/* kvq_paged_decode_attn_append: one decode step's cache write and attention
 * in one launch, the same result as kvq_cache_write of each sequence's newest
 * token (T = B) followed by kvq_paged_decode_attn (single query, FP8 or BF16,
 * MFMA family).  It saves the separate write launch, which at one token per
 * sequence is all fixed cost.
 *   k_new_dev, v_new_dev  bf16 [B][Hkv][D]; row b starts at b * new_token_stride
 *                         elements (as kvq_cache_write's source)
 *   slot_mapping_dev      int64 [B]: slot of sequence b's newest token, which
 *                         must be the slot of position seq_lens[b] - 1 in
 *                         block_tables (it is the token the attention reads);
 *                         < 0 writes nothing for b, and neither does a
 *                         sequence with seq_lens[b] == 0 (it has no newest
 *                         token; pass -1)
 *   the rest              as kvq_paged_decode_attn_ex (impl is MFMA)
 * Each token is quantized and stored by the work-group that reads it (the one
 * holding the sequence's last split for that KV head), before it reads it;
 * no other work-group reads that block in the call.  A slot that is not the
 * newest position's leaves the attention of that call undefined (a race with
 * whichever work-group reads it); the bytes written are the same either way.
 * Errors as kvq_cache_write and kvq_paged_decode_attn_ex. */
int kvq_paged_decode_attn_append(const void* k_new_dev, const void* v_new_dev, int64_t new_token_stride,
                                 const int64_t* slot_mapping_dev, const void* q_dev, void* k_cache_dev,
                                 void* v_cache_dev, int kv_dtype, const int32_t* block_tables_dev,
                                 int max_blocks_per_seq, const int32_t* seq_lens_dev, int max_seq_len,
                                 int B, int Hq, int Hkv, int D, int block_size, int num_blocks,
                                 float k_scale, float v_scale, float sm_scale, void* out_dev, int out_dtype,
                                 void* workspace_dev, size_t workspace_bytes, void* hip_stream,
                                 int split_tokens);

/* Split length (tokens) the automatic plan picks for this shape. */
int kvq_decode_plan_split_tokens(int B, int Hkv, int max_seq_len, int block_size);

/* ---- block-scaled 4-bit (NVFP4-style) KV cache -------------------------------
 * [RUN26]: a block-scaled 4-bit float with FP8 scale factors, 4.5 bits per
 * number, 1.8x smaller than FP8.  The pages give the format's name and size
 * only; the recipe here is this library's reading:
 *   - element E2M1 (values 0, 0.5, 1, 1.5, 2, 3, 4, 6 and sign), one E4M3
 *     block scale per 16 consecutive elements along D of a (token, head) row,
 *     and one fp32 global scale per tensor;
 *   - gscale = fp32(max(amax * 1.05 / (6 * 448), 1e-12)) (the [CAL] formula
 *     with the E2M1 * E4M3 range);
 *   - per 16-element group: bscale = E4M3(bamax / fp32(6 * gscale)),
 *     e = fp32(value(bscale) * gscale), code_i = E2M1(x_i / e) (fp32 division,
 *     round to nearest even, saturating at 6), all-zero codes when e == 0;
 *   - value = E2M1(code) * value(bscale) * gscale.
 * Cache region per (block, head), kvq_nvfp4_region_bytes(D, 16) = 9*D bytes:
 *   K: codes [16][D/2] (element 2i in the low nibble), scales [16][D/16];
 *   V: codes [D][8] (token 2j in the low nibble), scales [D/16][16].
 * A V code byte holds two tokens, so writes merge nibbles atomically; bytes of
 * other tokens are preserved. */
int kvq_nvfp4_calibrate(const float* amax_host, float* gscale_host, int n);
size_t kvq_nvfp4_region_bytes(int D, int block_size);

/* Bytes of one physical block of an NVFP4 K (or V) cache, all Hkv heads:
 * Hkv * kvq_nvfp4_region_bytes(D, block_size) (576 * Hkv at D 64, block 16:
 * 4.5 bits per element, [RUN26]).  Host only; 0 if Hkv <= 0 or the region
 * size is 0 (D not a positive multiple of 16, block_size odd or <= 0). */
size_t kvq_nvfp4_cache_bytes_per_block(int Hkv, int D, int block_size);

/* As kvq_cache_write, into NVFP4 caches [num_blocks][Hkv][region] bytes, with
 * the per-tensor global scales k_gscale, v_gscale (> 0, finite). */
int kvq_nvfp4_cache_write(const void* k_dev, const void* v_dev, int64_t src_token_stride,
                          const int64_t* slot_mapping_dev, int T, int Hkv, int D,
                          void* k_cache_dev, void* v_cache_dev, int num_blocks, int block_size,
                          float k_gscale, float v_gscale, void* hip_stream);

/* As kvq_paged_decode_attn over NVFP4 caches (MFMA family; the block scales
 * are applied while converting codes to MFMA operands, the global scales are
 * folded into the softmax exponent and the final division).  Same workspace
 * sizing (kvq_decode_workspace_bytes[_ex]). */
int kvq_nvfp4_paged_decode_attn(const void* q_dev, const void* k_cache_dev, const void* v_cache_dev,
                                const int32_t* block_tables_dev, int max_blocks_per_seq,
                                const int32_t* seq_lens_dev, int max_seq_len,
                                int B, int Hq, int Hkv, int D, int block_size, int num_blocks,
                                float k_gscale, float v_gscale, float sm_scale,
                                void* out_dev, int out_dtype,
                                void* workspace_dev, size_t workspace_bytes, void* hip_stream);
int kvq_nvfp4_paged_decode_attn_ex(const void* q_dev, const void* k_cache_dev, const void* v_cache_dev,
                                   const int32_t* block_tables_dev, int max_blocks_per_seq,
                                   const int32_t* seq_lens_dev, int max_seq_len,
                                   int B, int Hq, int Hkv, int D, int block_size, int num_blocks,
                                   float k_gscale, float v_gscale, float sm_scale,
                                   void* out_dev, int out_dtype,
                                   void* workspace_dev, size_t workspace_bytes, void* hip_stream,
                                   int split_tokens);

/* The NVFP4 decode step in one launch: kvq_nvfp4_cache_write of each
 * sequence's newest token followed by kvq_nvfp4_paged_decode_attn, with the
 * arguments and preconditions of kvq_paged_decode_attn_append (k_gscale /
 * v_gscale in place of the FP8 scales).  The token's V code bytes also hold
 * the nibble of the other slot of its pair, which is kept. */
int kvq_nvfp4_paged_decode_attn_append(const void* k_new_dev, const void* v_new_dev, int64_t new_token_stride,
                                       const int64_t* slot_mapping_dev, const void* q_dev, void* k_cache_dev,
                                       void* v_cache_dev, const int32_t* block_tables_dev,
                                       int max_blocks_per_seq, const int32_t* seq_lens_dev, int max_seq_len,
                                       int B, int Hq, int Hkv, int D, int block_size, int num_blocks,
                                       float k_gscale, float v_gscale, float sm_scale,
                                       void* out_dev, int out_dtype,
                                       void* workspace_dev, size_t workspace_bytes, void* hip_stream,
                                       int split_tokens);

/* ---- multi-query and sliding-window decode ---------------------------------
 * The verification step of speculative decoding (multi-token prediction and
 * draft models on the Radiance spec-decode campaign page, the DFlash and MTP
 * lanes of the dual-R9700 page): the q_len newest tokens of every sequence
 * attend at once over the same paged cache, each causally.  All q_len tokens
 * are already in the cache (written by kvq_cache_write / kvq_nvfp4_cache_write)
 * and counted in seq_lens.  Query i of sequence b is the token at position
 * seq_lens[b] - q_len + i and attends to tokens 0 .. seq_lens[b] - q_len + i:
 *   out[b][i][h][:] = the kvq_paged_decode_attn result of q[b][i][h] over the
 *                     first seq_lens[b] - q_len + 1 + i tokens (0 if none).
 * window > 0 restricts every query to its `window` newest tokens (sliding-
 * window attention, the layer type the dual-R9700 page's SWA section says
 * vLLM's ROCm custom paged path cannot serve): query i at position p sees
 * tokens max(0, p - window + 1) .. p.  Splits start at the window, so the
 * cost follows the window, not the sequence; block-table entries of blocks
 * wholly before the first query's window are never read (they may be stale
 * or freed).  window = 0 is full causal attention.
 * The cache is read once for all q_len queries: the G * q_len (query, head)
 * pairs of a KV head share each K/V load as MFMA columns.
 *   q_dev      bf16 [B][q_len][Hq][D]      out_dev  [B][q_len][Hq][D]
 *   workspace  >= kvq_decode_workspace_bytes_mq(...) bytes for the same
 *              q_len and window (same rules as kvq_paged_decode_attn's)
 * Other arguments and errors as kvq_paged_decode_attn[_ex] (MFMA family only).
 * Supported: 1 <= q_len <= 16 and G * q_len <= 64 at D 64, <= 32 at D 128,
 * <= 16 at D 256 (KVQ_EUNSUPPORTED otherwise), window >= 0; q_len = 1 with
 * window = 0 is the single-token decode. */
size_t kvq_decode_workspace_bytes_mq(int B, int q_len, int window, int Hq, int Hkv, int D, int max_seq_len,
                                     int block_size, int split_tokens);
int kvq_paged_decode_attn_mq(const void* q_dev, int q_len, int window, const void* k_cache_dev,
                             const void* v_cache_dev, int kv_dtype, const int32_t* block_tables_dev, int max_blocks_per_seq,
                             const int32_t* seq_lens_dev, int max_seq_len,
                             int B, int Hq, int Hkv, int D, int block_size, int num_blocks,
                             float k_scale, float v_scale, float sm_scale,
                             void* out_dev, int out_dtype,
                             void* workspace_dev, size_t workspace_bytes, void* hip_stream,
                             int split_tokens);
int kvq_nvfp4_paged_decode_attn_mq(const void* q_dev, int q_len, int window, const void* k_cache_dev,
                                   const void* v_cache_dev, const int32_t* block_tables_dev,
                                   int max_blocks_per_seq, const int32_t* seq_lens_dev, int max_seq_len,
                                   int B, int Hq, int Hkv, int D, int block_size, int num_blocks,
                                   float k_gscale, float v_gscale, float sm_scale,
                                   void* out_dev, int out_dtype,
                                   void* workspace_dev, size_t workspace_bytes, void* hip_stream,
                                   int split_tokens);
/* kvq_paged_decode_attn_mq_append: the speculative-verification step in one
 * launch, the same result as kvq_cache_write of the q_len new tokens of every
 * sequence followed by kvq_paged_decode_attn_mq (FP8 or BF16, MFMA family):
 * the drafted tokens' K/V go into the cache and all q_len of them are
 * verified against it.
 *   k_new_dev, v_new_dev  bf16 rows [B * q_len][Hkv][D]; new token i of
 *                         sequence b (position seq_lens[b] - q_len + i) is row
 *                         b * q_len + i, starting at (b * q_len + i) *
 *                         new_token_stride elements; 16-B aligned
 *   slot_mapping_dev      int64 [B][q_len]: slot of new token i of sequence
 *                         b, which must be the slot of its position in
 *                         block_tables; < 0 writes nothing for that token, and
 *                         neither does a position below 0 (a sequence shorter
 *                         than q_len)
 *   q_dev                 bf16 [B][q_len][Hq][D], the new tokens' queries
 *   the rest              as kvq_paged_decode_attn_mq (window >= 0), with its
 *                         workspace (kvq_decode_workspace_bytes_mq)
 * Each new token is quantized and stored by the work-group and wave that
 * read its block (the token's 64-token chunk of its split; q_len <= 16, so a
 * wave writes tokens of one chunk only, its last), before that wave reads it.
 * The new tokens' blocks must not be read by other sequences in the call
 * (the sequence's own last blocks).  Errors as kvq_cache_write and
 * kvq_paged_decode_attn_mq. */
int kvq_paged_decode_attn_mq_append(const void* k_new_dev, const void* v_new_dev, int64_t new_token_stride,
                                    const int64_t* slot_mapping_dev, const void* q_dev, int q_len, int window,
                                    void* k_cache_dev, void* v_cache_dev, int kv_dtype,
                                    const int32_t* block_tables_dev, int max_blocks_per_seq,
                                    const int32_t* seq_lens_dev, int max_seq_len, int B, int Hq, int Hkv, int D,
                                    int block_size, int num_blocks, float k_scale, float v_scale, float sm_scale,
                                    void* out_dev, int out_dtype, void* workspace_dev, size_t workspace_bytes,
                                    void* hip_stream, int split_tokens);

/* ---- FP8 Q and P variant -------------------------------------------------------
 * The Radiance FP8 guide observes Q maxima alongside K and V and names a
 * prob_scale on other attention paths.  This variant runs both products on
 * FP8 MFMA (v_mfma_f32_16x16x32_fp8_fp8) straight from the cache bytes, over an
 * FP8 cache, with the queries, causality and window of
 * kvq_paged_decode_attn_mq:
 *   qc_d = E4M3(fp32(q_d) / q_scale)    (q_scale from kvq_calibrate on Q maxima)
 *   x_t  = c * sum_d value(qc_d) * value(kc_td),
 *          c = fp32(sm_scale * q_scale * k_scale * log2 e) rounded once from fp64
 *   R    = ceil(max_t x_t), an integer: a power-of-two softmax reference
 *   pc_t = E4M3(448 * 2^(x_t - R))      (prob_scale 1/448: P in (0, 448])
 *   out  = v_scale * sum_t value(pc_t) value(vc_t) / sum_t value(pc_t)
 * The kernel keeps an integer running reference, so every rescale is an
 * exact power of two and a weight's code does not depend on the split or
 * chunk order, except for E4M3 subnormal weights, which round more finely
 * against an earlier, lower reference.  The FP8 MFMA dot step is not exact:
 * it sums each group of 8 products aligned to the group's largest exponent
 * sum 2^E and drops what lies below 2^(E-13), so scores, PV sums and the
 * weight sum carry a small bounded error and a weight near an E4M3 midpoint
 * may take either code.  The result lies within a band around the definition
 * derived from that model (median width ~2.5e-3 for unit-scale V).  3-bit Q
 * and P move every weight by a few per cent: on N(0,1) data the output is
 * ~8e-2 (relative L2) away from kvq_paged_decode_attn_mq's.  Same workspace
 * as kvq_decode_workspace_bytes_mq; errors as kvq_paged_decode_attn_mq plus
 * KVQ_EINVAL for a bad q_scale. */
int kvq_paged_decode_attn_fp8qp(const void* q_dev, int q_len, int window, const void* k_cache_dev,
                                const void* v_cache_dev, const int32_t* block_tables_dev, int max_blocks_per_seq,
                                const int32_t* seq_lens_dev, int max_seq_len,
                                int B, int Hq, int Hkv, int D, int block_size, int num_blocks,
                                float q_scale, float k_scale, float v_scale, float sm_scale,
                                void* out_dev, int out_dtype,
                                void* workspace_dev, size_t workspace_bytes, void* hip_stream,
                                int split_tokens);

/* ---- block copies for a host-memory KV tier --------------------------------
 * The Radiance FP8 guide's operator notes account offloaded KV by block bytes
 * (FP8 blocks are half the BF16 bytes) and the dual-R9700 page runs a 10 GiB
 * CPU KV tier.  A physical block of a K or V cache written by this library is
 * one contiguous run of kvq_cache_block_bytes bytes (all KV heads), so a tier
 * moves whole blocks by id.
 *   kv_format          KVQ_KV_BF16, KVQ_KV_FP8_E4M3, or 2 for NVFP4
 *   block_ids_dev      int32 [n] physical block ids (< the cache's num_blocks:
 *                      a device-side contract like the block tables)
 * kvq_gather_blocks: dst[i] = block ids[i] (dst: n * block_bytes device
 * bytes); kvq_scatter_blocks: block ids[i] = src[i].
 * kvq_offload_blocks: K blocks then V blocks of the listed ids, gathered into
 * staging_dev (2 * n * block_bytes device bytes, 16-B aligned, owned by the
 * caller) and copied with one hipMemcpyAsync to host_dst (2 * n * block_bytes,
 * pinned host memory for an asynchronous copy); kvq_restore_blocks is the
 * reverse into the listed (possibly different) block ids.  block_bytes must
 * be a positive multiple of 16; n = 0 does nothing.  All calls are
 * asynchronous on hip_stream; host_dst is complete when the stream is. */
size_t kvq_cache_block_bytes(int kv_format, int Hkv, int D, int block_size);
int kvq_gather_blocks(const void* cache_dev, size_t block_bytes, const int32_t* block_ids_dev, int n,
                      void* dst_dev, void* hip_stream);
int kvq_scatter_blocks(const void* src_dev, size_t block_bytes, const int32_t* block_ids_dev, int n,
                       void* cache_dev, void* hip_stream);
int kvq_offload_blocks(const void* k_cache_dev, const void* v_cache_dev, size_t block_bytes,
                       const int32_t* block_ids_dev, int n, void* staging_dev, void* host_dst, void* hip_stream);
int kvq_restore_blocks(const void* host_src, void* staging_dev, size_t block_bytes, const int32_t* block_ids_dev,
                       int n, void* k_cache_dev, void* v_cache_dev, void* hip_stream);

/* E2M1 codec utility: byte i of codes_dev holds two codes (low nibble first);
 * out_dev[2i], out_dev[2i+1] = value(code) * value(scale_code) as f16, where
 * scale_code is an E4M3 block-scale code -- computed exactly as the NVFP4
 * decode kernel builds its operands.  out_dev: 2 * n_bytes f16, 4-byte aligned. */
int kvq_e2m1_decode(const uint8_t* codes_dev, uint8_t scale_code, void* out_dev, int64_t n_bytes,
                    void* hip_stream);

#ifdef __cplusplus
}
#endif
#endif /* KVQ_H */
