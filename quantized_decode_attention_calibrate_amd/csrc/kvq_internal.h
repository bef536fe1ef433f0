// kvq_internal.h -- host-side declarations shared by the libkvq translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace kvq {

// Split-K plan for one decode call (host-computed from host-known bounds only).
struct DecodePlan {
    int split_tokens;  // tokens per work-group, multiple of 64
    int num_splits;    // ceil(max_seq_len / split_tokens)
};

// Largest split the kernels stage block ids for (LDS table of 512 ids).
constexpr int kMaxSplitTokens = 8192;
// Most splits one call may have (the merge keeps one weight per split in LDS).
constexpr int kMaxSplits = 16384;
constexpr int kChunkTokens = 64;   // tokens per wave iteration (4 blocks of 16)
constexpr int kMaxQueryLen = 16;   // queries per sequence of a multi-query decode
// KV cache formats of the decode kernels
// (kFmtFP8QP: FP8 cache with FP8 Q and P on FP8 MFMA)
enum : int { kFmtBF16 = 0, kFmtFP8 = 1, kFmtNVFP4 = 2, kFmtFP8QP = 3 };
constexpr int kBlockSize = 16;

// Device-side checks of the caller's data contract, compiled in only with
// -DKVQ_CHECK=1 (libkvq_check.so): block-table entries in [0, num_blocks),
// sequence lengths in [0, max_seq_len], slots below num_blocks * block_size
// (and block-copy ids >= 0).  A violation sets a bit in the translation
// unit's device flag word and the access is replaced by a safe one (block 0,
// a clamped length, a skipped write).
#ifndef KVQ_CHECK
#define KVQ_CHECK 0
#endif
enum : unsigned { kCheckBlockId = 1u, kCheckSeqLen = 2u, kCheckSlot = 4u };

// Phase trace, compiled in only with -DKVQ_TRACE=1 (libkvq_trace.so): the MFMA
// decode kernel and the merge kernel store s_memrealtime stamps of their
// phases into a device buffer set by trace_set_attn (null: off).  The stamps
// wait for outstanding memory operations first, so a traced call runs a
// little slower; its results are the release build's.
#ifndef KVQ_TRACE
#define KVQ_TRACE 0
#endif
int trace_set_attn(uint64_t* buf, int64_t decode_words, int64_t merge_words);
// Flag words of the kernel translation units: OR of the set bits; clear = zero
// them afterwards.  Synchronous copies (0 when compiled without checks).
unsigned check_flags_attn(bool clear);
unsigned check_flags_cache(bool clear);

struct DecodeArgs {
    const uint16_t* q;           // bf16 [B][q_len][Hq][D]
    const uint8_t* k_cache;      // FP8 or BF16 paged K cache (bytes)
    const uint8_t* v_cache;      // FP8 or BF16 paged V cache (bytes, dim-major blocks)
    const int32_t* block_tables; // [B][max_blocks]
    const int32_t* seq_lens;     // [B]
    float* ws_ml;                // [B][q_len][Hq][S][2] : running max (log2 units), sum of weights
    float* ws_acc;               // [B][q_len][Hq][S][D] : unnormalised weighted sum of V codes
    void* out;                   // [B][q_len][Hq][D]
    int max_blocks;
    int Hq, Hkv, G;
    int split_tokens, num_splits;
    float qk_scale_log2;         // sm_scale * k_scale * log2(e) (* q_scale for kFmtFP8QP)
    float q_scale;               // kFmtFP8QP: Q quantization scale
    float v_scale;               // applied once in the merge
    int out_f32;
    int q_len;                   // queries per sequence (1: single-token decode)
    int window;                  // > 0: each query sees its `window` newest tokens
    // Fused append (k_new != nullptr): sequence b's newest token (position
    // seq_lens[b] - 1) is quantized from bf16 rows k_new / v_new + b * new_stride
    // + g * D and stored at new_slots[b] (< 0: not written) by the work-group
    // that reads it, before it reads it.
    const uint16_t* k_new;
    const uint16_t* v_new;
    int64_t new_stride;
    const int64_t* new_slots;
    float k_scale_w, v_scale_w;  // cache quantization scales of the write (FP8)
    // the caller's bounds (read by the checked build only)
    int num_blocks;
    int max_seq_len;
};

// Workspace: [ml: B*Hq*S*2 f32][acc: B*Hq*S*D f32], the second region starting
// on a 256-byte boundary.
size_t decode_ml_bytes(int B, int Hq, int num_splits);
size_t decode_workspace_bytes(int B, int Hq, int D, int num_splits);
DecodePlan plan_decode(int B, int Hkv, int max_seq_len, int split_tokens_request);

hipError_t launch_amax_bf16(const void* x, int64_t rows, int64_t cols, int64_t stride, float* amax,
                            hipStream_t st);
hipError_t launch_e4m3_encode(const float* y, uint8_t* codes, int64_t n, hipStream_t st);
hipError_t launch_e4m3_decode(const uint8_t* codes, void* out, int kind, int64_t n, hipStream_t st);
// n_slots = num_blocks * block_size (slots at or past it: a contract violation)
hipError_t launch_cache_write(const void* k, const void* v, int64_t src_stride, const int64_t* slots, int T,
                              int Hkv, int D, void* k_cache, void* v_cache, int bs, int kv_dtype,
                              float k_scale, float v_scale, int64_t n_slots, hipStream_t st);
hipError_t launch_nvfp4_cache_write(const void* k, const void* v, int64_t src_stride, const int64_t* slots, int T,
                                    int Hkv, int D, void* k_cache, void* v_cache, float k_gscale, float v_gscale,
                                    int64_t n_slots, hipStream_t st);
hipError_t launch_block_copy(const void* src, void* dst, const int32_t* ids, int n, size_t block_bytes, int gather,
                             hipStream_t st);
hipError_t launch_e2m1_decode(const uint8_t* codes, uint32_t scale_code, void* out, int64_t n, hipStream_t st);
// Column tiles of 16 (query, head) pairs the MFMA kernel uses for G * q_len
// columns at head dim D; 0 if the shape is not supported.
int decode_column_tiles(int G, int q_len, int D);
// impl: 1 = VALU, 2 = MFMA.  B is the grid's z extent.
// fmt: kFmtBF16 / kFmtFP8 / kFmtNVFP4 (NVFP4 has the MFMA family only)
hipError_t launch_decode(const DecodeArgs& a, int B, int D, int fmt, int impl, hipStream_t st);

}  // namespace kvq
