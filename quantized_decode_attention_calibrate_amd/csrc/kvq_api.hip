// kvq_api.hip -- the C ABI of libkvq.so (declared in include/kvq.h).
//
// Every entry point validates its host arguments before touching HIP, so an
// invalid call enqueues nothing and returns a status; device work is enqueued
// asynchronously on the caller's stream.  The library allocates nothing.
#include <math.h>
#include <stdint.h>

#include <mutex>

#include "kvq.h"
#include "kvq_internal.h"

namespace kvq {

// Work-groups one decode launch aims for: one per CU on MI355X's 256 CUs.
// Each wave keeps two 64-token chunks in flight, so 4 waves per CU cover HBM
// latency, and fewer, longer splits keep the cross-split merge cheap (measured
// on gfx950: 16-32 splits per sequence beat 64-128 at 65k-131k tokens).
constexpr int kTargetWorkGroups = 256;
constexpr int kMinSplitTokens = 512;
// When the (sequence, KV head) units alone already fill the chip, splits
// only balance the tail of a ragged batch: 4,096 tokens measured best on a
// 64-sequence batch of 1k-131k tokens (FP8 523 -> 516 us, BF16 1,035 -> 1,005
// us against 8,192), while fewer, longer splits stay best for a few long
// sequences (4 x 126,976: 7,936 tokens).
constexpr int kManyUnitSplitTokens = 4096;

static size_t pad256(size_t n) { return (n + 255) / 256 * 256; }

size_t decode_ml_bytes(int B, int Hq, int num_splits) {
    return pad256((size_t)B * Hq * num_splits * 2 * sizeof(float));
}

size_t decode_workspace_bytes(int B, int Hq, int D, int num_splits) {
    return decode_ml_bytes(B, Hq, num_splits) + (size_t)B * Hq * num_splits * (size_t)D * sizeof(float);
}

DecodePlan plan_decode(int B, int Hkv, int max_seq_len, int split_tokens_request) {
    DecodePlan p;
    int split = split_tokens_request;
    if (split <= 0) {
        const int64_t units = (int64_t)(B > 0 ? B : 1) * (Hkv > 0 ? Hkv : 1);
        int64_t per_unit = (kTargetWorkGroups + units - 1) / units;
        if (per_unit < 1) per_unit = 1;
        int64_t s = ((int64_t)max_seq_len + per_unit - 1) / per_unit;
        s = (s + kChunkTokens - 1) / kChunkTokens * kChunkTokens;
        if (s < kMinSplitTokens) s = kMinSplitTokens;
        if (s > kMaxSplitTokens) s = kMaxSplitTokens;
        if (units >= kTargetWorkGroups && s > kManyUnitSplitTokens) s = kManyUnitSplitTokens;
        split = (int)s;
    }
    p.split_tokens = split;
    int S = (max_seq_len + split - 1) / split;
    p.num_splits = S < 1 ? 1 : S;
    return p;
}

}  // namespace kvq

using namespace kvq;

static thread_local int g_last_hip_error = 0;

static int hip_status(hipError_t e) {
    if (e == hipSuccess) return KVQ_OK;
    g_last_hip_error = (int)e;
    return KVQ_EHIP;
}

static bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
static bool supported_d(int D) { return D == 64 || D == 128 || D == 256; }
static bool good_scale(float s) { return isfinite(s) && s > 0.0f; }

extern "C" {

const char* kvq_strerror(int status) {
    switch (status) {
        case KVQ_OK: return "ok";
        case KVQ_EINVAL: return "invalid argument";
        case KVQ_EUNSUPPORTED: return "unsupported shape or option";
        case KVQ_EWORKSPACE: return "workspace too small";
        case KVQ_EHIP: return "HIP launch failed";
        default: return "unknown status";
    }
}

int kvq_last_hip_error(void) { return g_last_hip_error; }

int kvq_abi_version(void) { return KVQ_ABI_VERSION; }

int kvq_check_flags(unsigned* flags_host, int clear) {
    if (!flags_host) return KVQ_EINVAL;
    *flags_host = 0;
    if (!KVQ_CHECK) return KVQ_EUNSUPPORTED;
    const unsigned f = check_flags_attn(clear != 0) | check_flags_cache(clear != 0);
    if (f == ~0u) return hip_status(hipErrorUnknown);
    *flags_host = f;
    return KVQ_OK;
}

int kvq_trace_set(uint64_t* buf_dev, int64_t decode_words, int64_t merge_words) {
    if (decode_words < 0 || merge_words < 0) return KVQ_EINVAL;
    if (!KVQ_TRACE) return KVQ_EUNSUPPORTED;
    const int r = trace_set_attn(buf_dev, decode_words, merge_words);
    return r == 0 ? KVQ_OK : hip_status(hipErrorUnknown);
}

int kvq_e4m3_encode_f32(const float* y_dev, uint8_t* codes_dev, int64_t n, void* hip_stream) {
    if (n < 0) return KVQ_EINVAL;
    if (n == 0) return KVQ_OK;
    if (!y_dev || !codes_dev) return KVQ_EINVAL;
    return hip_status(launch_e4m3_encode(y_dev, codes_dev, n, (hipStream_t)hip_stream));
}

int kvq_e4m3_decode(const uint8_t* codes_dev, void* out_dev, int out_kind, int64_t n, void* hip_stream) {
    if (n < 0 || out_kind < 0 || out_kind > 2) return KVQ_EINVAL;
    if (n == 0) return KVQ_OK;
    if (!codes_dev || !out_dev) return KVQ_EINVAL;
    return hip_status(launch_e4m3_decode(codes_dev, out_dev, out_kind, n, (hipStream_t)hip_stream));
}

int kvq_amax_bf16(const void* x_dev, int64_t rows, int64_t cols, int64_t row_stride, float* amax_dev,
                  void* hip_stream) {
    if (rows < 0 || cols < 0 || !amax_dev) return KVQ_EINVAL;
    if (rows == 0 || cols == 0) return KVQ_OK;
    if (!x_dev || row_stride < cols) return KVQ_EINVAL;
    if (((cols & 7) == 0 && (row_stride & 7) == 0) && !aligned16(x_dev)) return KVQ_EINVAL;
    return hip_status(launch_amax_bf16(x_dev, rows, cols, row_stride, amax_dev, (hipStream_t)hip_stream));
}

static int scales_from_amax(const float* amax_host, float* scale_host, int n, double top) {
    if (n < 0 || (n > 0 && (!amax_host || !scale_host))) return KVQ_EINVAL;
    for (int i = 0; i < n; ++i)
        if (!(amax_host[i] >= 0.0f) || isinf(amax_host[i])) return KVQ_EINVAL;
    for (int i = 0; i < n; ++i) {
        double s = (double)amax_host[i] * 1.05 / top;
        scale_host[i] = (float)(s > 1e-12 ? s : 1e-12);
    }
    return KVQ_OK;
}

int kvq_calibrate(const float* amax_host, float* scale_host, int n) {
    return scales_from_amax(amax_host, scale_host, n, 448.0);
}

int kvq_nvfp4_calibrate(const float* amax_host, float* gscale_host, int n) {
    return scales_from_amax(amax_host, gscale_host, n, 6.0 * 448.0);
}

size_t kvq_nvfp4_region_bytes(int D, int block_size) {
    if (D <= 0 || D % 16 != 0 || block_size <= 0 || block_size % 2 != 0) return 0;
    return (size_t)block_size * D / 2 + (size_t)block_size * D / 16;
}

size_t kvq_nvfp4_cache_bytes_per_block(int Hkv, int D, int block_size) {
    if (Hkv <= 0) return 0;
    return (size_t)Hkv * kvq_nvfp4_region_bytes(D, block_size);
}

int kvq_e2m1_decode(const uint8_t* codes_dev, uint8_t scale_code, void* out_dev, int64_t n_bytes, void* hip_stream) {
    if (n_bytes < 0) return KVQ_EINVAL;
    if (n_bytes == 0) return KVQ_OK;
    if (!codes_dev || !out_dev || ((uintptr_t)out_dev & 3u) != 0) return KVQ_EINVAL;
    return hip_status(launch_e2m1_decode(codes_dev, scale_code, out_dev, n_bytes, (hipStream_t)hip_stream));
}

int kvq_nvfp4_cache_write(const void* k_dev, const void* v_dev, int64_t src_token_stride,
                          const int64_t* slot_mapping_dev, int T, int Hkv, int D, void* k_cache_dev,
                          void* v_cache_dev, int num_blocks, int block_size, float k_gscale, float v_gscale,
                          void* hip_stream) {
    if (T < 0 || Hkv <= 0 || num_blocks <= 0) return KVQ_EINVAL;
    if (!supported_d(D) || block_size != kBlockSize) return KVQ_EUNSUPPORTED;
    if (!good_scale(k_gscale) || !good_scale(v_gscale)) return KVQ_EINVAL;
    if (T == 0) return KVQ_OK;
    if (!k_dev || !v_dev || !slot_mapping_dev || !k_cache_dev || !v_cache_dev) return KVQ_EINVAL;
    if (src_token_stride < (int64_t)Hkv * D || (src_token_stride & 7) != 0) return KVQ_EINVAL;
    if (!aligned16(k_dev) || !aligned16(v_dev) || !aligned16(k_cache_dev) || !aligned16(v_cache_dev))
        return KVQ_EINVAL;
    return hip_status(launch_nvfp4_cache_write(k_dev, v_dev, src_token_stride, slot_mapping_dev, T, Hkv, D,
                                               k_cache_dev, v_cache_dev, k_gscale, v_gscale,
                                               (int64_t)num_blocks * kBlockSize, (hipStream_t)hip_stream));
}

int kvq_cache_write(const void* k_dev, const void* v_dev, int64_t src_token_stride,
                    const int64_t* slot_mapping_dev, int T, int Hkv, int D, void* k_cache_dev,
                    void* v_cache_dev, int num_blocks, int block_size, int kv_dtype, float k_scale,
                    float v_scale, void* hip_stream) {
    if (T < 0 || Hkv <= 0 || num_blocks <= 0) return KVQ_EINVAL;
    if (kv_dtype != KVQ_KV_BF16 && kv_dtype != KVQ_KV_FP8_E4M3) return KVQ_EINVAL;
    if (!supported_d(D) || block_size != kBlockSize) return KVQ_EUNSUPPORTED;
    if (kv_dtype == KVQ_KV_FP8_E4M3 && (!good_scale(k_scale) || !good_scale(v_scale))) return KVQ_EINVAL;
    if (T == 0) return KVQ_OK;
    if (!k_dev || !v_dev || !slot_mapping_dev || !k_cache_dev || !v_cache_dev) return KVQ_EINVAL;
    if (src_token_stride < (int64_t)Hkv * D || (src_token_stride & 7) != 0) return KVQ_EINVAL;
    if (!aligned16(k_dev) || !aligned16(v_dev) || !aligned16(k_cache_dev) || !aligned16(v_cache_dev))
        return KVQ_EINVAL;
    return hip_status(launch_cache_write(k_dev, v_dev, src_token_stride, slot_mapping_dev, T, Hkv, D,
                                         k_cache_dev, v_cache_dev, block_size, kv_dtype, k_scale, v_scale,
                                         (int64_t)num_blocks * kBlockSize, (hipStream_t)hip_stream));
}

int kvq_decode_plan_split_tokens(int B, int Hkv, int max_seq_len, int block_size) {
    (void)block_size;
    if (B < 0 || Hkv <= 0 || max_seq_len < 0) return KVQ_EINVAL;
    return plan_decode(B, Hkv, max_seq_len, 0).split_tokens;
}

size_t kvq_decode_workspace_bytes_ex(int B, int Hq, int Hkv, int D, int max_seq_len, int block_size,
                                     int split_tokens) {
    (void)block_size;
    if (B < 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || max_seq_len < 0) return 0;
    if (split_tokens < 0 || split_tokens % kChunkTokens != 0 || split_tokens > kMaxSplitTokens) return 0;
    DecodePlan p = plan_decode(B, Hkv, max_seq_len, split_tokens);
    if (p.num_splits > kMaxSplits) return 0;
    return decode_workspace_bytes(B, Hq, D, p.num_splits);
}

size_t kvq_decode_workspace_bytes(int B, int Hq, int Hkv, int D, int max_seq_len, int block_size) {
    return kvq_decode_workspace_bytes_ex(B, Hq, Hkv, D, max_seq_len, block_size, 0);
}

// Token span the split plan covers: with a window W, a sequence's splits
// start at most W + q_len - 1 tokens (plus chunk rounding) before its end.
static int plan_span(int max_seq_len, int q_len, int window) {
    if (window <= 0) return max_seq_len;
    const int64_t span = (int64_t)window + q_len - 1 + (kChunkTokens - 1);
    return span < max_seq_len ? (int)span : max_seq_len;
}

// The newest token of each sequence for kvq_paged_decode_attn_append.
struct AppendArgs {
    const void* k_new;
    const void* v_new;
    int64_t stride;
    const int64_t* slots;
};

// ---- the library's own scratch, for callers that cannot allocate ----------------
// kvq_paged_decode_attn_scratch keeps the split partials here instead of in a
// caller workspace: one array per GPU, held by the loaded code object until the
// process ends, shared by every such call on that GPU (calls that overlap on one
// GPU race).  Host code never passes the array's name to a kernel: its address
// on each device comes from hipGetSymbolAddress, taken once per device with that
// device current.
static_assert(KVQ_SCRATCH_MAX_BYTES % 256 == 0, "scratch size is a multiple of 256 bytes");
static __device__ __align__(256) unsigned char scratch[KVQ_SCRATCH_MAX_BYTES];

namespace {
constexpr int kMaxScratchDevices = 64;
struct ScratchSlot {
    std::once_flag once;
    void* ptr = nullptr;
    hipError_t err = hipSuccess;
};
ScratchSlot g_scratch[kMaxScratchDevices];
}  // namespace

// The current device's scratch address (first call per device: the lookup).
static int scratch_address(void** out) {
    int dev = -1;
    const hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_status(e);
    if (dev < 0 || dev >= kMaxScratchDevices) return KVQ_EUNSUPPORTED;
    ScratchSlot& slot = g_scratch[dev];
    std::call_once(slot.once, [&slot] { slot.err = hipGetSymbolAddress(&slot.ptr, HIP_SYMBOL(scratch)); });
    if (slot.err != hipSuccess) return hip_status(slot.err);
    *out = slot.ptr;
    return KVQ_OK;
}

// Where a decode call's split partials go: the caller's workspace, or the
// library's scratch (checked against its size before any HIP call).
enum WorkspaceMode { kCallerWorkspace = 0, kLibraryScratch = 1 };

static int decode_common(int fmt, const void* q_dev, int q_len, int window, const void* k_cache_dev,
                         const void* v_cache_dev,
                         const int32_t* block_tables_dev, int max_blocks_per_seq, const int32_t* seq_lens_dev,
                         int max_seq_len, int B, int Hq, int Hkv, int D, int block_size, int num_blocks,
                         float k_scale, float v_scale, float sm_scale, void* out_dev, int out_dtype,
                         void* workspace_dev, size_t workspace_bytes, void* hip_stream, int impl, int split_tokens,
                         float q_scale = 1.0f, const AppendArgs* app = nullptr,
                         WorkspaceMode ws_mode = kCallerWorkspace) {
    if (B < 0 || Hq <= 0 || Hkv <= 0 || num_blocks <= 0 || max_blocks_per_seq <= 0 || max_seq_len < 0)
        return KVQ_EINVAL;
    if (q_len < 1 || q_len > kMaxQueryLen || window < 0) return KVQ_EINVAL;
    if (Hq % Hkv != 0) return KVQ_EINVAL;
    if (out_dtype != KVQ_OUT_BF16 && out_dtype != KVQ_OUT_F32) return KVQ_EINVAL;
    if (impl < KVQ_IMPL_AUTO || impl > KVQ_IMPL_MFMA) return KVQ_EINVAL;
    if (split_tokens < 0 || split_tokens % kChunkTokens != 0 || split_tokens > kMaxSplitTokens)
        return KVQ_EINVAL;
    if (!supported_d(D) || block_size != kBlockSize) return KVQ_EUNSUPPORTED;
    const int G = Hq / Hkv;
    if (G > 16) return KVQ_EUNSUPPORTED;
    if ((q_len > 1 || window > 0) && impl == KVQ_IMPL_VALU) return KVQ_EUNSUPPORTED;
    if (decode_column_tiles(G, q_len, D) == 0) return KVQ_EUNSUPPORTED;
    if ((int64_t)max_seq_len > (int64_t)max_blocks_per_seq * block_size) return KVQ_EINVAL;
    if (!isfinite(sm_scale) || !(sm_scale > 0.0f)) return KVQ_EINVAL;
    if (fmt != kFmtBF16 && (!good_scale(k_scale) || !good_scale(v_scale))) return KVQ_EINVAL;
    if (fmt == kFmtFP8QP && !good_scale(q_scale)) return KVQ_EINVAL;
    if (B == 0) return KVQ_OK;
    if (!q_dev || !k_cache_dev || !v_cache_dev || !block_tables_dev || !seq_lens_dev || !out_dev ||
        (ws_mode == kCallerWorkspace && !workspace_dev))
        return KVQ_EINVAL;
    if (!aligned16(q_dev) || !aligned16(k_cache_dev) || !aligned16(v_cache_dev) || !aligned16(out_dev) ||
        (ws_mode == kCallerWorkspace && !aligned16(workspace_dev)))
        return KVQ_EINVAL;
    const DecodePlan plan = plan_decode(B, Hkv, plan_span(max_seq_len, q_len, window), split_tokens);
    if (plan.num_splits > kMaxSplits) return KVQ_EUNSUPPORTED;
    const size_t need = decode_workspace_bytes(B * q_len, Hq, D, plan.num_splits);
    if (ws_mode == kLibraryScratch) {
        if (need > (size_t)KVQ_SCRATCH_MAX_BYTES) return KVQ_EWORKSPACE;
        const int st = scratch_address(&workspace_dev);   // the first HIP call of this path
        if (st != KVQ_OK) return st;
        workspace_bytes = KVQ_SCRATCH_MAX_BYTES;
    }
    if (workspace_bytes < need) return KVQ_EWORKSPACE;
    if (impl == KVQ_IMPL_AUTO || fmt == kFmtNVFP4) impl = KVQ_IMPL_MFMA;

    const bool scaled = fmt != kFmtBF16;
    DecodeArgs a = {};
    a.q = (const uint16_t*)q_dev;
    a.k_cache = (const uint8_t*)k_cache_dev;
    a.v_cache = (const uint8_t*)v_cache_dev;
    a.block_tables = block_tables_dev;
    a.seq_lens = seq_lens_dev;
    a.ws_ml = (float*)workspace_dev;
    a.ws_acc = (float*)((char*)a.ws_ml + decode_ml_bytes(B * q_len, Hq, plan.num_splits));
    a.out = out_dev;
    a.max_blocks = max_blocks_per_seq;
    a.num_blocks = num_blocks;
    a.max_seq_len = max_seq_len;
    a.Hq = Hq;
    a.Hkv = Hkv;
    a.G = G;
    a.split_tokens = plan.split_tokens;
    a.num_splits = plan.num_splits;
    a.qk_scale_log2 = fmt == kFmtFP8QP
                          ? (float)((double)sm_scale * (double)q_scale * (double)k_scale * 1.4426950408889634)
                          : (float)((double)sm_scale * (scaled ? (double)k_scale : 1.0) * 1.4426950408889634);
    a.q_scale = q_scale;
    a.v_scale = scaled ? v_scale : 1.0f;
    a.out_f32 = out_dtype == KVQ_OUT_F32;
    a.q_len = q_len;
    a.window = window;
    if (app) {
        a.k_new = (const uint16_t*)app->k_new;
        a.v_new = (const uint16_t*)app->v_new;
        a.new_stride = app->stride;
        a.new_slots = app->slots;
        a.k_scale_w = k_scale;
        a.v_scale_w = v_scale;
    }
    return hip_status(launch_decode(a, B, D, fmt, impl, (hipStream_t)hip_stream));
}

int kvq_paged_decode_attn_ex(const void* q_dev, const void* k_cache_dev, const void* v_cache_dev, int kv_dtype,
                             const int32_t* block_tables_dev, int max_blocks_per_seq, const int32_t* seq_lens_dev,
                             int max_seq_len, int B, int Hq, int Hkv, int D, int block_size, int num_blocks,
                             float k_scale, float v_scale, float sm_scale, void* out_dev, int out_dtype,
                             void* workspace_dev, size_t workspace_bytes, void* hip_stream, int impl,
                             int split_tokens) {
    if (kv_dtype != KVQ_KV_BF16 && kv_dtype != KVQ_KV_FP8_E4M3) return KVQ_EINVAL;
    return decode_common(kv_dtype == KVQ_KV_FP8_E4M3 ? kFmtFP8 : kFmtBF16, q_dev, 1, 0, k_cache_dev, v_cache_dev,
                         block_tables_dev, max_blocks_per_seq, seq_lens_dev, max_seq_len, B, Hq, Hkv, D,
                         block_size, num_blocks, k_scale, v_scale, sm_scale, out_dev, out_dtype, workspace_dev,
                         workspace_bytes, hip_stream, impl, split_tokens);
}

int kvq_paged_decode_attn_scratch(const void* q_dev, const void* k_cache_dev, const void* v_cache_dev, int kv_dtype,
                                  const int32_t* block_tables_dev, int max_blocks_per_seq,
                                  const int32_t* seq_lens_dev, int max_seq_len, int B, int Hq, int Hkv, int D,
                                  int block_size, int num_blocks, float k_scale, float v_scale, float sm_scale,
                                  void* out_dev, int out_dtype, void* hip_stream) {
    if (kv_dtype != KVQ_KV_BF16 && kv_dtype != KVQ_KV_FP8_E4M3) return KVQ_EINVAL;
    return decode_common(kv_dtype == KVQ_KV_FP8_E4M3 ? kFmtFP8 : kFmtBF16, q_dev, 1, 0, k_cache_dev, v_cache_dev,
                         block_tables_dev, max_blocks_per_seq, seq_lens_dev, max_seq_len, B, Hq, Hkv, D,
                         block_size, num_blocks, k_scale, v_scale, sm_scale, out_dev, out_dtype, nullptr, 0,
                         hip_stream, KVQ_IMPL_AUTO, 0, 1.0f, nullptr, kLibraryScratch);
}

int kvq_nvfp4_paged_decode_attn_ex(const void* q_dev, const void* k_cache_dev, const void* v_cache_dev,
                                   const int32_t* block_tables_dev, int max_blocks_per_seq,
                                   const int32_t* seq_lens_dev, int max_seq_len, int B, int Hq, int Hkv, int D,
                                   int block_size, int num_blocks, float k_gscale, float v_gscale, float sm_scale,
                                   void* out_dev, int out_dtype, void* workspace_dev, size_t workspace_bytes,
                                   void* hip_stream, int split_tokens) {
    return decode_common(kFmtNVFP4, q_dev, 1, 0, k_cache_dev, v_cache_dev, block_tables_dev, max_blocks_per_seq,
                         seq_lens_dev, max_seq_len, B, Hq, Hkv, D, block_size, num_blocks, k_gscale, v_gscale,
                         sm_scale, out_dev, out_dtype, workspace_dev, workspace_bytes, hip_stream, KVQ_IMPL_MFMA,
                         split_tokens);
}

int kvq_nvfp4_paged_decode_attn(const void* q_dev, const void* k_cache_dev, const void* v_cache_dev,
                                const int32_t* block_tables_dev, int max_blocks_per_seq, const int32_t* seq_lens_dev,
                                int max_seq_len, int B, int Hq, int Hkv, int D, int block_size, int num_blocks,
                                float k_gscale, float v_gscale, float sm_scale, void* out_dev, int out_dtype,
                                void* workspace_dev, size_t workspace_bytes, void* hip_stream) {
    return kvq_nvfp4_paged_decode_attn_ex(q_dev, k_cache_dev, v_cache_dev, block_tables_dev, max_blocks_per_seq,
                                          seq_lens_dev, max_seq_len, B, Hq, Hkv, D, block_size, num_blocks,
                                          k_gscale, v_gscale, sm_scale, out_dev, out_dtype, workspace_dev,
                                          workspace_bytes, hip_stream, 0);
}

size_t kvq_decode_workspace_bytes_mq(int B, int q_len, int window, int Hq, int Hkv, int D, int max_seq_len,
                                     int block_size, int split_tokens) {
    (void)block_size;
    if (q_len < 1 || q_len > kMaxQueryLen || window < 0) return 0;
    if (B < 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || max_seq_len < 0) return 0;
    if (split_tokens < 0 || split_tokens % kChunkTokens != 0 || split_tokens > kMaxSplitTokens) return 0;
    const DecodePlan p = plan_decode(B, Hkv, plan_span(max_seq_len, q_len, window), split_tokens);
    if (p.num_splits > kMaxSplits) return 0;
    return decode_workspace_bytes(B * q_len, Hq, D, p.num_splits);
}

int kvq_paged_decode_attn_mq(const void* q_dev, int q_len, int window, const void* k_cache_dev,
                             const void* v_cache_dev, int kv_dtype, const int32_t* block_tables_dev, int max_blocks_per_seq,
                             const int32_t* seq_lens_dev, int max_seq_len, int B, int Hq, int Hkv, int D,
                             int block_size, int num_blocks, float k_scale, float v_scale, float sm_scale,
                             void* out_dev, int out_dtype, void* workspace_dev, size_t workspace_bytes,
                             void* hip_stream, int split_tokens) {
    if (kv_dtype != KVQ_KV_BF16 && kv_dtype != KVQ_KV_FP8_E4M3) return KVQ_EINVAL;
    return decode_common(kv_dtype == KVQ_KV_FP8_E4M3 ? kFmtFP8 : kFmtBF16, q_dev, q_len, window, k_cache_dev,
                         v_cache_dev, block_tables_dev, max_blocks_per_seq, seq_lens_dev, max_seq_len, B, Hq, Hkv,
                         D, block_size, num_blocks, k_scale, v_scale, sm_scale, out_dev, out_dtype, workspace_dev,
                         workspace_bytes, hip_stream, KVQ_IMPL_MFMA, split_tokens);
}

int kvq_nvfp4_paged_decode_attn_mq(const void* q_dev, int q_len, int window, const void* k_cache_dev,
                                   const void* v_cache_dev,
                                   const int32_t* block_tables_dev, int max_blocks_per_seq,
                                   const int32_t* seq_lens_dev, int max_seq_len, int B, int Hq, int Hkv, int D,
                                   int block_size, int num_blocks, float k_gscale, float v_gscale, float sm_scale,
                                   void* out_dev, int out_dtype, void* workspace_dev, size_t workspace_bytes,
                                   void* hip_stream, int split_tokens) {
    return decode_common(kFmtNVFP4, q_dev, q_len, window, k_cache_dev, v_cache_dev, block_tables_dev,
                         max_blocks_per_seq,
                         seq_lens_dev, max_seq_len, B, Hq, Hkv, D, block_size, num_blocks, k_gscale, v_gscale,
                         sm_scale, out_dev, out_dtype, workspace_dev, workspace_bytes, hip_stream, KVQ_IMPL_MFMA,
                         split_tokens);
}

size_t kvq_cache_block_bytes(int kv_format, int Hkv, int D, int block_size) {
    if (Hkv <= 0 || !supported_d(D) || block_size != kBlockSize) return 0;
    if (kv_format == 2) return (size_t)Hkv * (size_t)(kBlockSize * D / 2 + kBlockSize * D / 16);
    if (kv_format == KVQ_KV_BF16) return (size_t)Hkv * kBlockSize * D * 2;
    if (kv_format == KVQ_KV_FP8_E4M3) return (size_t)Hkv * kBlockSize * D;
    return 0;
}

static int block_copy_args(const void* a, const void* b, size_t block_bytes, const int32_t* ids, int n) {
    if (n < 0 || block_bytes == 0 || block_bytes % 16 != 0) return KVQ_EINVAL;
    if (n == 0) return KVQ_OK;
    if (!a || !b || !ids || !aligned16(a) || !aligned16(b)) return KVQ_EINVAL;
    return 1;
}

int kvq_gather_blocks(const void* cache_dev, size_t block_bytes, const int32_t* block_ids_dev, int n, void* dst_dev,
                      void* hip_stream) {
    const int v = block_copy_args(cache_dev, dst_dev, block_bytes, block_ids_dev, n);
    if (v != 1) return v;
    return hip_status(launch_block_copy(cache_dev, dst_dev, block_ids_dev, n, block_bytes, 1, (hipStream_t)hip_stream));
}

int kvq_scatter_blocks(const void* src_dev, size_t block_bytes, const int32_t* block_ids_dev, int n, void* cache_dev,
                       void* hip_stream) {
    const int v = block_copy_args(src_dev, cache_dev, block_bytes, block_ids_dev, n);
    if (v != 1) return v;
    return hip_status(launch_block_copy(src_dev, cache_dev, block_ids_dev, n, block_bytes, 0, (hipStream_t)hip_stream));
}

int kvq_offload_blocks(const void* k_cache_dev, const void* v_cache_dev, size_t block_bytes,
                       const int32_t* block_ids_dev, int n, void* staging_dev, void* host_dst, void* hip_stream) {
    int v = block_copy_args(k_cache_dev, v_cache_dev, block_bytes, block_ids_dev, n);
    if (v != 1) return v;
    if (!staging_dev || !host_dst || !aligned16(staging_dev)) return KVQ_EINVAL;
    const hipStream_t st = (hipStream_t)hip_stream;
    const size_t half = (size_t)n * block_bytes;
    v = hip_status(launch_block_copy(k_cache_dev, staging_dev, block_ids_dev, n, block_bytes, 1, st));
    if (v != KVQ_OK) return v;
    v = hip_status(launch_block_copy(v_cache_dev, (char*)staging_dev + half, block_ids_dev, n, block_bytes, 1, st));
    if (v != KVQ_OK) return v;
    return hip_status(hipMemcpyAsync(host_dst, staging_dev, 2 * half, hipMemcpyDeviceToHost, st));
}

int kvq_restore_blocks(const void* host_src, void* staging_dev, size_t block_bytes, const int32_t* block_ids_dev,
                       int n, void* k_cache_dev, void* v_cache_dev, void* hip_stream) {
    int v = block_copy_args(k_cache_dev, v_cache_dev, block_bytes, block_ids_dev, n);
    if (v != 1) return v;
    if (!staging_dev || !host_src || !aligned16(staging_dev)) return KVQ_EINVAL;
    const hipStream_t st = (hipStream_t)hip_stream;
    const size_t half = (size_t)n * block_bytes;
    v = hip_status(hipMemcpyAsync(staging_dev, host_src, 2 * half, hipMemcpyHostToDevice, st));
    if (v != KVQ_OK) return v;
    v = hip_status(launch_block_copy(staging_dev, k_cache_dev, block_ids_dev, n, block_bytes, 0, st));
    if (v != KVQ_OK) return v;
    return hip_status(launch_block_copy((const char*)staging_dev + half, v_cache_dev, block_ids_dev, n, block_bytes, 0,
                                        st));
}

int kvq_paged_decode_attn_append(const void* k_new_dev, const void* v_new_dev, int64_t new_token_stride,
                                 const int64_t* slot_mapping_dev, const void* q_dev, void* k_cache_dev,
                                 void* v_cache_dev, int kv_dtype, const int32_t* block_tables_dev,
                                 int max_blocks_per_seq, const int32_t* seq_lens_dev, int max_seq_len, int B, int Hq,
                                 int Hkv, int D, int block_size, int num_blocks, float k_scale, float v_scale,
                                 float sm_scale, void* out_dev, int out_dtype, void* workspace_dev,
                                 size_t workspace_bytes, void* hip_stream, int split_tokens) {
    if (kv_dtype != KVQ_KV_BF16 && kv_dtype != KVQ_KV_FP8_E4M3) return KVQ_EINVAL;
    if (B > 0) {
        if (!k_new_dev || !v_new_dev || !slot_mapping_dev) return KVQ_EINVAL;
        if (new_token_stride < (int64_t)Hkv * D || (new_token_stride & 7) != 0) return KVQ_EINVAL;
        if (!aligned16(k_new_dev) || !aligned16(v_new_dev)) return KVQ_EINVAL;
    }
    const AppendArgs app = {k_new_dev, v_new_dev, new_token_stride, slot_mapping_dev};
    return decode_common(kv_dtype == KVQ_KV_FP8_E4M3 ? kFmtFP8 : kFmtBF16, q_dev, 1, 0, k_cache_dev, v_cache_dev,
                         block_tables_dev, max_blocks_per_seq, seq_lens_dev, max_seq_len, B, Hq, Hkv, D,
                         block_size, num_blocks, k_scale, v_scale, sm_scale, out_dev, out_dtype, workspace_dev,
                         workspace_bytes, hip_stream, KVQ_IMPL_MFMA, split_tokens, 1.0f, &app);
}

int kvq_paged_decode_attn_mq_append(const void* k_new_dev, const void* v_new_dev, int64_t new_token_stride,
                                    const int64_t* slot_mapping_dev, const void* q_dev, int q_len, int window,
                                    void* k_cache_dev, void* v_cache_dev, int kv_dtype,
                                    const int32_t* block_tables_dev, int max_blocks_per_seq,
                                    const int32_t* seq_lens_dev, int max_seq_len, int B, int Hq, int Hkv, int D,
                                    int block_size, int num_blocks, float k_scale, float v_scale, float sm_scale,
                                    void* out_dev, int out_dtype, void* workspace_dev, size_t workspace_bytes,
                                    void* hip_stream, int split_tokens) {
    if (kv_dtype != KVQ_KV_BF16 && kv_dtype != KVQ_KV_FP8_E4M3) return KVQ_EINVAL;
    if (B > 0) {
        if (!k_new_dev || !v_new_dev || !slot_mapping_dev) return KVQ_EINVAL;
        if (new_token_stride < (int64_t)Hkv * D || (new_token_stride & 7) != 0) return KVQ_EINVAL;
        if (!aligned16(k_new_dev) || !aligned16(v_new_dev)) return KVQ_EINVAL;
    }
    const AppendArgs app = {k_new_dev, v_new_dev, new_token_stride, slot_mapping_dev};
    return decode_common(kv_dtype == KVQ_KV_FP8_E4M3 ? kFmtFP8 : kFmtBF16, q_dev, q_len, window, k_cache_dev,
                         v_cache_dev, block_tables_dev, max_blocks_per_seq, seq_lens_dev, max_seq_len, B, Hq, Hkv, D,
                         block_size, num_blocks, k_scale, v_scale, sm_scale, out_dev, out_dtype, workspace_dev,
                         workspace_bytes, hip_stream, KVQ_IMPL_MFMA, split_tokens, 1.0f, &app);
}

int kvq_nvfp4_paged_decode_attn_append(const void* k_new_dev, const void* v_new_dev, int64_t new_token_stride,
                                       const int64_t* slot_mapping_dev, const void* q_dev, void* k_cache_dev,
                                       void* v_cache_dev, const int32_t* block_tables_dev, int max_blocks_per_seq,
                                       const int32_t* seq_lens_dev, int max_seq_len, int B, int Hq, int Hkv, int D,
                                       int block_size, int num_blocks, float k_gscale, float v_gscale,
                                       float sm_scale, void* out_dev, int out_dtype, void* workspace_dev,
                                       size_t workspace_bytes, void* hip_stream, int split_tokens) {
    if (B > 0) {
        if (!k_new_dev || !v_new_dev || !slot_mapping_dev) return KVQ_EINVAL;
        if (new_token_stride < (int64_t)Hkv * D || (new_token_stride & 7) != 0) return KVQ_EINVAL;
        if (!aligned16(k_new_dev) || !aligned16(v_new_dev)) return KVQ_EINVAL;
    }
    const AppendArgs app = {k_new_dev, v_new_dev, new_token_stride, slot_mapping_dev};
    return decode_common(kFmtNVFP4, q_dev, 1, 0, k_cache_dev, v_cache_dev, block_tables_dev, max_blocks_per_seq,
                         seq_lens_dev, max_seq_len, B, Hq, Hkv, D, block_size, num_blocks, k_gscale, v_gscale,
                         sm_scale, out_dev, out_dtype, workspace_dev, workspace_bytes, hip_stream, KVQ_IMPL_MFMA,
                         split_tokens, 1.0f, &app);
}

int kvq_paged_decode_attn_fp8qp(const void* q_dev, int q_len, int window, const void* k_cache_dev,
                                const void* v_cache_dev, const int32_t* block_tables_dev, int max_blocks_per_seq,
                                const int32_t* seq_lens_dev, int max_seq_len, int B, int Hq, int Hkv, int D,
                                int block_size, int num_blocks, float q_scale, float k_scale, float v_scale,
                                float sm_scale, void* out_dev, int out_dtype, void* workspace_dev,
                                size_t workspace_bytes, void* hip_stream, int split_tokens) {
    return decode_common(kFmtFP8QP, q_dev, q_len, window, k_cache_dev, v_cache_dev, block_tables_dev,
                         max_blocks_per_seq, seq_lens_dev, max_seq_len, B, Hq, Hkv, D, block_size, num_blocks,
                         k_scale, v_scale, sm_scale, out_dev, out_dtype, workspace_dev, workspace_bytes, hip_stream,
                         KVQ_IMPL_MFMA, split_tokens, q_scale);
}

int kvq_paged_decode_attn(const void* q_dev, const void* k_cache_dev, const void* v_cache_dev, int kv_dtype,
                          const int32_t* block_tables_dev, int max_blocks_per_seq, const int32_t* seq_lens_dev,
                          int max_seq_len, int B, int Hq, int Hkv, int D, int block_size, int num_blocks,
                          float k_scale, float v_scale, float sm_scale, void* out_dev, int out_dtype,
                          void* workspace_dev, size_t workspace_bytes, void* hip_stream) {
    return kvq_paged_decode_attn_ex(q_dev, k_cache_dev, v_cache_dev, kv_dtype, block_tables_dev,
                                    max_blocks_per_seq, seq_lens_dev, max_seq_len, B, Hq, Hkv, D, block_size,
                                    num_blocks, k_scale, v_scale, sm_scale, out_dev, out_dtype, workspace_dev,
                                    workspace_bytes, hip_stream, KVQ_IMPL_AUTO, 0);
}

}  // extern "C"
