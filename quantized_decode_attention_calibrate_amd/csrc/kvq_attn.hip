// kvq_attn.hip -- split-K paged decode attention with the dequantization
// fused into the attention kernel, and the cross-split merge.  One kernel
// template covers the FP8, BF16 and NVFP4 caches, multi-query decode (the
// q_len newest tokens, each causal), sliding windows, the FP8 Q and P variant
// and the fused cache write of each sequence's newest token.
//
// The Run 26 video description (Skildcore, "KV Cache Precision") states the
// problem these kernels answer: each generated token reads the whole KV
// cache, so decode is a bandwidth-bound scan; halving the bytes with FP8 gave
// no speed-up on its hardware because no fused dequant kernel existed
// (chapter "The Missing Fused Dequant Kernel"); accuracy needs fp32
// accumulation at two levels ("two-level FP32 accumulation").  Here the
// levels are the per-split online softmax (fp32 m, l, acc) and the fp32
// log-sum-exp merge across splits.
//
// Work decomposition (MI355X: 256 CUs, wave64): one work-group of 4 waves (8
// for NVFP4 at D 64) per (split s, KV head g, sequence b).  A split is a
// fixed range of logical tokens (a multiple of 64), so results do not depend
// on physical block placement.  Each wave walks 64-token chunks (4 blocks of
// 16) of the split round-robin, staging the physical block ids of its own
// chunks in LDS (no work-group barrier before the loads); the waves merge through LDS and write one fp32 partial
// (m, l, acc[G][D]) per head to the workspace; the merge kernel combines the
// splits and applies v_scale.
//
// Two kernel families:
//   MFMA: QK^T on v_mfma_f32_16x16x32_bf16 (E4M3 -> bf16 is exact; bf16 x
//         bf16 products are exact in fp32) and PV on v_mfma_f32_16x16x32_f16
//         (E4M3 -> f16 is exact; each fp32 softmax weight is split into f16
//         hi + lo parts, two MFMAs on the same V operand).  The G query heads
//         sharing a KV head are the 16-wide N dimension (padded), so each K/V
//         byte is read once per KV head.
//   VALU: plain fp32 FMAs with Q staged in LDS; the comparator.
#include <type_traits>

#include "kvq_device.h"
#include "kvq_internal.h"

namespace kvq {

constexpr int kWaves = 4;                 // VALU family work-group
constexpr int kThreads = kWaves * 64;
// MFMA family: 8 waves per work-group for NVFP4 at D = 64, else 4.  The
// 4-bit path spends about twice the VALU work per byte of the FP8 path, and
// a second wave per SIMD hides it (measured 44 -> 42 us on a 2 x 131k-token
// decode); for FP8 and BF16 the extra waves only shorten each wave's chunk
// run and were measured neutral to slightly slower.
template <int D, int FMT, int NT>
constexpr int mfma_waves() { return (FMT == kFmtNVFP4 && D == 64 && NT == 1) ? 8 : 4; }
constexpr int kMaxSplitBlocks = kMaxSplitTokens / kBlockSize;

// Columns: a work-group serves the G query heads of one KV head for each of
// the q_len queries of its sequence (q_len = 1 for single-token decode):
// column c = i * G + hl is query i, head g * G + hl, and its output row is
// (b * q_len + i) * Hq + g * G + hl.  The MFMA family holds the columns in NT
// tiles of 16; GQ = G * q_len <= 16 * NT.
__device__ __forceinline__ int64_t column_row(const DecodeArgs& a, int b, int g, int c) {
    const int i = c / a.G;
    return ((int64_t)b * a.q_len + i) * a.Hq + (int64_t)g * a.G + (c - i * a.G);
}

// LDS layout shared by both families (dynamic shared memory):
//   int   blk[kMaxSplitBlocks]          physical block ids of this split
//   float m[W][16 NT], l[W][16 NT]      per-wave softmax state per column (W waves)
//   float acc[W][GQ][D]                 per-wave unnormalised outputs
//   (VALU only) float q[G][D], p[W][16][16]
__host__ __device__ constexpr int lds_merge_floats(int GQ, int D, int W, int NT = 1) {
    return W * 32 * NT + W * GQ * D;
}

// ---- phase trace (KVQ_TRACE builds) ------------------------------------------
// Decode: 8 words per wave at ((work-group linear id) * W + wave) * 8 of the
// decode region: stamps at the start, after the sequence length, after the
// block-id staging, after the first chunk, at the loop end and at the end;
// then chunks | split << 20 | KV head << 36 | sequence << 44, and
// 1 | XCC id << 8 | HW_ID << 16.  Merge: 4 words per output row of the merge
// region: start, after the split weights, end, 1.  Stamps count the 100 MHz
// real-time clock.
#if KVQ_TRACE
__device__ uint64_t* g_trace = nullptr;
__device__ int64_t g_trace_words[2] = {0, 0};   // decode region, merge region (words)
__device__ __forceinline__ uint64_t trace_now(bool drain) {
    if (drain) __builtin_amdgcn_s_waitcnt(0);   // stamp after the loads issued so far have landed
    return __builtin_amdgcn_s_memrealtime();
}
struct PhaseTrace {
    uint64_t t[6] = {0, 0, 0, 0, 0, 0};
    __device__ __forceinline__ void mark(int i, bool drain = true) { t[i] = trace_now(drain); }
    __device__ __forceinline__ void store_decode(int W, int wave, int lane, int chunks, int s, int g, int b) const {
        const int64_t wg = blockIdx.x + (int64_t)gridDim.x * (blockIdx.y + (int64_t)gridDim.y * blockIdx.z);
        const int64_t base = (wg * W + wave) * 8;
        if (lane != 0 || !g_trace || base + 8 > g_trace_words[0]) return;
        uint64_t* o = g_trace + base;
        for (int i = 0; i < 6; ++i) o[i] = t[i];
        o[6] = (uint64_t)chunks | ((uint64_t)s << 20) | ((uint64_t)g << 36) | ((uint64_t)b << 44);
        const uint32_t xcc = (uint32_t)__builtin_amdgcn_s_getreg(0xF814) & 15u;   // hwreg(HW_REG_XCC_ID)
        const uint32_t hw = (uint32_t)__builtin_amdgcn_s_getreg(0xF804);          // hwreg(HW_REG_HW_ID)
        o[7] = 1ull | ((uint64_t)xcc << 8) | ((uint64_t)hw << 16);
    }
    __device__ __forceinline__ void store_merge(int64_t row) const {
        const int64_t base = g_trace_words[0] + row * 4;
        if (threadIdx.x != 0 || !g_trace || row * 4 + 4 > g_trace_words[1]) return;
        uint64_t* o = g_trace + base;
        o[0] = t[0];
        o[1] = t[1];
        o[2] = t[2];
        o[3] = 1ull;
    }
};
#define KVQ_TRACE_DECL PhaseTrace trace_
#define KVQ_TRACE_MARK(...) trace_.mark(__VA_ARGS__)
#define KVQ_TRACE_STORE_DECODE(...) trace_.store_decode(__VA_ARGS__)
#define KVQ_TRACE_STORE_MERGE(row) trace_.store_merge(row)
#else
// (release and checked builds: no trace code at all)
#define KVQ_TRACE_DECL
#define KVQ_TRACE_MARK(...)
#define KVQ_TRACE_STORE_DECODE(...)
#define KVQ_TRACE_STORE_MERGE(row)
#endif

// Stage the physical block ids of logical blocks [lb0, lb0 + n) into LDS,
// clamping logical blocks past the sequence to its last block and blocks
// before a sliding window to the window's first block (those tokens are
// masked; the clamp keeps every address inside the cache and reads no table
// entry outside [first_lb, last_lb]).
__device__ __forceinline__ void stage_block_ids(int* s_blk, const int32_t* bt_row, int lb0, int n,
                                                int first_lb, int last_lb, int num_blocks) {
    for (int i = threadIdx.x; i < n; i += blockDim.x) {
        int lb = min(max(lb0 + i, first_lb), last_lb);
        int id = bt_row[lb];
        if (KVQ_CHECK && (unsigned)id >= (unsigned)num_blocks) {
            check_fail(kCheckBlockId);
            id = 0;
        }
        s_blk[i] = id;
    }
}

// Token range of sequence b's work-groups.  Query i is the token at position
// p = L - q_len + i and sees tokens max(0, p - window + 1) .. p (window 0:
// from 0).  `first` is the first token any query sees; splits start at
// `base` = first rounded down to a chunk, so no split lies wholly before it.
struct SeqRange {
    int L, first, base;
};
__device__ __forceinline__ int seq_len(const DecodeArgs& a, int b) {
    int L = a.seq_lens[b];
    if (KVQ_CHECK && (L < 0 || L > a.max_seq_len)) {
        check_fail(kCheckSeqLen);
        L = min(max(L, 0), a.max_seq_len);
    }
    return L;
}
__device__ __forceinline__ SeqRange seq_range(const DecodeArgs& a, int b) {
    SeqRange r;
    r.L = seq_len(a, b);
    r.first = a.window > 0 ? max(0, r.L - a.q_len - a.window + 1) : 0;
    r.base = r.first & ~(kChunkTokens - 1);
    return r;
}

// Merge the 4 waves' (m, l, acc) held in LDS into this split's result.  If the
// split holds the whole sequence the result is final and goes to `out`
// directly; otherwise it is stored as an fp32 partial for merge_splits_kernel.
__device__ __forceinline__ void store_out(const DecodeArgs& a, int64_t o, float v) {
    if (a.out_f32)
        reinterpret_cast<float*>(a.out)[o] = v;
    else
        reinterpret_cast<uint16_t*>(a.out)[o] = (uint16_t)f32_to_bf16_rne(v);
}

template <int W, int NT = 1>
__device__ __forceinline__ void finish_split(const DecodeArgs& a, const float* s_m, const float* s_l,
                                             const float* s_acc, int b, int g, int s, int S, int D) {
    constexpr int CP = 16 * NT;   // columns per wave in s_m / s_l
    const int GQ = a.G * a.q_len;
    for (int idx = threadIdx.x; idx < GQ * D; idx += W * 64) {
        const int c = idx / D, d = idx - c * D;
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < W; ++w) M = fmaxf(M, s_m[w * CP + c]);
        float acc = 0.f, l = 0.f;
#pragma unroll
        for (int w = 0; w < W; ++w) {
            const float mw = s_m[w * CP + c];
            const float f = (mw == -INFINITY) ? 0.f : fast_exp2(mw - M);
            acc += f * s_acc[(w * GQ + c) * D + d];
            l += f * s_l[w * CP + c];
        }
        const int64_t r = column_row(a, b, g, c);
        if (S == 1) {
            // l == 0: a query that sees no token (it sits before the sequence start)
            store_out(a, r * D + d, l > 0.f ? acc * (a.v_scale / l) : 0.f);
        } else {
            a.ws_acc[(r * a.num_splits + s) * D + d] = acc;
            if (d == 0) {
                a.ws_ml[(r * a.num_splits + s) * 2 + 0] = M;
                a.ws_ml[(r * a.num_splits + s) * 2 + 1] = l;
            }
        }
    }
}

// A sequence with no tokens: work-group (split 0) writes zeros for its columns.
__device__ __forceinline__ void write_empty(const DecodeArgs& a, int b, int g, int D) {
    const int GQ = a.G * a.q_len;
    for (int idx = threadIdx.x; idx < GQ * D; idx += blockDim.x) {
        const int c = idx / D;
        store_out(a, column_row(a, b, g, c) * D + (idx - c * D), 0.f);
    }
}

// =============================================================================
// MFMA family
// =============================================================================
//
// Lane roles (lane = 16 * grp + n, grp = lane / 16, n = lane % 16); a chunk is
// logical blocks c0 .. c0+3 of the split (chunk blocks 0..3).
//   QK tile i (i = 0..3), MFMA C = K_tile x Q^T:
//     A row m = n  <- token (chunk block n/4, offset 4i + n%4); the lane loads
//                     16 contiguous K bytes (dims 64j + 16grp .. +15) per
//                     64-dim slice j, i.e. two 8-wide k-steps
//     B col n      <- query head g*G + n (zero when n >= G), same dims
//     C            -> lane holds S[token (chunk block grp, offset 4i + r)][head n], r = 0..3
//   so after the 4 tiles each lane holds all 16 scores of chunk block grp for
//   head n, which is exactly the P^T operand layout PV needs.
//   PV, dim tile dt (D/16 tiles), half hh (tokens 8hh..8hh+7), MFMA C = V^T x P^T:
//     A row m = n  <- dim 16dt + n of chunk block grp: the V block is dim-major,
//                     so the lane's 16 contiguous bytes are that dim's 16 tokens
//     B col n      <- weights of head n for the same 8 tokens
//     C            -> acc[dt]: lane holds out[dim 16dt + 4grp + r][head n]

// Raw bytes of one 64-token chunk as this lane needs them, per cache format.
template <int D, int FMT>
struct MfmaChunk;
template <int D>
struct MfmaChunk<D, kFmtFP8> {        // 16 K bytes per (tile, slice); 16 tokens of one V dim
    u32x4 kw[4][D / 64];
    u32x4 vw[D / 16];
};
template <int D>
struct MfmaChunk<D, kFmtBF16> {       // the same elements at two bytes each
    u32x4 kw[4][D / 64][2];
    u32x4 vw[D / 16][2];
};
template <int D>
struct MfmaChunk<D, kFmtFP8QP> : MfmaChunk<D, kFmtFP8> {};   // the same raw FP8 bytes
template <int D>
struct MfmaChunk<D, kFmtNVFP4> {      // 16 E2M1 codes + 1 scale per (tile, slice); V dim row + 16 token scales
    u32x2 kc[4][D / 64];
    uint32_t ks[4][D / 64];
    u32x2 vc[D / 16];
    u32x4 vs[D / 16];
};

// Per-wave running softmax state of column 16 nt + n (lane % 16) per tile nt.
template <int D, int NT>
struct MfmaState {
    f32x4 acc[NT][D / 16];
    float m_run[NT], l_run[NT];
};

template <int D, int FMT>
__device__ __forceinline__ void mfma_load(MfmaChunk<D, FMT>& c, const DecodeArgs& a, const int* s_blk, int ch,
                                          int g, int n, int grp) {
    constexpr int KJ = D / 64, DT = D / 16;
    const int pk = s_blk[ch * 4 + (n >> 2)];   // block of this lane's K rows
    const int pv = s_blk[ch * 4 + grp];        // block of this lane's V rows
    if constexpr (FMT == kFmtNVFP4) {
        constexpr int64_t region = 9 * D;              // 16*D/2 code bytes + 16*D/16 scale bytes
        constexpr int64_t codes = 8 * D;
        const uint8_t* kr = a.k_cache + ((int64_t)pk * a.Hkv + g) * region;
        const uint8_t* vr = a.v_cache + ((int64_t)pv * a.Hkv + g) * region;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int off = 4 * i + (n & 3);
#pragma unroll
            for (int j = 0; j < KJ; ++j) {
                c.kc[i][j] = *reinterpret_cast<const u32x2*>(kr + off * (D / 2) + 32 * j + 8 * grp);
                // the aligned dword holding this row's 4 block scales of slice j; the
                // lane's (byte grp) is selected at use.  A byte load here made the
                // compiler zero-extend the next chunk's scales at the end of the
                // loop body, which waited on that chunk's just-issued loads.
                c.ks[i][j] = *reinterpret_cast<const uint32_t*>(kr + codes + off * (D / 16) + 4 * j);
            }
        }
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
            c.vc[dt] = *reinterpret_cast<const u32x2*>(vr + (16 * dt + n) * 8);
            c.vs[dt] = *reinterpret_cast<const u32x4*>(vr + codes + 16 * dt);
        }
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int off = 4 * i + (n & 3);
            const int64_t row = (((int64_t)pk * a.Hkv + g) * kBlockSize + off) * D;
#pragma unroll
            for (int j = 0; j < KJ; ++j) {
                if constexpr (FMT == kFmtFP8 || FMT == kFmtFP8QP) {
                    c.kw[i][j] = *reinterpret_cast<const u32x4*>(a.k_cache + row + 64 * j + 16 * grp);
                } else {
                    const uint16_t* kc = reinterpret_cast<const uint16_t*>(a.k_cache) + row + 64 * j + 16 * grp;
                    c.kw[i][j][0] = *reinterpret_cast<const u32x4*>(kc);
                    c.kw[i][j][1] = *reinterpret_cast<const u32x4*>(kc + 8);
                }
            }
        }
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
            const int64_t vrow = (((int64_t)pv * a.Hkv + g) * D + 16 * dt + n) * kBlockSize;
            if constexpr (FMT == kFmtFP8 || FMT == kFmtFP8QP) {
                c.vw[dt] = *reinterpret_cast<const u32x4*>(a.v_cache + vrow);
            } else {
                const uint16_t* vc = reinterpret_cast<const uint16_t*>(a.v_cache) + vrow;
                c.vw[dt][0] = *reinterpret_cast<const u32x4*>(vc);
                c.vw[dt][1] = *reinterpret_cast<const u32x4*>(vc + 8);
            }
        }
    }
}

// K operand of k-step (tile i, slice j, half hh): dims 64j + 16grp + 8hh .. +7
// of the tile's token row; bf16 for FP8 / BF16 caches, f16 for NVFP4 (codes
// times the group's E4M3 block scale, exact in f16).
template <int FMT>
using QkOperand = typename std::conditional<
    FMT == kFmtNVFP4, f16x8, typename std::conditional<FMT == kFmtFP8QP, long, bf16x8>::type>::type;

template <int D, int FMT>
__device__ __forceinline__ QkOperand<FMT> k_operand(const MfmaChunk<D, FMT>& c, int i, int j, int hh) {
    if constexpr (FMT == kFmtFP8QP) {
        return __builtin_bit_cast(long, u32x2{c.kw[i][j][2 * hh], c.kw[i][j][2 * hh + 1]});   // raw codes
    } else if constexpr (FMT == kFmtFP8) {
        return e4m3x8_to_bf16(c.kw[i][j][2 * hh], c.kw[i][j][2 * hh + 1]);
    } else if constexpr (FMT == kFmtBF16) {
        return __builtin_bit_cast(bf16x8, c.kw[i][j][hh]);
    } else {
        const int grp = (threadIdx.x & 63) >> 4;   // the lane's 16-dim block within the 64-dim slice
        return e2m1x8_scaled_f16(c.kc[i][j][hh], e4m3x2_to_f16(c.ks[i][j] >> (8 * grp), false)[0]);
    }
}

// V operand of (dim tile dt, half hh) as f16: tokens 8hh .. 8hh+7 of the lane's dim.
template <int D, int FMT>
__device__ __forceinline__ f16x8 v_operand_f16(const MfmaChunk<D, FMT>& c, int dt, int hh) {
    if constexpr (FMT == kFmtFP8) {
        return e4m3x8_to_f16(c.vw[dt][2 * hh], c.vw[dt][2 * hh + 1]);
    } else {
        // E2M1 codes times each token's own block scale (exact in f16)
        const uint32_t w = c.vc[dt][hh];
        const f16x2 v0 = e2m1x2_to_f16<0>(w), v1 = e2m1x2_to_f16<1>(w);
        const f16x2 v2 = e2m1x2_to_f16<2>(w), v3 = e2m1x2_to_f16<3>(w);
        const f16x2 s0 = e4m3x2_to_f16(c.vs[dt][2 * hh], false), s1 = e4m3x2_to_f16(c.vs[dt][2 * hh], true);
        const f16x2 s2 = e4m3x2_to_f16(c.vs[dt][2 * hh + 1], false), s3 = e4m3x2_to_f16(c.vs[dt][2 * hh + 1], true);
        const f16x2 p0 = v0 * s0, p1 = v1 * s1, p2 = v2 * s2, p3 = v3 * s3;
        return f16x8{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
    }
}

// One 64-token chunk for all NT column tiles: K and V are unpacked once and
// shared by the tiles.  This lane's column in tile nt sees tokens
// [cbeg[nt], cend[nt]) (cbeg 0 and cend = tok_end for single-token decode
// without a window).  Chunks in [head_until, tail_from) need no masking;
// V data of tokens outside [vbeg, tok_end) is zeroed.
template <int D, int FMT, int NT>
__device__ __forceinline__ void mfma_process(MfmaState<D, NT>& st, MfmaChunk<D, FMT>& c,
                                             const QkOperand<FMT> (*qb)[2 * (D / 64)], const float* cs,
                                             const int* cbeg, const int* cend, int chunk_tok, int tok_end,
                                             int tail_from, int head_until, int vbeg, int grp) {
    constexpr int KJ = D / 64, DT = D / 16;
    constexpr bool kF16V = FMT != kFmtBF16;   // V operand in f16 (FP8, NVFP4) or bf16
    // ---- S = K Q^T ---------------------------------------------------------
    float sv[NT][16];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        f32x4 t[NT];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) t[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < KJ; ++j)
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                const QkOperand<FMT> ka = k_operand(c, i, j, hh);
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) {
                    if constexpr (FMT == kFmtNVFP4)
                        t[nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ka, qb[nt][2 * j + hh], t[nt], 0, 0, 0);
                    else
                        t[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, qb[nt][2 * j + hh], t[nt], 0, 0, 0);
                }
            }
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
            for (int r = 0; r < 4; ++r) sv[nt][4 * i + r] = t[nt][r];   // raw scores; scaled inside the exp
    }

    // ---- online softmax over this chunk (column n, chunk block grp) ---------
    // The score scale cs (> 0) is applied as exp2(fma(s, cs, -m)); the running
    // max m is kept in scaled units.  Masking runs only on chunks that reach a
    // column's end (a wave-uniform branch).  A column that has seen no token
    // yet keeps m = -inf; its weights are 0 (and its acc and l are still 0).
    const bool tail = chunk_tok + kChunkTokens > tail_from || chunk_tok < head_until;
    const int tok0 = chunk_tok + 16 * grp;   // token of sv[.][0]
    f16x8 pfh[NT][2], pfl[NT][2];
    bf16x8 pbh[NT][2], pbl[NT][2];
    float alpha[NT];
    // Lazy rescale (FP8 and BF16): a column's reference max m stays until the
    // chunk max exceeds it by more than kLazy (log2 units), so most chunks
    // skip the accumulator rescale; the weights' exp2 offset is 15 - kLazy, so
    // they still stay below 2^15.  The arithmetic is per column and the same
    // for every tile count, so a row's result does not depend on how many
    // queries share the launch.  NVFP4 (VALU-bound at one tile) keeps the
    // exact-max update (kLazy = 0: bitwise the plain online softmax).
    constexpr float kLazy = FMT == kFmtNVFP4 ? 0.0f : 8.0f;
    bool rescale = false;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        if (tail) {
            const int lo = cbeg[nt] - tok0, hi = cend[nt] - tok0;   // offsets of block grp this column sees
#pragma unroll
            for (int e = 0; e < 16; ++e)  // sv[4i + r] is token offset 4i + r of block grp
                if (e >= hi || e < lo) sv[nt][e] = -INFINITY;
        }
        float mloc = sv[nt][0];
#pragma unroll
        for (int e = 1; e < 16; ++e) mloc = fmaxf(mloc, sv[nt][e]);
        mloc = max_xor32(max_xor16(mloc));
        const float m_new = fmaxf(st.m_run[nt], mloc * cs[nt]);
        const bool keep = m_new <= st.m_run[nt] + kLazy;
        const float m_ref = keep ? st.m_run[nt] : m_new;
        const float m_use = m_ref == -INFINITY ? 0.f : m_ref;
        alpha[nt] = keep ? 1.f : fast_exp2(st.m_run[nt] - m_use);
        rescale = rescale || !keep;
        st.m_run[nt] = m_ref;

        // Weights in the PV operand layout (half hh = tokens 8hh..8hh+7).  They
        // are scaled by 2^(15 - kLazy) (exp2 offset; at most 2^15 over the
        // reference) so they sit in f16's normal range,
        // and split into hi + lo 16-bit parts so the two PV MFMAs on the same
        // exact V operand reproduce the fp32 weight to ~2^-21.  The scale is
        // common to acc and l and cancels in the final division.
        const float m_off = m_use - (15.0f - kLazy);
        // lo = p - hi is exact in fp32 (hi is p truncated to 11 bits), so an
        // fma with -1 gives the same bits as the subtraction; with the -1 in a
        // register the compiler takes hi straight from its f16 half
        // (v_fma_mix_f32) instead of converting it first
        float neg_one;
        asm("v_mov_b32 %0, -1.0" : "=v"(neg_one));
        float psum = 0.f;
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
#pragma unroll
            for (int e2 = 0; e2 < 4; ++e2) {
                const float p0 = fast_exp2(__builtin_fmaf(sv[nt][8 * hh + 2 * e2], cs[nt], -m_off));
                const float p1 = fast_exp2(__builtin_fmaf(sv[nt][8 * hh + 2 * e2 + 1], cs[nt], -m_off));
                psum += p0 + p1;
                if constexpr (kF16V) {
                    const f16x2 h = __builtin_bit_cast(f16x2, __builtin_amdgcn_cvt_pkrtz(p0, p1));
                    const f16x2 l = __builtin_bit_cast(
                        f16x2, __builtin_amdgcn_cvt_pkrtz(__builtin_fmaf((float)h[0], neg_one, p0),
                                                          __builtin_fmaf((float)h[1], neg_one, p1)));
                    pfh[nt][hh][2 * e2] = h[0];
                    pfh[nt][hh][2 * e2 + 1] = h[1];
                    pfl[nt][hh][2 * e2] = l[0];
                    pfl[nt][hh][2 * e2 + 1] = l[1];
                } else {
                    const __bf16 h0 = (__bf16)p0, h1 = (__bf16)p1;
                    pbh[nt][hh][2 * e2] = h0;
                    pbh[nt][hh][2 * e2 + 1] = h1;
                    pbl[nt][hh][2 * e2] = (__bf16)(p0 - (float)h0);
                    pbl[nt][hh][2 * e2 + 1] = (__bf16)(p1 - (float)h1);
                }
            }
        }
        st.l_run[nt] = st.l_run[nt] * alpha[nt] + psum;
    }

    // Zero V data of tokens past the sequence end and before the window: their
    // weight is 0 but the bytes may be anything (unwritten slots, or another
    // block's data through the clamped block ids).  FP8: V bytes; NVFP4: the
    // tokens' block scales (the E2M1 codes are always finite); BF16: V
    // halfwords.  Tokens inside [vbeg, tok_end) but outside a column's range
    // are finite; their weight is 0.
    if (chunk_tok + kChunkTokens > tok_end || chunk_tok < vbeg) {
        const int valid = tok_end - tok0, vlo = vbeg - tok0;
        if constexpr (FMT == kFmtBF16) {
            u32x4 keep[2];
#pragma unroll
            for (int x = 0; x < 2; ++x)
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    uint32_t mask = 0;
#pragma unroll
                    for (int e = 0; e < 2; ++e)
                        if (8 * x + 2 * w + e < valid && 8 * x + 2 * w + e >= vlo) mask |= 0xFFFFu << (16 * e);
                    keep[x][w] = mask;
                }
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) {
                c.vw[dt][0] &= keep[0];
                c.vw[dt][1] &= keep[1];
            }
        } else {
            u32x4 keep;   // word w holds tokens 4w .. 4w+3, one byte each
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                uint32_t mask = 0;
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (4 * w + e < valid && 4 * w + e >= vlo) mask |= 0xFFu << (8 * e);
                keep[w] = mask;
            }
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) {
                if constexpr (FMT == kFmtFP8)
                    c.vw[dt] &= keep;
                else
                    c.vs[dt] &= keep;
            }
        }
    }

    // ---- acc = alpha * acc + V^T P^T ----------------------------------------
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
        // (one tile or NVFP4: unconditional; the multiply by alpha = 1 is exact)
        if (NT == 1 || FMT == kFmtNVFP4 || __builtin_amdgcn_ballot_w64(rescale) != 0) {
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) st.acc[nt][dt] *= alpha[nt];
        }
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
            if constexpr (kF16V) {
                const f16x8 va = v_operand_f16(c, dt, hh);
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) {
                    st.acc[nt][dt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(va, pfh[nt][hh], st.acc[nt][dt], 0, 0, 0);
                    st.acc[nt][dt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(va, pfl[nt][hh], st.acc[nt][dt], 0, 0, 0);
                }
            } else {
                const bf16x8 va = __builtin_bit_cast(bf16x8, c.vw[dt][hh]);
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) {
                    st.acc[nt][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pbh[nt][hh], st.acc[nt][dt], 0, 0, 0);
                    st.acc[nt][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pbl[nt][hh], st.acc[nt][dt], 0, 0, 0);
                }
            }
        }
    }
}

// FP8 Q and P: one 64-token chunk on v_mfma_f32_16x16x32_fp8_fp8 with the raw
// K and V bytes as operands.  The softmax reference R is an integer (in log2
// units), so each rescale is an exact power of two and the P codes
// E4M3(448 * 2^(x - R)) do not depend on the chunk order (up to E4M3
// subnormals, which round more finely against a lower reference).  l is the
// column sum of the P codes, taken with one MFMA against an all-ones A
// operand, so every lane holds its column's whole sum.  The FP8 dot steps
// round their multi-product sums (the ISA states no bound), so scores and
// sums are close to, not equal to, their exact values; a weight near an
// E4M3 midpoint may take either neighbouring code.
template <int D, int NT>
__device__ __forceinline__ void mfma_process_qp8(MfmaState<D, NT>& st, MfmaChunk<D, kFmtFP8QP>& c,
                                                 const long (*qb)[2 * (D / 64)], float cs, const int* cbeg,
                                                 const int* cend, int chunk_tok, int tok_end, int tail_from,
                                                 int head_until, int vbeg, int grp) {
    constexpr int KJ = D / 64, DT = D / 16;
    float sv[NT][16];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        f32x4 t[NT];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) t[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < KJ; ++j)
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                const long ka = k_operand(c, i, j, hh);
#pragma unroll
                for (int nt = 0; nt < NT; ++nt)
                    t[nt] = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(ka, qb[nt][2 * j + hh], t[nt], 0, 0, 0);
            }
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
            for (int r = 0; r < 4; ++r) sv[nt][4 * i + r] = t[nt][r];
    }
    const bool tail = chunk_tok + kChunkTokens > tail_from || chunk_tok < head_until;
    const int tok0 = chunk_tok + 16 * grp;
    constexpr long kOnes = 0x3838383838383838L;   // eight E4M3 1.0
    long pq[NT][2];
    float alpha[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        if (tail) {
            const int lo = cbeg[nt] - tok0, hi = cend[nt] - tok0;
#pragma unroll
            for (int e = 0; e < 16; ++e)
                if (e >= hi || e < lo) sv[nt][e] = -INFINITY;
        }
        float mloc = sv[nt][0];
#pragma unroll
        for (int e = 1; e < 16; ++e) mloc = fmaxf(mloc, sv[nt][e]);
        mloc = max_xor32(max_xor16(mloc));
        const float r_new = fmaxf(st.m_run[nt], __builtin_ceilf(mloc * cs));   // integer-valued
        const float r_use = r_new == -INFINITY ? 0.f : r_new;
        alpha[nt] = st.m_run[nt] == -INFINITY ? 0.f : __builtin_ldexpf(1.0f, (int)(st.m_run[nt] - r_use));
        st.m_run[nt] = r_new;
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
            u32x2 w;
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                float y[4];
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    y[e] = 448.0f * fast_exp2(__builtin_fmaf(sv[nt][8 * hh + 4 * q + e], cs, -r_use));
                // y <= 448 up to one fp32 rounding of the reference (448.00003 rounds
                // to 448): round to nearest even, no saturation or NaN to handle
                uint32_t lo16 = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], 0, false) & 0xFFFFu;
                w[q] = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], (int)lo16, true);
            }
            pq[nt][hh] = __builtin_bit_cast(long, w);
        }
        f32x4 ls = {0.f, 0.f, 0.f, 0.f};
        ls = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(kOnes, pq[nt][0], ls, 0, 0, 0);
        ls = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(kOnes, pq[nt][1], ls, 0, 0, 0);
        st.l_run[nt] = st.l_run[nt] * alpha[nt] + ls[0];
    }
    if (chunk_tok + kChunkTokens > tok_end || chunk_tok < vbeg) {
        const int valid = tok_end - tok0, vlo = vbeg - tok0;
        u32x4 keep;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            uint32_t mask = 0;
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (4 * w + e < valid && 4 * w + e >= vlo) mask |= 0xFFu << (8 * e);
            keep[w] = mask;
        }
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) c.vw[dt] &= keep;
    }
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) st.acc[nt][dt] *= alpha[nt];
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
            const long va = __builtin_bit_cast(long, u32x2{c.vw[dt][2 * hh], c.vw[dt][2 * hh + 1]});
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
                st.acc[nt][dt] = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(va, pq[nt][hh], st.acc[nt][dt], 0, 0, 0);
        }
    }
}

template <int D, int FMT, int NT>
__device__ __forceinline__ void process_chunk(MfmaState<D, NT>& st, MfmaChunk<D, FMT>& c,
                                              const QkOperand<FMT> (*qb)[2 * (D / 64)], const float* cs,
                                              const int* cbeg, const int* cend, int chunk_tok, int tok_end,
                                              int tail_from, int head_until, int vbeg, int grp) {
    if constexpr (FMT == kFmtFP8QP)
        mfma_process_qp8(st, c, qb, cs[0], cbeg, cend, chunk_tok, tok_end, tail_from, head_until, vbeg, grp);
    else
        mfma_process(st, c, qb, cs, cbeg, cend, chunk_tok, tok_end, tail_from, head_until, vbeg, grp);
}

// Orders this wave's cache stores before its later loads of the same bytes:
// a work-group-scope fence, plus an explicit wait for every outstanding
// memory operation of the wave (stores included), so the stores have reached
// L2 before the chunk's loads are issued.  No other wave has loaded those
// lines in this kernel, so the loads cannot hit a stale L1 copy.  Waiting here
// costs nothing measurable: the only loads still in flight are the previous
// chunk's, which the wave needs next anyway.
__device__ __forceinline__ void append_fence() {
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
    __builtin_amdgcn_s_waitcnt(0);
}

// APPEND: the fused cache write of the new tokens (kvq_paged_decode_attn_append:
// each sequence's newest token, kAppendOne; kvq_paged_decode_attn_mq_append:
// its q_len newest, kAppendMany).  A new token's block is read by one
// work-group only, the one holding the split with that token for this KV
// head, and within it by the wave whose round-robin share ends with the
// chunk holding that token.  That wave quantizes the token and stores it
// right after its block ids are staged, and before it loads that chunk it
// waits for its own stores (a work-group-scope fence), so the chunk's loads
// see the new bytes.  The one-token case has a kernel of its own: the
// general writer costs the decode step about 0.2 us at D 64.
constexpr int kAppendNone = 0, kAppendOne = 1, kAppendMany = 2;

template <int D, int FMT, int NT, int W = mfma_waves<D, FMT, NT>(), int APPEND = kAppendNone>
__global__ void __launch_bounds__(W * 64) decode_mfma_kernel(DecodeArgs a) {
    constexpr int KJ = D / 64;
    constexpr int DT = D / 16;
    constexpr int CP = 16 * NT;   // padded columns
    // two chunks in flight per wave where the registers allow it (measured
    // faster than one for every D <= 128 shape, single and multi-query; a
    // ring of three or four chunks was measured slower at D 64)
    constexpr bool kPrefetch = D <= 128;
    extern __shared__ float lds[];
    int* s_blk = reinterpret_cast<int*>(lds);
    float* s_m = lds + kMaxSplitBlocks;
    float* s_l = s_m + W * CP;
    float* s_acc = s_l + W * CP;

    const int s = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
    KVQ_TRACE_DECL;
    KVQ_TRACE_MARK(0);
    const SeqRange sr = seq_range(a, b);
    const int L = sr.L;
    const int tok_begin = sr.base + s * a.split_tokens;
    if (tok_begin >= L) {
        if (L <= 0 && s == 0) write_empty(a, b, g, D);
        return;
    }
    KVQ_TRACE_MARK(1);
    const int tok_end = min(L, tok_begin + a.split_tokens);
    const int S = (L - sr.base + a.split_tokens - 1) / a.split_tokens;   // splits holding tokens
    // the wave index as a scalar: every per-wave loop bound below is then uniform,
    // so its loops branch on SCC instead of masking exec (a masked loop keeps the
    // prefetch of its last pass live into the header, which then drains all loads)
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int n = lane & 15, grp = lane >> 4;
    const int G = a.G, GQ = G * a.q_len;

    const int lb0 = tok_begin / kBlockSize;
    const int n_chunks = (tok_end - tok_begin + kChunkTokens - 1) / kChunkTokens;
    // Fused append.  kAppendOne (a decode step: each sequence's newest token):
    // the wave owning the split's last chunk writes it, one row over the
    // wave's lanes.  kAppendMany (a verification step: the q_len new tokens,
    // positions L - q_len .. L - 1 that are >= 0): they lie in the split's
    // last two chunks at most (q_len <= 16 < 64), each chunk's tokens written
    // by the wave owning that chunk, this wave's being [new_lo, new_hi).  For
    // W >= 2 a written chunk is its wave's last, so the wave writes before that
    // chunk's first load (append_fence).  The bf16 rows are loaded here, in
    // flight with the block-id staging, and stored after it.
    int new_lo = 0, new_hi = 0;
    if constexpr (APPEND == kAppendMany) {
        const int p0 = max(max(L - a.q_len, 0), tok_begin);   // new tokens of this split: [p0, tok_end)
        if (p0 < tok_end) {
            const int c0 = (p0 - tok_begin) / kChunkTokens, c1 = (tok_end - 1 - tok_begin) / kChunkTokens;
            const int c = c0 % W == wave ? c0 : (c1 % W == wave ? c1 : -1);
            if (c >= 0) {
                new_lo = max(p0, tok_begin + c * kChunkTokens);
                new_hi = min(tok_end, tok_begin + (c + 1) * kChunkTokens);
            }
        }
    }
    const bool writer = APPEND == kAppendOne ? tok_end == L && wave == (n_chunks - 1) % W
                                             : APPEND == kAppendMany && new_lo < new_hi;
    constexpr int NG = D / 16;                 // NVFP4 blocks per (token, head) row
    uint16_t k_one[D / 64], v_one[D / 64];     // kAppendOne, FP8 / BF16: dims lane + 64 r
    u32x4 n_w0 = {}, n_w1 = {};                // kAppendOne, NVFP4: lane < NG: K block lane; lane < 2 NG: V block
    int64_t new_slot = -1;                     // kAppendOne
    // kAppendMany: token new_lo + k, dims [E lane, E lane + E) of its row (kE
    // 32-bit words; at D 64 the aligned pair holding the lane's dim); lane
    // t < new_hi - new_lo holds token new_lo + t's slot
    constexpr int E = D / 64, kE = (E + 1) / 2, kMany = APPEND == kAppendMany ? kMaxQueryLen : 1;
    uint32_t nk[kMany][kE], nv[kMany][kE];
    int64_t ns = -1;
    if constexpr (APPEND == kAppendOne) {
        if (writer) {
            new_slot = a.new_slots[b];
            if (KVQ_CHECK && new_slot >= (int64_t)a.num_blocks * kBlockSize) {
                check_fail(kCheckSlot);
                new_slot = -1;
            }
            const int64_t row = (int64_t)b * a.new_stride + (int64_t)g * D;
            if constexpr (FMT == kFmtNVFP4) {
                if (lane < 2 * NG) {
                    const uint16_t* src = (lane < NG ? a.k_new : a.v_new) + row + 16 * (lane % NG);
                    n_w0 = *reinterpret_cast<const u32x4*>(src);
                    n_w1 = *reinterpret_cast<const u32x4*>(src + 8);
                }
            } else {
#pragma unroll
                for (int r = 0; r < D / 64; ++r) {
                    k_one[r] = a.k_new[row + lane + 64 * r];
                    v_one[r] = a.v_new[row + lane + 64 * r];
                }
            }
        }
    } else if constexpr (APPEND == kAppendMany) {
        if (writer) {
            const int i0 = new_lo - (L - a.q_len);   // index of token new_lo among the q_len new tokens
            if (lane < new_hi - new_lo) {
                ns = a.new_slots[(int64_t)b * a.q_len + i0 + lane];
                if (KVQ_CHECK && ns >= (int64_t)a.num_blocks * kBlockSize) {
                    check_fail(kCheckSlot);
                    ns = -1;
                }
            }
#pragma unroll
            for (int k = 0; k < kMany; ++k) {
                if (k < new_hi - new_lo) {
                    const int64_t row = ((int64_t)b * a.q_len + i0 + k) * a.new_stride + (int64_t)g * D + E * lane;
                    if constexpr (E == 1) {
                        nk[k][0] = *reinterpret_cast<const uint32_t*>(a.k_new + (row & ~(int64_t)1));
                        nv[k][0] = *reinterpret_cast<const uint32_t*>(a.v_new + (row & ~(int64_t)1));
                    } else if constexpr (E == 2) {
                        nk[k][0] = *reinterpret_cast<const uint32_t*>(a.k_new + row);
                        nv[k][0] = *reinterpret_cast<const uint32_t*>(a.v_new + row);
                    } else {
                        static_assert(E == 4, "D is 64, 128 or 256");
                        const u32x2 kw = *reinterpret_cast<const u32x2*>(a.k_new + row);
                        const u32x2 vw = *reinterpret_cast<const u32x2*>(a.v_new + row);
                        nk[k][0] = kw[0], nk[k][1] = kw[1];
                        nv[k][0] = vw[0], nv[k][1] = vw[1];
                    }
                }
            }
        }
    }
    // this wave's chunks: wave, wave + W, ...; each wave stages the block ids of
    // its own chunks only, so no barrier is needed before its loads
    const int my = wave < n_chunks ? (n_chunks - wave + W - 1) / W : 0;
    {
        const int32_t* bt_row = a.block_tables + (int64_t)b * a.max_blocks;
        const int first_lb = sr.first / kBlockSize, last_lb = (L + kBlockSize - 1) / kBlockSize - 1;
        for (int i = lane; i < 4 * my; i += 64) {
            const int e = 4 * (wave + W * (i >> 2)) + (i & 3);   // entry of chunk wave + W * (i / 4)
            int id = bt_row[min(max(lb0 + e, first_lb), last_lb)];
            if (KVQ_CHECK && (unsigned)id >= (unsigned)a.num_blocks) {
                check_fail(kCheckBlockId);
                id = 0;
            }
            s_blk[e] = id;
        }
    }

    // Query i (token L - q_len + i) sees tokens [cbeg, cend): cend = that
    // token + 1, cbeg = cend - window (or 0).
    const int q0_end = L - a.q_len + 1;
    int cbeg[NT], cend[NT];
    // Q^T operands per tile: k-step (j, hh) covers dims 64j + 16grp + 8hh .. +7
    // of column 16 nt + n (zero past GQ).  For NVFP4 the QK product runs in
    // f16: the column's q is scaled by a power of two 2^qs (max |q| lands in
    // [2^13, 2^14), far inside f16's range; the conversion is exact for every
    // element within 2^27 of the max) and its score scale is divided by the
    // same power of two.
    QkOperand<FMT> qb[NT][2 * KJ];
    float cs[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        const int c = 16 * nt + n;
        const bool live = c < GQ;
        const int qi = live ? c / G : 0;
        cend[nt] = live ? min(tok_end, q0_end + qi) : tok_end;
        cbeg[nt] = live && a.window > 0 ? max(0, q0_end + qi - a.window) : 0;
        const uint16_t* qrow = a.q + (live ? column_row(a, b, g, c) : 0) * D;
        u32x4 qw[2 * KJ];
#pragma unroll
        for (int j = 0; j < KJ; ++j)
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                u32x4 w = {0u, 0u, 0u, 0u};
                if (live) w = *reinterpret_cast<const u32x4*>(qrow + 64 * j + 16 * grp + 8 * hh);
                qw[2 * j + hh] = w;
            }
        cs[nt] = a.qk_scale_log2;
        if constexpr (FMT == kFmtFP8QP) {
            // q codes E4M3(fp32(q) / q_scale), the cache write's quantizer
#pragma clang fp contract(off)
#pragma unroll
            for (int k = 0; k < 2 * KJ; ++k) {
                u32x2 wc;
#pragma unroll
                for (int h2 = 0; h2 < 2; ++h2)
                    wc[h2] = e4m3_encode4(bf16_lo(qw[k][2 * h2]) / a.q_scale, bf16_hi(qw[k][2 * h2]) / a.q_scale,
                                          bf16_lo(qw[k][2 * h2 + 1]) / a.q_scale,
                                          bf16_hi(qw[k][2 * h2 + 1]) / a.q_scale);
                qb[nt][k] = live ? __builtin_bit_cast(long, wc) : 0L;
            }
        } else if constexpr (FMT == kFmtNVFP4) {
            float qmax = 0.f;
#pragma unroll
            for (int k = 0; k < 2 * KJ; ++k)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    qmax = fmaxf(qmax, fmaxf(__builtin_fabsf(bf16_lo(qw[k][e])), __builtin_fabsf(bf16_hi(qw[k][e]))));
            qmax = max_xor32(max_xor16(qmax));
            // exponent of qmax: qmax = m * 2^ex with m in [0.5, 1)
            const int ex = qmax > 0.f ? __builtin_amdgcn_frexp_expf(qmax) : 0;
            const int qs = min(14 - ex, 100);   // denormal-only rows stay finite
            const float up = __builtin_ldexpf(1.0f, qs);
            cs[nt] = __builtin_ldexpf(cs[nt], -qs);
#pragma unroll
            for (int k = 0; k < 2 * KJ; ++k) {
                f16x8 v;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    v[2 * e] = (_Float16)(bf16_lo(qw[k][e]) * up);
                    v[2 * e + 1] = (_Float16)(bf16_hi(qw[k][e]) * up);
                }
                qb[nt][k] = v;
            }
        } else {
#pragma unroll
            for (int k = 0; k < 2 * KJ; ++k) qb[nt][k] = __builtin_bit_cast(bf16x8, qw[k]);
        }
    }
    const int tail_from = min(tok_end, q0_end);
    const int head_until = a.window > 0 ? max(0, L - a.window) : 0;   // the newest query's window start
    KVQ_TRACE_MARK(2, false);
    if constexpr (APPEND) {
        uint8_t* kc = const_cast<uint8_t*>(a.k_cache);
        uint8_t* vc = const_cast<uint8_t*>(a.v_cache);
        if constexpr (FMT == kFmtNVFP4) {
            if (writer && new_slot >= 0) {   // the cache write's quantizer
                const int64_t blk = new_slot / kBlockSize;
                const int off = (int)(new_slot - blk * kBlockSize);
                // one lane per block: K codes are a whole token row; a V code byte holds
                // this token's nibble and the other slot's of the pair, which this
                // work-group alone touches in the call, so it is read, merged and stored
                constexpr int64_t region = 9 * D, code_bytes = 8 * D;
                if (lane < 2 * NG) {
                    const int gb = lane % NG;
                    uint32_t codes[16], bcode;
                    nvfp4_quantize_group(n_w0, n_w1, lane < NG ? a.k_scale_w : a.v_scale_w, codes, &bcode);
                    if (lane < NG) {
                        uint8_t* kr = kc + (blk * a.Hkv + g) * region;
                        u32x2 packed = {0u, 0u};
#pragma unroll
                        for (int j = 0; j < 16; ++j) packed[j >> 3] |= codes[j] << (4 * (j & 7));
                        *reinterpret_cast<u32x2*>(kr + (int64_t)off * (D / 2) + gb * 8) = packed;
                        kr[code_bytes + (int64_t)off * NG + gb] = (uint8_t)bcode;
                    } else {
                        uint8_t* vr = vc + (blk * a.Hkv + g) * region;
                        vr[code_bytes + (int64_t)gb * kBlockSize + off] = (uint8_t)bcode;
                        const uint32_t sh = 4u * (uint32_t)(off & 1);
#pragma unroll
                        for (int j = 0; j < 16; ++j) {
                            uint8_t* pb = vr + (int64_t)(16 * gb + j) * (kBlockSize / 2) + (off >> 1);
                            *pb = (uint8_t)(((uint32_t)*pb & ~(0xFu << sh)) | (codes[j] << sh));
                        }
                    }
                }
            }
        } else if constexpr (APPEND == kAppendOne) {
            if (writer && new_slot >= 0) {   // the cache write's quantizer, element by element
                const int64_t blk = new_slot / kBlockSize;
                const int off = (int)(new_slot - blk * kBlockSize);
#pragma unroll
                for (int r = 0; r < D / 64; ++r) {
                    const int d = lane + 64 * r;
                    const int64_t ki = ((blk * a.Hkv + g) * kBlockSize + off) * D + d;   // [blk][g][off][d]
                    const int64_t vi = ((blk * a.Hkv + g) * D + d) * kBlockSize + off;   // [blk][g][d][off]
                    if constexpr (FMT == kFmtFP8) {
#pragma clang fp contract(off)
                        kc[ki] = (uint8_t)e4m3_encode(bits_f32((uint32_t)k_one[r] << 16) / a.k_scale_w);
                        vc[vi] = (uint8_t)e4m3_encode(bits_f32((uint32_t)v_one[r] << 16) / a.v_scale_w);
                    } else {
                        reinterpret_cast<uint16_t*>(kc)[ki] = k_one[r];
                        reinterpret_cast<uint16_t*>(vc)[vi] = v_one[r];
                    }
                }
            }
        } else if (writer) {
            // the same quantizer: K rows [blk][g][off][d] take this lane's E
            // contiguous dims, V columns [blk][g][d][off] one element per dim.
            // One wait for the rows and slots first (vmcnt 0, the other counters
            // untouched), on every path into the loop: otherwise each token's
            // first use waits there, and with the previous token's stores then
            // outstanding that wait is a full write round trip per token
            __builtin_amdgcn_s_waitcnt(0x0F70);
#pragma unroll
            for (int k = 0; k < kMany; ++k) {
                if (k < new_hi - new_lo) {
                    const uint32_t s_lo = __builtin_amdgcn_readlane((uint32_t)ns, k);
                    const uint32_t s_hi = __builtin_amdgcn_readlane((uint32_t)((uint64_t)ns >> 32), k);
                    const int64_t slot = (int64_t)(((uint64_t)s_hi << 32) | s_lo);
                    if (slot >= 0) {
                        const int64_t blk = slot / kBlockSize;
                        const int off = (int)(slot - blk * kBlockSize);
                        const int64_t ki = ((blk * a.Hkv + g) * kBlockSize + off) * D + E * lane;
                        const int64_t vi = ((blk * a.Hkv + g) * D + E * lane) * kBlockSize + off;
                        // this lane's E values: bf16 halves of its words (at D 64 the
                        // half of the pair that holds its dim)
                        uint32_t kh[E], vh[E];
#pragma unroll
                        for (int j = 0; j < E; ++j) {
                            const bool hi = (E == 1 ? lane : j) & 1;
                            kh[j] = hi ? nk[k][j / 2] >> 16 : nk[k][j / 2] & 0xFFFFu;
                            vh[j] = hi ? nv[k][j / 2] >> 16 : nv[k][j / 2] & 0xFFFFu;
                        }
                        if constexpr (FMT == kFmtFP8) {
#pragma clang fp contract(off)
                            uint32_t kb[E];
#pragma unroll
                            for (int j = 0; j < E; ++j) {
                                kb[j] = e4m3_encode(bits_f32(kh[j] << 16) / a.k_scale_w);
                                vc[vi + (int64_t)j * kBlockSize] = (uint8_t)e4m3_encode(bits_f32(vh[j] << 16) / a.v_scale_w);
                            }
                            if constexpr (E == 1) {
                                kc[ki] = (uint8_t)kb[0];
                            } else if constexpr (E == 2) {
                                *reinterpret_cast<uint16_t*>(kc + ki) = (uint16_t)(kb[0] | kb[1] << 8);
                            } else {
                                *reinterpret_cast<uint32_t*>(kc + ki) = kb[0] | kb[1] << 8 | kb[2] << 16 | kb[3] << 24;
                            }
                        } else {
                            uint16_t* k16 = reinterpret_cast<uint16_t*>(kc);
                            uint16_t* v16 = reinterpret_cast<uint16_t*>(vc);
                            if constexpr (E == 1) {
                                k16[ki] = (uint16_t)kh[0];
                            } else if constexpr (E == 2) {
                                *reinterpret_cast<uint32_t*>(k16 + ki) = nk[k][0];
                            } else {
                                *reinterpret_cast<u32x2*>(k16 + ki) = u32x2{nk[k][0], nk[k][1]};
                            }
#pragma unroll
                            for (int j = 0; j < E; ++j) v16[vi + (int64_t)j * kBlockSize] = (uint16_t)vh[j];
                        }
                    }
                }
            }
        }
    }

    MfmaState<D, NT> st;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) st.acc[nt][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
        st.m_run[nt] = -INFINITY;
        st.l_run[nt] = 0.f;
    }
    if constexpr (kPrefetch) {
        // Software pipeline: the next chunk's loads are in flight while the
        // current one is computed.  The prefetch is unconditional so wait
        // counts stay static: past a wave's last chunk it re-issues that
        // chunk's addresses (L2 hits; the registers are never read).  A pass
        // takes two chunks and has no exit inside it, so every path back to
        // the loop header has consumed the pass's first prefetch; an odd last
        // chunk is computed after the loop.
        MfmaChunk<D, FMT> A, Bc;
        if (my > 0) {
            int ch = wave;
            if (APPEND && writer && my == 1) append_fence();
            mfma_load(A, a, s_blk, ch, g, n, grp);
            for (int i = 0; i + 1 < my; i += 2) {
                const int chb = ch + W;
                if (APPEND && writer && i + 2 == my) append_fence();
                mfma_load(Bc, a, s_blk, chb, g, n, grp);
                // issue the prefetch before any of the current chunk's math: the
                // first conversion waits on the current chunk's oldest load.  Only
                // for single-query tiles at D = 64, where a chunk's math is short;
                // elsewhere the fence costs registers (a spill with two BF16 tiles
                // at D = 128) or time (about 1.5% for FP8 at D = 128)
                if constexpr (NT == 1 && D == 64) __builtin_amdgcn_sched_barrier(0);
                process_chunk(st, A, qb, cs, cbeg, cend, tok_begin + ch * kChunkTokens, tok_end, tail_from,
                              head_until, sr.first, grp);
#if KVQ_TRACE
                if (i == 0) KVQ_TRACE_MARK(3, false);
#endif
                const int cha = i + 2 < my ? chb + W : chb;
                if (APPEND && writer && i + 3 == my) append_fence();
                mfma_load(A, a, s_blk, cha, g, n, grp);
                if constexpr (NT == 1 && D == 64) __builtin_amdgcn_sched_barrier(0);
                process_chunk(st, Bc, qb, cs, cbeg, cend, tok_begin + chb * kChunkTokens, tok_end, tail_from,
                              head_until, sr.first, grp);
                ch = cha;
            }
            if (my & 1) {
                process_chunk(st, A, qb, cs, cbeg, cend, tok_begin + ch * kChunkTokens, tok_end, tail_from,
                              head_until, sr.first, grp);
#if KVQ_TRACE
                if (my == 1) KVQ_TRACE_MARK(3, false);
#endif
            }
        }
    } else {
        for (int i = 0; i < my; ++i) {
            const int ch = wave + i * W;
            MfmaChunk<D, FMT> A;
            if (APPEND && writer && i + 1 == my) append_fence();
            mfma_load(A, a, s_blk, ch, g, n, grp);
            process_chunk(st, A, qb, cs, cbeg, cend, tok_begin + ch * kChunkTokens, tok_end, tail_from,
                          head_until, sr.first, grp);
#if KVQ_TRACE
            if (i == 0) KVQ_TRACE_MARK(3, false);
#endif
        }
    }
    KVQ_TRACE_MARK(4);

    // ---- wave results -> LDS ---------------------------------------------------
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        float l_run = st.l_run[nt];
        if constexpr (FMT != kFmtFP8QP) {   // (the FP8 Q/P path already holds whole column sums)
            l_run = sum_xor32(sum_xor16(l_run));
        }
        const int c = 16 * nt + n;
        if (grp == 0) {
            s_m[wave * CP + c] = st.m_run[nt];
            s_l[wave * CP + c] = l_run;
        }
        if (c < GQ) {
#pragma unroll
            for (int dt = 0; dt < DT; ++dt)
#pragma unroll
                for (int r = 0; r < 4; ++r) s_acc[(wave * GQ + c) * D + 16 * dt + 4 * grp + r] = st.acc[nt][dt][r];
        }
    }
    __syncthreads();
    finish_split<W, NT>(a, s_m, s_l, s_acc, b, g, s, S, D);
    KVQ_TRACE_MARK(5);
    KVQ_TRACE_STORE_DECODE(W, wave, lane, my, s, g, b);
}

// =============================================================================
// VALU family (comparator)
// =============================================================================
// Per wave iteration: one 16-token block.  QK: lane = (token off = lane/4,
// quarter qq = lane%4 of D); partial dots over D/4 dims with Q from LDS, quad
// reduction.  PV: lane = dim (D/64 dims per lane) over the dim-major V block,
// weights broadcast through LDS.
template <int D, bool FP8>
__global__ void __launch_bounds__(kThreads) decode_valu_kernel(DecodeArgs a) {
    constexpr int QD = D / 4;    // dims per lane in QK
    constexpr int VD = D / 64;   // dims per lane in PV
    constexpr int MAXG = 16;
    extern __shared__ float lds[];
    int* s_blk = reinterpret_cast<int*>(lds);
    float* s_m = lds + kMaxSplitBlocks;
    float* s_l = s_m + kWaves * 16;
    float* s_acc = s_l + kWaves * 16;
    const int G = a.G;
    float* s_q = s_acc + kWaves * G * D;         // [G][D]
    float* s_p = s_q + G * D;                    // [kWaves][16 heads][16 tokens]

    const int s = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
    const int L = seq_len(a, b);
    const int tok_begin = s * a.split_tokens;
    if (tok_begin >= L) {
        if (L <= 0 && s == 0) write_empty(a, b, g, D);
        return;
    }
    const int tok_end = min(L, tok_begin + a.split_tokens);
    const int S = (L + a.split_tokens - 1) / a.split_tokens;   // splits holding tokens
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int Hkv = a.Hkv;

    const int lb0 = tok_begin / kBlockSize;
    const int n_blocks = (tok_end - tok_begin + kBlockSize - 1) / kBlockSize;
    stage_block_ids(s_blk, a.block_tables + (int64_t)b * a.max_blocks, lb0, n_blocks, 0,
                    (L + kBlockSize - 1) / kBlockSize - 1, a.num_blocks);
    for (int i = threadIdx.x; i < G * D; i += kThreads) {
        const int h = i / D, d = i - h * D;
        s_q[i] = bits_f32((uint32_t)a.q[((int64_t)b * a.Hq + g * G + h) * D + d] << 16);
    }
    __syncthreads();

    const int off = lane >> 2, qq = lane & 3;
    float* my_p = s_p + wave * 256;
    float m_run[MAXG], l_run[MAXG], acc[MAXG][VD];
#pragma unroll
    for (int h = 0; h < MAXG; ++h) {
        m_run[h] = -INFINITY;
        l_run[h] = 0.f;
#pragma unroll
        for (int e = 0; e < VD; ++e) acc[h][e] = 0.f;
    }
    const float c = a.qk_scale_log2;

    for (int blk = wave; blk < n_blocks; blk += kWaves) {
        const int phys = s_blk[blk];
        const int valid = tok_end - (tok_begin + blk * kBlockSize);
        // K slice: QD elements of token `off`
        float kf[QD];
        {
            const int64_t row = (((int64_t)phys * Hkv + g) * kBlockSize + off) * D + qq * QD;
            if constexpr (FP8) {
#pragma unroll
                for (int x = 0; x < QD / 16; ++x) {
                    u32x4 w = *reinterpret_cast<const u32x4*>(a.k_cache + row + 16 * x);
#pragma unroll
                    for (int y = 0; y < 4; ++y) {
                        f32x2 lo = e4m3x2_to_f32(w[y], false), hi = e4m3x2_to_f32(w[y], true);
                        kf[16 * x + 4 * y + 0] = lo[0];
                        kf[16 * x + 4 * y + 1] = lo[1];
                        kf[16 * x + 4 * y + 2] = hi[0];
                        kf[16 * x + 4 * y + 3] = hi[1];
                    }
                }
            } else {
                const uint16_t* kc = reinterpret_cast<const uint16_t*>(a.k_cache);
#pragma unroll
                for (int x = 0; x < QD / 8; ++x) {
                    u32x4 w = *reinterpret_cast<const u32x4*>(kc + row + 8 * x);
#pragma unroll
                    for (int y = 0; y < 4; ++y) {
                        kf[8 * x + 2 * y] = bf16_lo(w[y]);
                        kf[8 * x + 2 * y + 1] = bf16_hi(w[y]);
                    }
                }
            }
        }
        // V^T rows: dims lane + 64e, 16 tokens each
        float vf[VD][16];
#pragma unroll
        for (int e = 0; e < VD; ++e) {
            const int64_t vrow = (((int64_t)phys * Hkv + g) * D + lane + 64 * e) * kBlockSize;
            if constexpr (FP8) {
                u32x4 w = *reinterpret_cast<const u32x4*>(a.v_cache + vrow);
#pragma unroll
                for (int y = 0; y < 4; ++y) {
                    f32x2 lo = e4m3x2_to_f32(w[y], false), hi = e4m3x2_to_f32(w[y], true);
                    vf[e][4 * y + 0] = lo[0];
                    vf[e][4 * y + 1] = lo[1];
                    vf[e][4 * y + 2] = hi[0];
                    vf[e][4 * y + 3] = hi[1];
                }
            } else {
                const uint16_t* vc = reinterpret_cast<const uint16_t*>(a.v_cache);
#pragma unroll
                for (int x = 0; x < 2; ++x) {
                    u32x4 w = *reinterpret_cast<const u32x4*>(vc + vrow + 8 * x);
#pragma unroll
                    for (int y = 0; y < 4; ++y) {
                        vf[e][8 * x + 2 * y] = bf16_lo(w[y]);
                        vf[e][8 * x + 2 * y + 1] = bf16_hi(w[y]);
                    }
                }
            }
#pragma unroll
            for (int t = 0; t < 16; ++t)
                if (t >= valid) vf[e][t] = 0.f;
        }

#pragma unroll
        for (int h = 0; h < MAXG; ++h) {
            if (h >= G) break;
            const float* qh = s_q + h * D + qq * QD;
            float part = 0.f;
#pragma unroll
            for (int x = 0; x < QD; x += 4) {
                const f32x4 qv = *reinterpret_cast<const f32x4*>(qh + x);
                part += qv[0] * kf[x] + qv[1] * kf[x + 1] + qv[2] * kf[x + 2] + qv[3] * kf[x + 3];
            }
            part += shfl_xor(part, 1);
            part += shfl_xor(part, 2);
            float sh = (off < valid) ? part * c : -INFINITY;
            float bm = sh;
            bm = fmaxf(bm, shfl_xor(bm, 4));
            bm = fmaxf(bm, shfl_xor(bm, 8));
            bm = fmaxf(bm, shfl_xor(bm, 16));
            bm = fmaxf(bm, shfl_xor(bm, 32));
            const float m_new = fmaxf(m_run[h], bm);
            const float alpha = fast_exp2(m_run[h] - m_new);
            m_run[h] = m_new;
            const float p = fast_exp2(sh - m_new);
            l_run[h] = l_run[h] * alpha + (qq == 0 ? p : 0.f);
            if (qq == 0) my_p[h * 16 + off] = p;
#pragma unroll
            for (int e = 0; e < VD; ++e) acc[h][e] *= alpha;
        }
        // weights written by this wave are read back by the same wave only
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
        for (int h = 0; h < MAXG; ++h) {
            if (h >= G) break;
            const float* ph = my_p + h * 16;
#pragma unroll
            for (int t = 0; t < 16; t += 4) {
                const f32x4 pv4 = *reinterpret_cast<const f32x4*>(ph + t);
#pragma unroll
                for (int e = 0; e < VD; ++e)
                    acc[h][e] += pv4[0] * vf[e][t] + pv4[1] * vf[e][t + 1] + pv4[2] * vf[e][t + 2] +
                                 pv4[3] * vf[e][t + 3];
            }
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }

#pragma unroll
    for (int h = 0; h < MAXG; ++h) {
        if (h >= G) break;
        float l = l_run[h];
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) l += shfl_xor(l, o);
        if (lane == 0) {
            s_m[wave * 16 + h] = m_run[h];
            s_l[wave * 16 + h] = l;
        }
#pragma unroll
        for (int e = 0; e < VD; ++e) s_acc[(wave * G + h) * D + lane + 64 * e] = acc[h][e];
    }
    __syncthreads();
    finish_split<kWaves, 1>(a, s_m, s_l, s_acc, b, g, s, S, D);
}

// =============================================================================
// cross-split merge: out = v_scale * sum_s 2^(m_s - M) acc_s / sum_s 2^(m_s - M) l_s
// =============================================================================
// One work-group per (sequence, query head) whose sequence has two or more
// splits.  Every load is issued up front (the first 4 partial rows per thread
// and the first 64 (m, l) pairs), so the merge costs about one memory round
// trip.  Wave 0 alone turns the (m, l) pairs into split weights and the
// final scale with cross-lane reductions (permlane swaps and DPP row
// rotations: no LDS round trips); after one barrier, P = 256 / (D/4) thread
// groups each sum every P-th split of one 4-dim column, and a second barrier
// joins the groups.
constexpr int kMergeThreads = 256;

// Rotation by K lanes within each row of 16 lanes (DPP row_ror:K).
template <int K>
__device__ __forceinline__ float row_ror(float v) {
    return bits_f32((uint32_t)__builtin_amdgcn_mov_dpp((int)f32_bits(v), 0x120 + K, 0xF, 0xF, false));
}
// Max / sum over the 64 lanes of a wave, in every lane.
__device__ __forceinline__ float wave_max(float v) {
    v = max_xor32(max_xor16(v));
    v = fmaxf(v, row_ror<8>(v));
    v = fmaxf(v, row_ror<4>(v));
    v = fmaxf(v, row_ror<2>(v));
    return fmaxf(v, row_ror<1>(v));
}
__device__ __forceinline__ float wave_sum(float v) {
    v = sum_xor32(sum_xor16(v));
    v += row_ror<8>(v);
    v += row_ror<4>(v);
    v += row_ror<2>(v);
    return v + row_ror<1>(v);
}

template <int D>
__global__ void __launch_bounds__(kMergeThreads) merge_splits_kernel(DecodeArgs a) {
    constexpr int C4 = D / 4;                 // float4 columns of a partial row
    constexpr int P = kMergeThreads / C4;     // split groups: 16, 8, 4 for D = 64, 128, 256
    constexpr int PRE = 4;                    // partial rows loaded up front per thread
    extern __shared__ float s_w[];            // [num_splits] split weights
    __shared__ float s_scale;
    __shared__ f32x4 part[P][C4];
    const int hq = blockIdx.x;                // output row (b * q_len + i) * Hq + h
    KVQ_TRACE_DECL;
    KVQ_TRACE_MARK(0);
    const int b = hq / (a.Hq * a.q_len);
    const int t = threadIdx.x;
    const int d4 = t % C4, p = t / C4;
    const int NS = a.num_splits;
    const float* ml = a.ws_ml + (int64_t)hq * NS * 2;
    const f32x4* col = reinterpret_cast<const f32x4*>(a.ws_acc + (int64_t)hq * NS * D) + d4;
    // The first partial rows and (m, l) pairs are loaded before the sequence
    // length is known (they lie inside the row's num_splits slots), so they
    // are in flight together with seq_lens[b]; slots of splits past the
    // sequence's last hold stale data and are masked once S is known.
    f32x4 pre[PRE];
#pragma unroll
    for (int k = 0; k < PRE; ++k) {
        const int s = p + k * P;
        pre[k] = s < NS ? col[(int64_t)s * C4] : f32x4{0.f, 0.f, 0.f, 0.f};
    }
    const float m0 = t < NS && t < 64 ? ml[2 * t] : -INFINITY, l0 = t < NS && t < 64 ? ml[2 * t + 1] : 0.f;
    const SeqRange sr = seq_range(a, b);
    const int S = (sr.L - sr.base + a.split_tokens - 1) / a.split_tokens;
    if (S <= 1) return;                       // written by the decode kernel
    if (t < 64) {                             // wave 0: split weights and the final scale
        float m = t < S ? m0 : -INFINITY;
        for (int s = t + 64; s < S; s += 64) m = fmaxf(m, ml[2 * s]);
        const float M = wave_max(m);
        float den = 0.f;
        for (int s = t; s < S; s += 64) {
            // M = -inf: no split saw a token for this row (a query before the start)
            const float ms = s == t ? m0 : ml[2 * s], ls = s == t ? l0 : ml[2 * s + 1];
            const float w = M == -INFINITY ? 0.f : fast_exp2(ms - M);
            s_w[s] = w;
            den += w * ls;
        }
        den = wave_sum(den);
        if (t == 0) s_scale = den > 0.f ? a.v_scale / den : 0.f;
    }
    __syncthreads();
    KVQ_TRACE_MARK(1, false);
    f32x4 num = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < PRE; ++k) {
        const int s = p + k * P;
        if (s < S) num += s_w[s] * pre[k];
    }
    for (int s = p + PRE * P; s < S; s += P) num += s_w[s] * col[(int64_t)s * C4];
    part[p][d4] = num;
    __syncthreads();
    if (p == 0) {
#pragma unroll
        for (int q = 1; q < P; ++q) num += part[q][d4];
        const float scale = s_scale;
        const int64_t o = (int64_t)hq * D + 4 * d4;
#pragma unroll
        for (int e = 0; e < 4; ++e) store_out(a, o + e, num[e] * scale);
    }
    KVQ_TRACE_MARK(2);
    KVQ_TRACE_STORE_MERGE(hq);
}

template <int D, int FMT, int NT>
static hipError_t launch_family(const DecodeArgs& a, int B, int impl, hipStream_t st) {
    dim3 grid(a.num_splits, a.Hkv, B);
    constexpr int W = mfma_waves<D, FMT, NT>();
    const int GQ = a.G * a.q_len;
    const size_t lds_mfma = sizeof(float) * (kMaxSplitBlocks + lds_merge_floats(GQ, D, W, NT));
    if (a.k_new) {   // fused append (MFMA family): one new token, or FP8 / BF16 up to kMaxQueryLen
        constexpr bool kOne = NT == 1 && (FMT == kFmtFP8 || FMT == kFmtBF16 || FMT == kFmtNVFP4);
        constexpr bool kMany = FMT == kFmtFP8 || FMT == kFmtBF16;
        if (kOne && a.q_len == 1) {
            if constexpr (kOne)
                hipLaunchKernelGGL((decode_mfma_kernel<D, FMT, NT, W, kAppendOne>), grid, dim3(W * 64), lds_mfma, st,
                                   a);
        } else if constexpr (kMany) {
            hipLaunchKernelGGL((decode_mfma_kernel<D, FMT, NT, W, kAppendMany>), grid, dim3(W * 64), lds_mfma, st, a);
        } else {
            return hipErrorInvalidValue;
        }
    } else if (FMT == kFmtNVFP4 || FMT == kFmtFP8QP || impl == 2 || NT > 1) {
        hipLaunchKernelGGL((decode_mfma_kernel<D, FMT, NT>), grid, dim3(W * 64), lds_mfma, st, a);
    } else {
        if constexpr ((FMT == kFmtFP8 || FMT == kFmtBF16) && NT == 1) {
            const size_t lds = sizeof(float) * (kMaxSplitBlocks + lds_merge_floats(a.G, D, kWaves) + a.G * D +
                                                kWaves * 256);
            hipLaunchKernelGGL((decode_valu_kernel<D, FMT == kFmtFP8>), grid, dim3(kThreads), lds, st, a);
        }
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.num_splits <= 1) return e;
    hipLaunchKernelGGL((merge_splits_kernel<D>), dim3(B * a.q_len * a.Hq), dim3(kMergeThreads),
                       sizeof(float) * a.num_splits, st, a);
    return hipGetLastError();
}

// Column tiles per work-group: G * q_len columns in tiles of 16 (1, 2 or 4;
// at most 64 columns at D 64, 32 at D 128, 16 at D 256).
int decode_column_tiles(int G, int q_len, int D) {
    const int gq = G * q_len;
    const int nt = gq <= 16 ? 1 : gq <= 32 ? 2 : gq <= 64 ? 4 : 0;
    if (nt == 0 || nt * D > 256) return 0;
    return nt;
}

template <int FMT, int D>
static hipError_t launch_nt(const DecodeArgs& a, int B, int impl, hipStream_t st) {
    switch (decode_column_tiles(a.G, a.q_len, D)) {
        case 1: return launch_family<D, FMT, 1>(a, B, impl, st);
        case 2:
            if constexpr (D <= 128) return launch_family<D, FMT, 2>(a, B, impl, st);
            return hipErrorInvalidValue;
        case 4:
            if constexpr (D <= 64) return launch_family<D, FMT, 4>(a, B, impl, st);
            return hipErrorInvalidValue;
        default: return hipErrorInvalidValue;
    }
}

template <int FMT>
static hipError_t launch_d(const DecodeArgs& a, int B, int D, int impl, hipStream_t st) {
    switch (D) {
        case 64: return launch_nt<FMT, 64>(a, B, impl, st);
        case 128: return launch_nt<FMT, 128>(a, B, impl, st);
        case 256: return launch_nt<FMT, 256>(a, B, impl, st);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_decode(const DecodeArgs& a, int B, int D, int fmt, int impl, hipStream_t st) {
    switch (fmt) {
        case kFmtBF16: return launch_d<kFmtBF16>(a, B, D, impl, st);
        case kFmtFP8: return launch_d<kFmtFP8>(a, B, D, impl, st);
        case kFmtNVFP4: return launch_d<kFmtNVFP4>(a, B, D, impl, st);
        case kFmtFP8QP: return launch_d<kFmtFP8QP>(a, B, D, impl, st);
        default: return hipErrorInvalidValue;
    }
}

int trace_set_attn(uint64_t* buf, int64_t decode_words, int64_t merge_words) {
#if KVQ_TRACE
    const int64_t words[2] = {buf ? decode_words : 0, buf ? merge_words : 0};
    if (hipMemcpyToSymbol(HIP_SYMBOL(g_trace), &buf, sizeof(buf)) != hipSuccess) return -1;
    if (hipMemcpyToSymbol(HIP_SYMBOL(g_trace_words), words, sizeof(words)) != hipSuccess) return -1;
    return 0;
#else
    (void)buf;
    (void)decode_words;
    (void)merge_words;
    return 1;
#endif
}

unsigned check_flags_attn(bool clear) {
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
