/*
 * kvq_oracle.c -- the CPU definition of the quantized paged decode-attention
 * path.  TEST INFRASTRUCTURE ONLY (see kvq_oracle.h): only tests, the smoke
 * check and the CPU-baseline leg of the benchmark load it.
 *
 * Build: gcc -O2 -std=c99 -fPIC -shared -ffp-contract=off (no -ffast-math:
 * the quantize step is defined as one IEEE fp32 division).
 */
#define _POSIX_C_SOURCE 200809L
#include "kvq_oracle.h"

#include <math.h>
#include <pthread.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------ */
/* codecs                                                                    */
/* ------------------------------------------------------------------------ */

double kvqo_e4m3_value(uint8_t code) {
    int s = code >> 7;
    int e = (code >> 3) & 15;
    int m = code & 7;
    double mag;
    if (e == 15 && m == 7) return NAN;           /* the only NaN encodings */
    if (e == 0) mag = ldexp((double)m / 8.0, -6); /* subnormal: 0.mmm * 2^-6 */
    else mag = ldexp(1.0 + (double)m / 8.0, e - 7);
    return s ? -mag : mag;
}

/* values of the 127 non-negative finite codes 0x00..0x7E, filled once */
static double g_e4m3_pos[0x7F];
static pthread_once_t g_e4m3_once = PTHREAD_ONCE_INIT;
static void fill_e4m3_pos(void) {
    for (int c = 0; c <= 0x7E; ++c) g_e4m3_pos[c] = kvqo_e4m3_value((uint8_t)c);
}

uint8_t kvqo_e4m3_encode(float y) {
    uint8_t sign = signbit(y) ? 0x80 : 0x00;
    if (isnan(y)) return (uint8_t)(0x7F | sign);
    double a = fabs((double)y);
    if (a > 448.0) return (uint8_t)(0x7E | sign); /* saturate (Inf too) */
    pthread_once(&g_e4m3_once, fill_e4m3_pos);
    int best = 0;
    double best_d = INFINITY;
    for (int c = 0; c <= 0x7E; ++c) {             /* all non-negative finite codes */
        double d = fabs(g_e4m3_pos[c] - a);
        if (d < best_d || (d == best_d && (c & 1) == 0)) {
            best = c;
            best_d = d;
        }
    }
    return (uint8_t)(best | sign);
}

void kvqo_e4m3_encode_array(const float* y, uint8_t* codes, int64_t n) {
    for (int64_t i = 0; i < n; ++i) codes[i] = kvqo_e4m3_encode(y[i]);
}

float kvqo_bf16_to_float(uint16_t bits) {
    uint32_t w = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &w, sizeof f);
    return f;
}

uint8_t kvqo_e4m3_quantize(uint16_t x_bf16, float scale) {
    volatile float x = kvqo_bf16_to_float(x_bf16);
    volatile float y = x / scale; /* one IEEE fp32 division, round to nearest even */
    return kvqo_e4m3_encode(y);
}

double kvqo_e2m1_value(uint8_t nibble) {
    static const double mag[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};
    double v = mag[nibble & 7];
    return (nibble & 8) ? -v : v;
}

uint8_t kvqo_e2m1_encode(float y) {
    uint8_t sign = signbit(y) ? 0x8 : 0x0;
    if (isnan(y)) return (uint8_t)(0x7 | sign);
    double a = fabs((double)y);
    if (a > 6.0) return (uint8_t)(0x7 | sign);
    int best = 0;
    double best_d = INFINITY;
    for (int c = 0; c < 8; ++c) {
        double d = fabs(kvqo_e2m1_value((uint8_t)c) - a);
        if (d < best_d || (d == best_d && (c & 1) == 0)) {
            best = c;
            best_d = d;
        }
    }
    return (uint8_t)(best | sign);
}

/* ------------------------------------------------------------------------ */
/* calibration                                                               */
/* ------------------------------------------------------------------------ */

static int scale_from_amax(const float* amax, float* scale, int n, double top) {
    for (int i = 0; i < n; ++i)
        if (!(amax[i] >= 0.0f) || isinf(amax[i])) return -1;
    for (int i = 0; i < n; ++i) {
        double s = (double)amax[i] * 1.05 / top;
        if (s < 1e-12) s = 1e-12;
        scale[i] = (float)s;
    }
    return 0;
}

int kvqo_calibrate(const float* amax, float* scale, int n) {
    return scale_from_amax(amax, scale, n, 448.0);
}

int kvqo_nvfp4_calibrate(const float* amax, float* gscale, int n) {
    return scale_from_amax(amax, gscale, n, 6.0 * 448.0);
}

float kvqo_amax_bf16(const uint16_t* x, int64_t rows, int64_t cols, int64_t row_stride) {
    double m = 0.0;
    int saw_nan = 0;
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t c = 0; c < cols; ++c) {
            double a = fabs((double)kvqo_bf16_to_float(x[r * row_stride + c]));
            if (isnan(a)) saw_nan = 1;
            else if (a > m) m = a;
        }
    return saw_nan ? NAN : (float)m;
}

/* ------------------------------------------------------------------------ */
/* paged cache                                                               */
/* ------------------------------------------------------------------------ */

int64_t kvqo_nvfp4_region_bytes(int D, int block_size) {
    return (int64_t)block_size * D / 2 + (int64_t)block_size * D / 16;
}

/* byte/element offset of (slot, g, d) in the K and V layouts */
static int64_t k_index(int64_t slot, int g, int d, int Hkv, int D, int bs) {
    int64_t blk = slot / bs, off = slot % bs;
    return ((blk * Hkv + g) * bs + off) * D + d;
}
static int64_t v_index(int64_t slot, int g, int d, int Hkv, int D, int bs) {
    int64_t blk = slot / bs, off = slot % bs;
    return ((blk * Hkv + g) * D + d) * bs + off;
}

/* Which tokens a write thread handles: those whose slot pair (slot / 2) falls
 * to it.  Every write to one slot (and to the two slots that share an NVFP4 V
 * byte) then happens in one thread, in token order, so the bytes equal the
 * serial write's for any slot mapping, repeated slots included. */
static int write_share(int64_t slot, int tid, int nthreads) {
    return slot >= 0 && (int)((slot / 2) % nthreads) == tid;
}

typedef struct {
    const uint16_t *k, *v;
    int64_t src_stride;
    const int64_t* slot_mapping;
    int T, Hkv, D;
    void *k_cache, *v_cache;
    int block_size, kv_dtype;
    float k_scale, v_scale;
    int tid, nthreads;
} write_job;

static void* cache_write_worker(void* arg) {
    const write_job* j = (const write_job*)arg;
    for (int t = 0; t < j->T; ++t) {
        int64_t slot = j->slot_mapping[t];
        if (!write_share(slot, j->tid, j->nthreads)) continue;
        for (int g = 0; g < j->Hkv; ++g)
            for (int d = 0; d < j->D; ++d) {
                uint16_t xk = j->k[t * j->src_stride + (int64_t)g * j->D + d];
                uint16_t xv = j->v[t * j->src_stride + (int64_t)g * j->D + d];
                int64_t ki = k_index(slot, g, d, j->Hkv, j->D, j->block_size);
                int64_t vi = v_index(slot, g, d, j->Hkv, j->D, j->block_size);
                if (j->kv_dtype == 0) {
                    ((uint16_t*)j->k_cache)[ki] = xk;
                    ((uint16_t*)j->v_cache)[vi] = xv;
                } else {
                    ((uint8_t*)j->k_cache)[ki] = kvqo_e4m3_quantize(xk, j->k_scale);
                    ((uint8_t*)j->v_cache)[vi] = kvqo_e4m3_quantize(xv, j->v_scale);
                }
            }
    }
    return NULL;
}

/* Runs worker over nthreads shares of the tokens (one share: the caller's thread). */
static void run_write(write_job* base, void* (*worker)(void*), int nthreads) {
    if (nthreads < 1) nthreads = 1;
    write_job* jobs = (write_job*)malloc(sizeof(write_job) * (size_t)nthreads);
    pthread_t* th = (pthread_t*)malloc(sizeof(pthread_t) * (size_t)nthreads);
    for (int i = 0; i < nthreads; ++i) {
        jobs[i] = *base;
        jobs[i].tid = i;
        jobs[i].nthreads = nthreads;
    }
    for (int i = 1; i < nthreads; ++i) pthread_create(&th[i], NULL, worker, &jobs[i]);
    worker(&jobs[0]);
    for (int i = 1; i < nthreads; ++i) pthread_join(th[i], NULL);
    free(th);
    free(jobs);
}

void kvqo_cache_write(const uint16_t* k, const uint16_t* v, int64_t src_stride,
                      const int64_t* slot_mapping, int T, int Hkv, int D,
                      void* k_cache, void* v_cache, int block_size, int kv_dtype,
                      float k_scale, float v_scale, int nthreads) {
    write_job j = {k, v, src_stride, slot_mapping, T, Hkv, D, k_cache, v_cache, block_size, kv_dtype,
                   k_scale, v_scale, 0, 1};
    run_write(&j, cache_write_worker, nthreads);
}

/* NVFP4: quantize one 16-element group x[0..15] into codes[16] and a scale code */
static void nvfp4_group(const uint16_t* x, float gscale, uint8_t* codes, uint8_t* bscale_code) {
    float bamax = 0.0f;
    int saw_nan = 0;
    for (int i = 0; i < 16; ++i) {
        float a = fabsf(kvqo_bf16_to_float(x[i]));
        if (isnan(a)) saw_nan = 1;
        else if (a > bamax) bamax = a;
    }
    if (saw_nan) bamax = NAN;
    volatile float top = 6.0f * gscale;       /* fp32 product */
    volatile float ratio = bamax / top;        /* fp32 division */
    *bscale_code = kvqo_e4m3_encode(ratio);
    volatile float e = (float)kvqo_e4m3_value(*bscale_code) * gscale; /* fp32 product */
    for (int i = 0; i < 16; ++i) {
        if (e == 0.0f) {
            codes[i] = 0;
        } else {
            volatile float y = kvqo_bf16_to_float(x[i]) / e; /* fp32 division */
            codes[i] = kvqo_e2m1_encode(y);
        }
    }
}

static void set_nibble(uint8_t* p, int64_t nib_index, uint8_t code) {
    uint8_t* byte = p + nib_index / 2;
    if (nib_index % 2 == 0) *byte = (uint8_t)((*byte & 0xF0) | (code & 0xF));
    else *byte = (uint8_t)((*byte & 0x0F) | ((code & 0xF) << 4));
}

static uint8_t get_nibble(const uint8_t* p, int64_t nib_index) {
    uint8_t byte = p[nib_index / 2];
    return (nib_index % 2 == 0) ? (byte & 0xF) : (byte >> 4);
}

static void* nvfp4_write_worker(void* arg) {
    const write_job* j = (const write_job*)arg;
    const int D = j->D, Hkv = j->Hkv, block_size = j->block_size;
    int64_t region = kvqo_nvfp4_region_bytes(D, block_size);
    int64_t codes_bytes = (int64_t)block_size * D / 2;
    uint8_t* k_cache = (uint8_t*)j->k_cache;
    uint8_t* v_cache = (uint8_t*)j->v_cache;
    for (int t = 0; t < j->T; ++t) {
        int64_t slot = j->slot_mapping[t];
        if (!write_share(slot, j->tid, j->nthreads)) continue;
        int64_t blk = slot / block_size, off = slot % block_size;
        for (int g = 0; g < Hkv; ++g) {
            uint8_t* kr = k_cache + (blk * Hkv + g) * region;
            uint8_t* vr = v_cache + (blk * Hkv + g) * region;
            for (int grp = 0; grp < D / 16; ++grp) {
                uint8_t codes[16], sc;
                const uint16_t* xk = j->k + t * j->src_stride + (int64_t)g * D + grp * 16;
                nvfp4_group(xk, j->k_scale, codes, &sc);
                for (int i = 0; i < 16; ++i)
                    set_nibble(kr, off * D + grp * 16 + i, codes[i]);      /* [bs][D] nibbles */
                kr[codes_bytes + off * (D / 16) + grp] = sc;

                const uint16_t* xv = j->v + t * j->src_stride + (int64_t)g * D + grp * 16;
                nvfp4_group(xv, j->v_scale, codes, &sc);
                for (int i = 0; i < 16; ++i)
                    set_nibble(vr, (int64_t)(grp * 16 + i) * block_size + off, codes[i]); /* [D][bs] nibbles */
                vr[codes_bytes + (int64_t)grp * block_size + off] = sc;                  /* [D/16][bs] */
            }
        }
    }
    return NULL;
}

void kvqo_nvfp4_cache_write(const uint16_t* k, const uint16_t* v, int64_t src_stride,
                            const int64_t* slot_mapping, int T, int Hkv, int D,
                            uint8_t* k_cache, uint8_t* v_cache, int block_size,
                            float k_gscale, float v_gscale, int nthreads) {
    write_job j = {k, v, src_stride, slot_mapping, T, Hkv, D, k_cache, v_cache, block_size, 2,
                   k_gscale, v_gscale, 0, 1};
    /* a V code byte holds two slots' nibbles (d * bs + off, d * bs + off + 1): with an
       odd block size such a pair is not a slot pair, so write on one thread */
    run_write(&j, nvfp4_write_worker, block_size % 2 ? 1 : nthreads);
}

double kvqo_nvfp4_k_value(const uint8_t* k_cache, int64_t slot, int g, int d,
                          int Hkv, int D, int block_size, float k_gscale) {
    int64_t region = kvqo_nvfp4_region_bytes(D, block_size);
    int64_t blk = slot / block_size, off = slot % block_size;
    const uint8_t* r = k_cache + (blk * Hkv + g) * region;
    uint8_t code = get_nibble(r, off * D + d);
    uint8_t sc = r[(int64_t)block_size * D / 2 + off * (D / 16) + d / 16];
    return kvqo_e2m1_value(code) * kvqo_e4m3_value(sc) * (double)k_gscale;
}

double kvqo_nvfp4_v_value(const uint8_t* v_cache, int64_t slot, int g, int d,
                          int Hkv, int D, int block_size, float v_gscale) {
    int64_t region = kvqo_nvfp4_region_bytes(D, block_size);
    int64_t blk = slot / block_size, off = slot % block_size;
    const uint8_t* r = v_cache + (blk * Hkv + g) * region;
    uint8_t code = get_nibble(r, (int64_t)d * block_size + off);
    uint8_t sc = r[(int64_t)block_size * D / 2 + (int64_t)(d / 16) * block_size + off];
    return kvqo_e2m1_value(code) * kvqo_e4m3_value(sc) * (double)v_gscale;
}

/* ------------------------------------------------------------------------ */
/* attention                                                                 */
/* ------------------------------------------------------------------------ */

typedef struct {
    const uint16_t* q;
    const void* k_cache;
    const void* v_cache;
    int kv_dtype;
    const int32_t* block_tables;
    int max_blocks;
    const int32_t* seq_lens;
    int B, Hq, Hkv, D, block_size;
    float k_scale, v_scale, sm_scale;
    const int32_t* units; /* NULL: unit u is (b, i, h) = (u / (q_len*Hq), u / Hq % q_len, u % Hq) */
    int n_units;
    int q_len;            /* queries per sequence: the q_len newest tokens */
    int window;           /* > 0: each query sees at most its `window` newest tokens */
    int fp8qp;            /* FP8 Q and P variant (FP8 cache only) */
    float q_scale;        /* fp8qp: Q quantization scale */
    double* out;
    int next_unit;
    pthread_mutex_t lock;
} attn_job;

static double k_value(const attn_job* j, int64_t slot, int g, int d) {
    if (j->kv_dtype == 2)
        return kvqo_nvfp4_k_value((const uint8_t*)j->k_cache, slot, g, d, j->Hkv, j->D,
                                  j->block_size, j->k_scale);
    int64_t i = k_index(slot, g, d, j->Hkv, j->D, j->block_size);
    if (j->kv_dtype == 0) return (double)kvqo_bf16_to_float(((const uint16_t*)j->k_cache)[i]);
    return kvqo_e4m3_value(((const uint8_t*)j->k_cache)[i]) * (double)j->k_scale;
}

static double v_value(const attn_job* j, int64_t slot, int g, int d) {
    if (j->kv_dtype == 2)
        return kvqo_nvfp4_v_value((const uint8_t*)j->v_cache, slot, g, d, j->Hkv, j->D,
                                  j->block_size, j->v_scale);
    int64_t i = v_index(slot, g, d, j->Hkv, j->D, j->block_size);
    if (j->kv_dtype == 0) return (double)kvqo_bf16_to_float(((const uint16_t*)j->v_cache)[i]);
    return kvqo_e4m3_value(((const uint8_t*)j->v_cache)[i]) * (double)j->v_scale;
}

/* Query i of sequence b (the token at position p = seq_len - q_len + i)
 * attends causally: to tokens 0 .. p, i.e. L = p + 1 of them, or with a
 * sliding window W > 0 to tokens max(0, p - W + 1) .. p; out = 0 when L <= 0. */
static void attend_one(const attn_job* j, int b, int i, int h, double* out, double* s) {
    int G = j->Hq / j->Hkv;
    int g = h / G;
    int L = j->seq_lens[b] - j->q_len + 1 + i;
    int D = j->D;
    const uint16_t* q = j->q + (((int64_t)b * j->q_len + i) * j->Hq + h) * D;
    for (int d = 0; d < D; ++d) out[d] = 0.0;
    if (L <= 0) return;
    int t0 = (j->window > 0 && L > j->window) ? L - j->window : 0;
    double m = -INFINITY;
    for (int t = t0; t < L; ++t) {
        int64_t slot = (int64_t)j->block_tables[(int64_t)b * j->max_blocks + t / j->block_size] *
                           j->block_size + t % j->block_size;
        double dot = 0.0;
        for (int d = 0; d < D; ++d) dot += (double)kvqo_bf16_to_float(q[d]) * k_value(j, slot, g, d);
        s[t] = (double)j->sm_scale * dot;
        if (s[t] > m) m = s[t];
    }
    double denom = 0.0;
    for (int t = t0; t < L; ++t) {
        int64_t slot = (int64_t)j->block_tables[(int64_t)b * j->max_blocks + t / j->block_size] *
                           j->block_size + t % j->block_size;
        double w = exp(s[t] - m);
        denom += w;
        for (int d = 0; d < D; ++d) out[d] += w * v_value(j, slot, g, d);
    }
    for (int d = 0; d < D; ++d) out[d] /= denom;
}

/* FP8 Q and P: q codes E4M3(fp32(q) / q_scale); x_t = c * sum_d value(qc_d) *
 * value(kc_td) with c = fp32(sm_scale * q_scale * k_scale * log2 e); integer
 * reference R = ceil(max_t x_t); P code pc_t = E4M3(fp32(448 * 2^(x_t - R)));
 * out = v_scale * sum_t value(pc_t) value(vc_t) / sum_t value(pc_t). */
static void attend_one_fp8qp(const attn_job* j, int b, int i, int h, double* out, double* s) {
    int G = j->Hq / j->Hkv;
    int g = h / G;
    int L = j->seq_lens[b] - j->q_len + 1 + i;
    int D = j->D;
    const uint16_t* q = j->q + (((int64_t)b * j->q_len + i) * j->Hq + h) * D;
    for (int d = 0; d < D; ++d) out[d] = 0.0;
    if (L <= 0) return;
    int t0 = (j->window > 0 && L > j->window) ? L - j->window : 0;
    const double c = (double)(float)((double)j->sm_scale * (double)j->q_scale * (double)j->k_scale *
                                     1.4426950408889634);
    double qv[256];
    for (int d = 0; d < D; ++d) qv[d] = kvqo_e4m3_value(kvqo_e4m3_quantize(q[d], j->q_scale));
    const uint8_t* kc = (const uint8_t*)j->k_cache;
    const uint8_t* vc = (const uint8_t*)j->v_cache;
    double xmax = -INFINITY;
    for (int t = t0; t < L; ++t) {
        int64_t slot = (int64_t)j->block_tables[(int64_t)b * j->max_blocks + t / j->block_size] *
                           j->block_size + t % j->block_size;
        double dot = 0.0;
        for (int d = 0; d < D; ++d) dot += qv[d] * kvqo_e4m3_value(kc[k_index(slot, g, d, j->Hkv, D, j->block_size)]);
        s[t] = c * dot;
        if (s[t] > xmax) xmax = s[t];
    }
    const double R = ceil(xmax);
    double denom = 0.0;
    for (int t = t0; t < L; ++t) {
        int64_t slot = (int64_t)j->block_tables[(int64_t)b * j->max_blocks + t / j->block_size] *
                           j->block_size + t % j->block_size;
        double pw = kvqo_e4m3_value(kvqo_e4m3_encode((float)(448.0 * exp2(s[t] - R))));
        denom += pw;
        for (int d = 0; d < D; ++d) out[d] += pw * kvqo_e4m3_value(vc[v_index(slot, g, d, j->Hkv, D, j->block_size)]);
    }
    for (int d = 0; d < D; ++d) out[d] = out[d] * (double)j->v_scale / denom;
}

static void* attn_worker(void* arg) {
    attn_job* j = (attn_job*)arg;
    int max_L = 0;
    for (int b = 0; b < j->B; ++b)
        if (j->seq_lens[b] > max_L) max_L = j->seq_lens[b];
    double* s = (double*)malloc(sizeof(double) * (size_t)(max_L > 0 ? max_L : 1));
    for (;;) {
        pthread_mutex_lock(&j->lock);
        int u = j->next_unit++;
        pthread_mutex_unlock(&j->lock);
        if (u >= j->n_units) break;
        int b, i, h;
        if (j->units) {
            b = j->units[2 * u];
            i = 0;
            h = j->units[2 * u + 1];
        } else {
            b = u / (j->q_len * j->Hq);
            i = u / j->Hq % j->q_len;
            h = u % j->Hq;
        }
        if (j->fp8qp)
            attend_one_fp8qp(j, b, i, h, j->out + (int64_t)u * j->D, s);
        else
            attend_one(j, b, i, h, j->out + (int64_t)u * j->D, s);
    }
    free(s);
    return NULL;
}

static void run_attn(attn_job* j, int nthreads) {
    if (nthreads < 1) nthreads = 1;
    pthread_mutex_init(&j->lock, NULL);
    j->next_unit = 0;
    if (nthreads == 1) {
        attn_worker(j);
    } else {
        pthread_t* th = (pthread_t*)malloc(sizeof(pthread_t) * (size_t)nthreads);
        for (int i = 0; i < nthreads; ++i) pthread_create(&th[i], NULL, attn_worker, j);
        for (int i = 0; i < nthreads; ++i) pthread_join(th[i], NULL);
        free(th);
    }
    pthread_mutex_destroy(&j->lock);
}

void kvqo_decode_attn(const uint16_t* q, const void* k_cache, const void* v_cache,
                      int kv_dtype, const int32_t* block_tables, int max_blocks,
                      const int32_t* seq_lens, int B, int Hq, int Hkv, int D,
                      int block_size, float k_scale, float v_scale, float sm_scale,
                      double* out, int nthreads) {
    attn_job j = {q, k_cache, v_cache, kv_dtype, block_tables, max_blocks, seq_lens,
                  B, Hq, Hkv, D, block_size, k_scale, v_scale, sm_scale,
                  NULL, B * Hq, 1, 0, 0, 0.0f, out, 0};
    run_attn(&j, nthreads);
}

void kvqo_decode_attn_mq(const uint16_t* q, int q_len, int window, const void* k_cache, const void* v_cache,
                         int kv_dtype, const int32_t* block_tables, int max_blocks,
                         const int32_t* seq_lens, int B, int Hq, int Hkv, int D,
                         int block_size, float k_scale, float v_scale, float sm_scale,
                         double* out, int nthreads) {
    attn_job j = {q, k_cache, v_cache, kv_dtype, block_tables, max_blocks, seq_lens,
                  B, Hq, Hkv, D, block_size, k_scale, v_scale, sm_scale,
                  NULL, B * q_len * Hq, q_len, window, 0, 0.0f, out, 0};
    run_attn(&j, nthreads);
}

void kvqo_decode_attn_units(const uint16_t* q, const void* k_cache, const void* v_cache,
                            int kv_dtype, const int32_t* block_tables, int max_blocks,
                            const int32_t* seq_lens, int B, int Hq, int Hkv, int D,
                            int block_size, float k_scale, float v_scale, float sm_scale,
                            const int32_t* units, int n_units, double* out, int nthreads) {
    attn_job j = {q, k_cache, v_cache, kv_dtype, block_tables, max_blocks, seq_lens,
                  B, Hq, Hkv, D, block_size, k_scale, v_scale, sm_scale,
                  units, n_units, 1, 0, 0, 0.0f, out, 0};
    run_attn(&j, nthreads);
}

void kvqo_decode_attn_fp8qp(const uint16_t* q, int q_len, int window, const uint8_t* k_cache,
                            const uint8_t* v_cache, const int32_t* block_tables, int max_blocks,
                            const int32_t* seq_lens, int B, int Hq, int Hkv, int D, int block_size,
                            float q_scale, float k_scale, float v_scale, float sm_scale, double* out,
                            int nthreads) {
    attn_job j = {q, k_cache, v_cache, 1, block_tables, max_blocks, seq_lens,
                  B, Hq, Hkv, D, block_size, k_scale, v_scale, sm_scale,
                  NULL, B * q_len * Hq, q_len, window, 1, q_scale, out, 0};
    run_attn(&j, nthreads);
}

/* Grid spacing of E4M3 at magnitude y: 2^(e - 3) in the binade [2^e, 2^(e+1)),
 * and the subnormal spacing 2^-9 below 2^-6. */
static double e4m3_step(double y) {
    int e;
    if (y < 0.015625) return ldexp(1.0, -9);
    frexp(y, &e); /* y = f * 2^e, f in [0.5, 1) */
    return ldexp(1.0, e - 1 - 3);
}

/* Tolerance of kvqo_decode_attn_fp8qp: see kvq_oracle.h for the assumptions.
 * All quantities of one (b, i, h) row are in code units of the definition's
 * frame R (v_scale applied at the end). */
void kvqo_decode_attn_fp8qp_tol(const uint16_t* q, int q_len, int window, const uint8_t* k_cache,
                                const uint8_t* v_cache, const int32_t* block_tables, int max_blocks,
                                const int32_t* seq_lens, int B, int Hq, int Hkv, int D, int block_size,
                                float q_scale, float k_scale, float v_scale, float sm_scale, double eps,
                                double* tol, int64_t* n_open, double* w_out, double* delta_out) {
    const int G = Hq / Hkv;
    const double c = (double)(float)((double)sm_scale * (double)q_scale * (double)k_scale * 1.4426950408889634);
    int max_L = 1;
    for (int b = 0; b < B; ++b)
        if (seq_lens[b] > max_L) max_L = seq_lens[b];
    double* x = (double*)malloc(sizeof(double) * (size_t)max_L);
    double* dx = (double*)malloc(sizeof(double) * (size_t)max_L);
    double* w = (double*)malloc(sizeof(double) * (size_t)max_L);
    double* dl = (double*)malloc(sizeof(double) * (size_t)max_L);
    *n_open = 0;
    for (int b = 0; b < B; ++b)
        for (int i = 0; i < q_len; ++i)
            for (int h = 0; h < Hq; ++h) {
                const int64_t row = ((int64_t)b * q_len + i) * Hq + h;
                double* trow = tol + row * D;
                for (int d = 0; d < D; ++d) trow[d] = 0.0;
                const int L = seq_lens[b] - q_len + 1 + i;
                if (L <= 0) continue;
                const int t0 = (window > 0 && L > window) ? L - window : 0;
                const int g = h / G;
                const uint16_t* qr = q + row * D;
                double qv[256];
                for (int d = 0; d < D; ++d) qv[d] = kvqo_e4m3_value(kvqo_e4m3_quantize(qr[d], q_scale));
                /* scores, as the definition computes them, and their error bound:
                   (A1) on the dot, plus fp32 rounding of the scale step and exp2 */
                double xmax = -INFINITY, dxmax = 0.0;
                for (int t = t0; t < L; ++t) {
                    const int64_t slot = (int64_t)block_tables[(int64_t)b * max_blocks + t / block_size] *
                                             block_size + t % block_size;
                    double dot = 0.0, sabs = 0.0;
                    for (int d = 0; d < D; ++d) {
                        const double p = qv[d] * kvqo_e4m3_value(k_cache[k_index(slot, g, d, Hkv, D, block_size)]);
                        dot += p;
                        sabs += fabs(p);
                    }
                    x[t] = c * dot;
                    if (x[t] > xmax) xmax = x[t];
                    dx[t] = eps * fabs(c) * sabs;
                }
                const double R = ceil(xmax);
                int bad = 0;
                double W = 0.0, DW = 0.0;
                for (int t = t0; t < L; ++t) {
                    dx[t] += ldexp(2.0 + fabs(x[t]) + fabs(x[t] - R), -20);
                    if (dx[t] > dxmax) dxmax = dx[t];
                    /* the definition's weight, then the extreme arguments a score error of dx allows */
                    const double a = 448.0 * exp2(x[t] - R);
                    w[t] = kvqo_e4m3_value(kvqo_e4m3_encode((float)a));
                    const double lo_a = a * exp2(-dx[t]);
                    const double hi_a = fmin(448.0, a * exp2(dx[t]));
                    if (lo_a >= 0.03125) {
                        /* in the normal range of the definition's frame and of every frame
                           an implementation may hold (A3: at most one binade coarser, or finer
                           with the argument still <= 448), where E4M3 rounding commutes with
                           the power-of-two rescale: the weight is the rounding of an argument
                           in [lo_a, hi_a], and rounding is monotone */
                        const double wl = kvqo_e4m3_value(kvqo_e4m3_encode((float)lo_a));
                        const double wh = kvqo_e4m3_value(kvqo_e4m3_encode((float)hi_a));
                        dl[t] = fmax(w[t] - wl, wh - w[t]);
                        if (dl[t] > 0.0) ++*n_open;
                    } else {
                        /* near or below the subnormal range: the weight may be rounded on the grid
                           of any frame up to R + 1, whose spacing at hi_a is at most twice E4M3's at
                           hi_a / 2, so it moves by at most half that spacing, and never by more than
                           the value itself; plus the definition's own rounding and the score bound */
                        dl[t] = fabs(a - w[t]) + (hi_a - a) + fmin(hi_a, e4m3_step(hi_a / 2.0));
                    }
                    W += w[t];
                    DW += dl[t];
                    if (w_out) {
                        w_out[row * max_L + t] = w[t];
                        delta_out[row * max_L + t] = dl[t];
                    }
                }
                if (dxmax >= 0.5 || !(W > DW)) bad = 1;
                for (int d = 0; d < D; ++d) {
                    double num = 0.0;
                    for (int t = t0; t < L; ++t) {
                        const int64_t slot = (int64_t)block_tables[(int64_t)b * max_blocks + t / block_size] *
                                                 block_size + t % block_size;
                        num += w[t] * kvqo_e4m3_value(v_cache[v_index(slot, g, d, Hkv, D, block_size)]);
                    }
                    const double o = num / W;
                    double e1 = 0.0, a_abs = 0.0;
                    for (int t = t0; t < L; ++t) {
                        const int64_t slot = (int64_t)block_tables[(int64_t)b * max_blocks + t / block_size] *
                                                 block_size + t % block_size;
                        const double vv = kvqo_e4m3_value(v_cache[v_index(slot, g, d, Hkv, D, block_size)]);
                        e1 += dl[t] * fabs(vv - o);
                        a_abs += (w[t] + dl[t]) * fabs(vv);
                    }
                    /* o' - o = (sum (w'-w)(v - o) + eta_N - o eta_W) / W'', |eta_N| <= eps a_abs,
                       |eta_W| <= eps (W + DW), W'' >= (W - DW)(1 - eps); then the fp32 epilogue */
                    trow[d] = bad ? INFINITY
                                  : (double)v_scale * ((e1 + eps * (a_abs + fabs(o) * (W + DW))) /
                                                           ((W - DW) * (1.0 - eps)) +
                                                       ldexp(fabs(o), -20));
                }
            }
    free(x);
    free(dx);
    free(w);
    free(dl);
}

double kvqo_fp8_cos_sim(const uint16_t* x, int64_t n, float scale) {
    double xy = 0.0, xx = 0.0, yy = 0.0;
    for (int64_t i = 0; i < n; ++i) {
        double a = (double)kvqo_bf16_to_float(x[i]);
        double r = kvqo_e4m3_value(kvqo_e4m3_quantize(x[i], scale)) * (double)scale;
        xy += a * r;
        xx += a * a;
        yy += r * r;
    }
    return xy / sqrt(xx * yy);
}

/* ------------------------------------------------------------------------ */
/* block copies for a host-memory tier                                        */
/* ------------------------------------------------------------------------ */

size_t kvqo_block_bytes(int kv_dtype, int Hkv, int D, int block_size) {
    size_t per_head;
    if (kv_dtype == 2)
        per_head = (size_t)block_size * D / 2 + (size_t)block_size * D / 16;
    else
        per_head = (size_t)block_size * D * (kv_dtype == 0 ? 2 : 1);
    return (size_t)Hkv * per_head;
}

void kvqo_gather_blocks(const uint8_t* cache, size_t block_bytes, const int32_t* ids, int n, uint8_t* dst) {
    for (int i = 0; i < n; ++i)
        memcpy(dst + (size_t)i * block_bytes, cache + (size_t)ids[i] * block_bytes, block_bytes);
}

void kvqo_scatter_blocks(const uint8_t* src, size_t block_bytes, const int32_t* ids, int n, uint8_t* cache) {
    for (int i = 0; i < n; ++i)
        memcpy(cache + (size_t)ids[i] * block_bytes, src + (size_t)i * block_bytes, block_bytes);
}
