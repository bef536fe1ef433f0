/* A plain C99 client of libkvq.so: it includes include/kvq.h, takes the
 * address of every declared entry point (so each one must be exported with C
 * linkage) and exercises the host-only calls and host validation, none of
 * which touches a GPU: status strings, the ABI version, calibration (the
 * scale formula of the FP8 calibration guide's calibrator paragraph:
 * max(amax * 1.05 / 448, 1e-12)), split planning and workspace sizing, and
 * invalid arguments rejected before any HIP call.  Built and run by
 * tests/test_c_client.py; prints "c client: ok" on success. */
#include <math.h>
#include <stdio.h>
#include <string.h>

#include "kvq.h"

#define CHECK(cond)                                                          \
    do {                                                                     \
        if (!(cond)) {                                                       \
            fprintf(stderr, "c client: check failed at line %d: %s\n", __LINE__, #cond); \
            return 1;                                                        \
        }                                                                    \
    } while (0)

typedef void (*any_fn)(void);

int main(void) {
    /* every entry point, by address */
    const any_fn fns[] = {
        (any_fn)kvq_strerror, (any_fn)kvq_last_hip_error, (any_fn)kvq_abi_version, (any_fn)kvq_check_flags,
        (any_fn)kvq_e4m3_encode_f32, (any_fn)kvq_e4m3_decode, (any_fn)kvq_amax_bf16, (any_fn)kvq_calibrate,
        (any_fn)kvq_cache_write, (any_fn)kvq_decode_workspace_bytes, (any_fn)kvq_paged_decode_attn,
        (any_fn)kvq_decode_workspace_bytes_ex, (any_fn)kvq_paged_decode_attn_ex,
        (any_fn)kvq_paged_decode_attn_append, (any_fn)kvq_decode_plan_split_tokens, (any_fn)kvq_nvfp4_calibrate,
        (any_fn)kvq_nvfp4_region_bytes, (any_fn)kvq_nvfp4_cache_bytes_per_block,
        (any_fn)kvq_nvfp4_cache_write, (any_fn)kvq_nvfp4_paged_decode_attn,
        (any_fn)kvq_nvfp4_paged_decode_attn_ex, (any_fn)kvq_nvfp4_paged_decode_attn_append,
        (any_fn)kvq_decode_workspace_bytes_mq, (any_fn)kvq_paged_decode_attn_mq,
        (any_fn)kvq_nvfp4_paged_decode_attn_mq, (any_fn)kvq_paged_decode_attn_mq_append,
        (any_fn)kvq_paged_decode_attn_fp8qp, (any_fn)kvq_cache_block_bytes,
        (any_fn)kvq_gather_blocks, (any_fn)kvq_scatter_blocks, (any_fn)kvq_offload_blocks,
        (any_fn)kvq_restore_blocks, (any_fn)kvq_e2m1_decode, (any_fn)kvq_paged_decode_attn_scratch,
        (any_fn)kvq_trace_set,
    };
    for (size_t i = 0; i < sizeof(fns) / sizeof(fns[0]); ++i) CHECK(fns[i] != NULL);

    CHECK(kvq_abi_version() == KVQ_ABI_VERSION);
    CHECK(strlen(kvq_strerror(KVQ_OK)) > 0);
    CHECK(strcmp(kvq_strerror(KVQ_EWORKSPACE), "workspace too small") == 0);

    /* calibration: fp32(max(amax * 1.05 / 448, 1e-12)), evaluated in double */
    const float amax[4] = {0.0f, 1.0f, 448.0f / 1.05f, 1000.0f};
    float scale[4];
    CHECK(kvq_calibrate(amax, scale, 4) == KVQ_OK);
    for (int i = 0; i < 4; ++i) {
        double want = (double)amax[i] * 1.05 / 448.0;
        if (want < 1e-12) want = 1e-12;
        CHECK(scale[i] == (float)want);
    }
    const float bad[1] = {NAN};
    CHECK(kvq_calibrate(bad, scale, 1) == KVQ_EINVAL);
    CHECK(kvq_calibrate(NULL, scale, 1) == KVQ_EINVAL);

    /* planning and workspace sizing (host only) */
    CHECK(kvq_decode_plan_split_tokens(1, 8, 65536, 16) == 2048);
    CHECK(kvq_decode_workspace_bytes(1, 64, 8, 64, 65536, 16) > 0);
    CHECK(kvq_decode_workspace_bytes_ex(1, 8, 2, 64, 100, 16, 100) == 0);   /* split not a multiple of 64 */
    CHECK(kvq_nvfp4_region_bytes(64, 16) == 9 * 64);
    CHECK(kvq_nvfp4_cache_bytes_per_block(8, 64, 16) == 8 * 576 && kvq_nvfp4_cache_bytes_per_block(0, 64, 16) == 0);

    /* host validation: rejected before any HIP call (pointers never used) */
    char fake[64];
    void* p = fake + (16 - ((uintptr_t)fake & 15));
    const int64_t* slots = (const int64_t*)p;
    const int32_t* ids = (const int32_t*)p;
    CHECK(kvq_cache_write(p, p, 128, slots, 5, 2, 96, p, p, 4, 16, KVQ_KV_FP8_E4M3, 0.5f, 0.5f, NULL) ==
          KVQ_EUNSUPPORTED);                                                 /* D = 96 */
    CHECK(kvq_cache_write(p, p, 128, slots, 5, 2, 64, p, p, 4, 16, 7, 0.5f, 0.5f, NULL) == KVQ_EINVAL);
    CHECK(kvq_paged_decode_attn(p, p, p, KVQ_KV_FP8_E4M3, ids, 4, ids, 64, 1, 12, 8, 64, 16, 4, 0.5f, 0.5f, 0.125f,
                                p, KVQ_OUT_F32, p, 1 << 20, NULL) == KVQ_EINVAL);   /* Hq % Hkv != 0 */
    CHECK(kvq_paged_decode_attn(p, p, p, KVQ_KV_FP8_E4M3, ids, 4, ids, 64, 1, 8, 8, 64, 16, 4, 0.5f, 0.5f, 0.125f,
                                p, KVQ_OUT_F32, p, 16, NULL) == KVQ_EWORKSPACE);
    unsigned flags = 1;
    CHECK(kvq_check_flags(&flags, 0) == KVQ_EUNSUPPORTED && flags == 0);   /* the release build */
    CHECK(kvq_trace_set(NULL, 0, 0) == KVQ_EUNSUPPORTED && kvq_trace_set(NULL, -1, 0) == KVQ_EINVAL);
    printf("c client: ok\n");
    return 0;
}
