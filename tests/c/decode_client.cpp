// A C++ client of libkvq.so with no PyTorch in the process: the decode path
// driven through include/kvq.h on raw HIP allocations and a stream of its
// own -- calibrate (amax on the device, the scale formula on the host), write
// the FP8 (or BF16) paged cache, then decode attention -- the order the FP8
// calibration guide gives (observe BF16 K/V maxima, derive per-layer scales,
// store FP8 with them) followed by the decode the Run 26 description times.
//
//   decode_client DIR
//
// DIR holds the inputs (raw little-endian arrays written by
// tests/test_gpu_c_client.py): params.txt
//   "B Hq Hkv D T num_blocks max_blocks max_seq_len kv_dtype split_tokens sm_scale",
// q.bin (bf16 [B][Hq][D]), k.bin / v.bin (bf16 [T][Hkv][D]), slots.bin
// (int64 [T]), bt.bin (int32 [B][max_blocks]), sl.bin (int32 [B]).  It writes
// scales.txt (the K and V amax, then k_scale and v_scale, as %a hex floats),
// kc.bin / vc.bin (the caches) and out.bin (fp32 [B][Hq][D]).  Exit status 0 on success; any failed call
// prints its status and exits 1.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <string>
#include <vector>

#include "kvq.h"

namespace {

[[noreturn]] void die(const char* what, int status) {
    std::fprintf(stderr, "decode_client: %s failed: %d (%s, hip %d)\n", what, status,
                 status < 0 ? kvq_strerror(status) : "hip", kvq_last_hip_error());
    std::exit(1);
}

void hip_check(hipError_t e, const char* what) {
    if (e != hipSuccess) die(what, (int)e);
}

void kvq_check(int s, const char* what) {
    if (s != KVQ_OK) die(what, s);
}

template <class T>
std::vector<T> read_file(const std::string& path, size_t count) {
    std::vector<T> v(count);
    FILE* f = std::fopen(path.c_str(), "rb");
    if (!f || std::fread(v.data(), sizeof(T), count, f) != count) die(path.c_str(), -100);
    std::fclose(f);
    return v;
}

template <class T>
void write_file(const std::string& path, const std::vector<T>& v) {
    FILE* f = std::fopen(path.c_str(), "wb");
    if (!f || std::fwrite(v.data(), sizeof(T), v.size(), f) != v.size()) die(path.c_str(), -101);
    std::fclose(f);
}

template <class T>
T* to_device(const std::vector<T>& h) {
    T* d = nullptr;
    hip_check(hipMalloc(&d, h.size() * sizeof(T) + 16), "hipMalloc");
    hip_check(hipMemcpy(d, h.data(), h.size() * sizeof(T), hipMemcpyHostToDevice), "hipMemcpy H2D");
    return d;
}

}  // namespace

int main(int argc, char** argv) {
    if (argc != 2) {
        std::fprintf(stderr, "usage: decode_client DIR\n");
        return 2;
    }
    const std::string dir = argv[1];
    int B = 0, Hq = 0, Hkv = 0, D = 0, T = 0, num_blocks = 0, max_blocks = 0, max_seq_len = 0, kv_dtype = 0,
        split = 0;
    float sm_scale = 0.0f;
    {
        FILE* f = std::fopen((dir + "/params.txt").c_str(), "r");
        if (!f || std::fscanf(f, "%d %d %d %d %d %d %d %d %d %d %f", &B, &Hq, &Hkv, &D, &T, &num_blocks, &max_blocks,
                              &max_seq_len, &kv_dtype, &split, &sm_scale) != 11)
            die("params.txt", -102);
        std::fclose(f);
    }
    const auto q = read_file<uint16_t>(dir + "/q.bin", (size_t)B * Hq * D);
    const auto k = read_file<uint16_t>(dir + "/k.bin", (size_t)T * Hkv * D);
    const auto v = read_file<uint16_t>(dir + "/v.bin", (size_t)T * Hkv * D);
    const auto slots = read_file<int64_t>(dir + "/slots.bin", (size_t)T);
    const auto bt = read_file<int32_t>(dir + "/bt.bin", (size_t)B * max_blocks);
    const auto sl = read_file<int32_t>(dir + "/sl.bin", (size_t)B);

    hipStream_t st;
    hip_check(hipStreamCreate(&st), "hipStreamCreate");
    uint16_t* d_q = to_device(q);
    uint16_t* d_k = to_device(k);
    uint16_t* d_v = to_device(v);
    int64_t* d_slots = to_device(slots);
    int32_t* d_bt = to_device(bt);
    int32_t* d_sl = to_device(sl);

    // calibrate: amax of K and V on the device, the scales on the host
    float* d_amax = nullptr;
    hip_check(hipMalloc(&d_amax, 2 * sizeof(float)), "hipMalloc amax");
    hip_check(hipMemsetAsync(d_amax, 0, 2 * sizeof(float), st), "hipMemsetAsync");
    kvq_check(kvq_amax_bf16(d_k, T, (int64_t)Hkv * D, (int64_t)Hkv * D, d_amax, st), "kvq_amax_bf16 K");
    kvq_check(kvq_amax_bf16(d_v, T, (int64_t)Hkv * D, (int64_t)Hkv * D, d_amax + 1, st), "kvq_amax_bf16 V");
    float amax[2], scale[2] = {1.0f, 1.0f};
    hip_check(hipMemcpyAsync(amax, d_amax, sizeof(amax), hipMemcpyDeviceToHost, st), "hipMemcpy amax");
    hip_check(hipStreamSynchronize(st), "hipStreamSynchronize");
    if (kv_dtype == KVQ_KV_FP8_E4M3) kvq_check(kvq_calibrate(amax, scale, 2), "kvq_calibrate");

    // the paged cache (0xFF in unwritten slots) and its write
    const size_t elem = kv_dtype == KVQ_KV_FP8_E4M3 ? 1 : 2;
    const size_t cache_bytes = (size_t)num_blocks * Hkv * 16 * D * elem;
    void *d_kc = nullptr, *d_vc = nullptr;
    hip_check(hipMalloc(&d_kc, cache_bytes), "hipMalloc kc");
    hip_check(hipMalloc(&d_vc, cache_bytes), "hipMalloc vc");
    hip_check(hipMemsetAsync(d_kc, 0xFF, cache_bytes, st), "hipMemsetAsync kc");
    hip_check(hipMemsetAsync(d_vc, 0xFF, cache_bytes, st), "hipMemsetAsync vc");
    kvq_check(kvq_cache_write(d_k, d_v, (int64_t)Hkv * D, d_slots, T, Hkv, D, d_kc, d_vc, num_blocks, 16, kv_dtype,
                              scale[0], scale[1], st),
              "kvq_cache_write");

    // decode attention, fp32 output
    const size_t ws_bytes = kvq_decode_workspace_bytes_ex(B, Hq, Hkv, D, max_seq_len, 16, split);
    if (ws_bytes == 0) die("kvq_decode_workspace_bytes_ex", -103);
    void* d_ws = nullptr;
    float* d_out = nullptr;
    hip_check(hipMalloc(&d_ws, ws_bytes), "hipMalloc workspace");
    hip_check(hipMalloc(&d_out, (size_t)B * Hq * D * sizeof(float)), "hipMalloc out");
    kvq_check(kvq_paged_decode_attn_ex(d_q, d_kc, d_vc, kv_dtype, d_bt, max_blocks, d_sl, max_seq_len, B, Hq, Hkv, D,
                                       16, num_blocks, scale[0], scale[1], sm_scale, d_out, KVQ_OUT_F32, d_ws,
                                       ws_bytes, st, KVQ_IMPL_AUTO, split),
              "kvq_paged_decode_attn_ex");

    std::vector<float> out((size_t)B * Hq * D);
    std::vector<uint8_t> kc(cache_bytes), vc(cache_bytes);
    hip_check(hipMemcpyAsync(out.data(), d_out, out.size() * sizeof(float), hipMemcpyDeviceToHost, st), "D2H out");
    hip_check(hipMemcpyAsync(kc.data(), d_kc, cache_bytes, hipMemcpyDeviceToHost, st), "D2H kc");
    hip_check(hipMemcpyAsync(vc.data(), d_vc, cache_bytes, hipMemcpyDeviceToHost, st), "D2H vc");
    hip_check(hipStreamSynchronize(st), "hipStreamSynchronize");
    write_file(dir + "/out.bin", out);
    write_file(dir + "/kc.bin", kc);
    write_file(dir + "/vc.bin", vc);
    {
        FILE* f = std::fopen((dir + "/scales.txt").c_str(), "w");
        if (!f) die("scales.txt", -104);
        std::fprintf(f, "%a %a %a %a\n", (double)amax[0], (double)amax[1], (double)scale[0], (double)scale[1]);
        std::fclose(f);
    }
    for (void* p : {(void*)d_q, (void*)d_k, (void*)d_v, (void*)d_slots, (void*)d_bt, (void*)d_sl, (void*)d_amax, d_kc,
                    d_vc, d_ws, (void*)d_out})
        hip_check(hipFree(p), "hipFree");
    hip_check(hipStreamDestroy(st), "hipStreamDestroy");
    std::printf("decode_client: ok\n");
    return 0;
}
