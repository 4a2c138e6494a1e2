// api.hip -- the C ABI of libjq4k: argument checks, kernel choice, launch.
// Every check runs before the first HIP call, so rejected calls launch
// nothing and can be exercised without a GPU.
#include <atomic>
#include <stdint.h>

#include "../../include/jq4k.h"
#include "q4k_device.h"

namespace jq4k {
hipError_t launch_gemv(const uint8_t* W, const uint16_t* X, float* Y, int N, int K, int R,
                       hipStream_t stream);
size_t gemv_lds_bytes(int nb, int R);
hipError_t launch_gemm_mfma(const uint8_t* W, const uint16_t* X, float* Y, int M, int N, int K,
                            int tile, hipStream_t stream);
long gemm_tile_count(int M, int N, int tile);
hipError_t launch_unpack_fields(const uint8_t* W, long nblocks, uint8_t* q, uint8_t* sc,
                                uint8_t* m, hipStream_t stream);
hipError_t launch_dequant_f32(const uint8_t* W, long nblocks, float* w, hipStream_t stream);
hipError_t launch_dequant_bf16(const uint8_t* W, long nblocks, uint16_t* w, hipStream_t stream);
}  // namespace jq4k

namespace {

constexpr int kMaxDevices = 64;
constexpr int kQuickReturn = 1;
constexpr int kGemvMaxRows = 64;
constexpr size_t kGemvLdsLimit = 64 * 1024;

std::atomic<int> g_cu_count[kMaxDevices];

// Compute units of the current device (cached; 256 on an MI355X).
int cu_count() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 256;
    int v = g_cu_count[dev].load(std::memory_order_relaxed);
    if (v <= 0) {
        if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            v <= 0)
            v = 256;
        g_cu_count[dev].store(v, std::memory_order_relaxed);
    }
    return v;
}

bool misaligned(const void* p, uintptr_t a) { return reinterpret_cast<uintptr_t>(p) % a != 0; }

// 0 = go, kQuickReturn = nothing to do, < 0 = error code.
int check_matmul(const void* W, const void* X, const void* Y, int M, int N, int K) {
    if (K <= 0 || K % jq4k::kQK != 0 || M < 0 || N < 0) return JQ4K_EINVAL;
    if (M == 0 || N == 0) return kQuickReturn;
    if (W == nullptr || X == nullptr || Y == nullptr) return JQ4K_EINVAL;
    if (misaligned(W, 16) || misaligned(X, 16) || misaligned(Y, 4)) return JQ4K_EALIGN;
    return 0;
}

// Rows per workgroup of the GEMV: enough workgroups to cover every compute
// unit about twice, at most 64 rows, within the LDS budget.
int gemv_rows_per_block(int N, int K) {
    const int nb = K / jq4k::kQK;
    const long want = 2L * cu_count();
    long R = (N + want - 1) / want;
    if (R < 1) R = 1;
    if (R > kGemvMaxRows) R = kGemvMaxRows;
    while (R > 1 && jq4k::gemv_lds_bytes(nb, static_cast<int>(R)) > kGemvLdsLimit) --R;
    return static_cast<int>(R);
}

int run_gemv(const block_q4_K* W, const jq4k_bf16* X, float* Y, int N, int K,
             hipStream_t stream) {
    const hipError_t e = jq4k::launch_gemv(reinterpret_cast<const uint8_t*>(W), X, Y, N, K,
                                           gemv_rows_per_block(N, K), stream);
    return static_cast<int>(e);
}

int mfma_tile_for(int M, int N) {
    if (M <= 64) return 64;
    if (jq4k::gemm_tile_count(M, N, 256) >= cu_count()) return 256;
    return 128;
}

int run_mfma(const block_q4_K* W, const jq4k_bf16* X, float* Y, int M, int N, int K, int tile,
             hipStream_t stream) {
    if (jq4k::gemm_tile_count(M, N, tile) > 0x7FFFFFFFL - 8) return JQ4K_EINVAL;
    const hipError_t e = jq4k::launch_gemm_mfma(reinterpret_cast<const uint8_t*>(W), X, Y, M, N,
                                                K, tile, stream);
    return static_cast<int>(e);
}

int check_export(const void* W, long nblocks, const void* out, uintptr_t out_align) {
    if (nblocks < 0) return JQ4K_EINVAL;
    if (nblocks == 0) return kQuickReturn;
    if (nblocks > (0x7FFFFFFFFFFFFFFFL / jq4k::kQK)) return JQ4K_EINVAL;
    if (W == nullptr || out == nullptr) return JQ4K_EINVAL;
    if (misaligned(W, 16) || misaligned(out, out_align)) return JQ4K_EALIGN;
    return 0;
}

}  // namespace

extern "C" {

int jq4k_gemv(const block_q4_K* W, const jq4k_bf16* X, float* Y, int M, int N, int K,
              hipStream_t stream) {
    if (M != 1 || K > JQ4K_GEMV_MAX_K) return JQ4K_EINVAL;
    const int rc = check_matmul(W, X, Y, M, N, K);
    if (rc != 0) return rc == kQuickReturn ? JQ4K_OK : rc;
    return run_gemv(W, X, Y, N, K, stream);
}

int jq4k_gemm_path(const block_q4_K* W, const jq4k_bf16* X, float* Y, int M, int N, int K,
                   int path, hipStream_t stream) {
    if (path < JQ4K_PATH_AUTO || path > JQ4K_PATH_MFMA_T256) return JQ4K_EINVAL;
    if (path == JQ4K_PATH_GEMV && (M != 1 || K > JQ4K_GEMV_MAX_K)) return JQ4K_EINVAL;
    const int rc = check_matmul(W, X, Y, M, N, K);
    if (rc != 0) return rc == kQuickReturn ? JQ4K_OK : rc;
    switch (path) {
        case JQ4K_PATH_GEMV: return run_gemv(W, X, Y, N, K, stream);
        case JQ4K_PATH_MFMA: return run_mfma(W, X, Y, M, N, K, mfma_tile_for(M, N), stream);
        case JQ4K_PATH_MFMA_T64: return run_mfma(W, X, Y, M, N, K, 64, stream);
        case JQ4K_PATH_MFMA_T128: return run_mfma(W, X, Y, M, N, K, 128, stream);
        case JQ4K_PATH_MFMA_T256: return run_mfma(W, X, Y, M, N, K, 256, stream);
        default:
            if (M == 1 && K <= JQ4K_GEMV_MAX_K) return run_gemv(W, X, Y, N, K, stream);
            return run_mfma(W, X, Y, M, N, K, mfma_tile_for(M, N), stream);
    }
}

int jq4k_gemm(const block_q4_K* W, const jq4k_bf16* X, float* Y, int M, int N, int K,
              hipStream_t stream) {
    return jq4k_gemm_path(W, X, Y, M, N, K, JQ4K_PATH_AUTO, stream);
}

int jq4k_unpack_fields(const block_q4_K* W, long nblocks, uint8_t* q, uint8_t* sc, uint8_t* m,
                       hipStream_t stream) {
    int rc = check_export(W, nblocks, q, 1);
    if (rc == 0 && (sc == nullptr || m == nullptr)) rc = JQ4K_EINVAL;
    if (rc != 0) return rc == kQuickReturn ? JQ4K_OK : rc;
    return static_cast<int>(jq4k::launch_unpack_fields(reinterpret_cast<const uint8_t*>(W),
                                                       nblocks, q, sc, m, stream));
}

int jq4k_dequant_f32(const block_q4_K* W, long nblocks, float* w, hipStream_t stream) {
    const int rc = check_export(W, nblocks, w, 4);
    if (rc != 0) return rc == kQuickReturn ? JQ4K_OK : rc;
    return static_cast<int>(
        jq4k::launch_dequant_f32(reinterpret_cast<const uint8_t*>(W), nblocks, w, stream));
}

int jq4k_dequant_bf16(const block_q4_K* W, long nblocks, jq4k_bf16* w, hipStream_t stream) {
    const int rc = check_export(W, nblocks, w, 4);
    if (rc != 0) return rc == kQuickReturn ? JQ4K_OK : rc;
    return static_cast<int>(
        jq4k::launch_dequant_bf16(reinterpret_cast<const uint8_t*>(W), nblocks, w, stream));
}

const char* jq4k_strerror(int code) {
    switch (code) {
        case JQ4K_OK: return "success";
        case JQ4K_EINVAL: return "invalid argument";
        case JQ4K_EALIGN: return "misaligned pointer";
        default:
            if (code > 0) return hipGetErrorString(static_cast<hipError_t>(code));
            return "unknown error";
    }
}

int jq4k_version(void) { return 100; }

}  // extern "C"
