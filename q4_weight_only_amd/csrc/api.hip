// api.hip -- the C ABI of libjq4k: argument checks, kernel choice, launch.
// Every check runs before the first HIP call, so rejected calls launch
// nothing and can be exercised without a GPU.
#include <atomic>
#include <mutex>
#include <stdint.h>

#include "jq4k.h"
#include "q4k_device.h"
#include "tile_sched.h"

namespace jq4k {
hipError_t launch_gemv(const uint8_t* W, const uint16_t* X, float* Y, int N, int K, int R,
                       hipStream_t stream);
size_t gemv_lds_bytes(int nb, int R, int mats);
hipError_t launch_gemv_batched(const uint8_t* const* W, const uint16_t* const* X,
                               float* const* Y, const int* N, const int* K, const int* R,
                               int count, hipStream_t stream);
hipError_t launch_gemm_mfma(const uint8_t* const* W, const uint16_t* const* X, float* const* Y,
                            const int* M, const int* N, const int* K, int count, int tile,
                            hipStream_t stream);
long gemm_launch_size(const int* M, const int* N, int count, int tile,
                      const int* splits = nullptr);
constexpr int kTileBig = 512;   // tile code of the 256 x 256 kernel (gemm_big.hip)
constexpr int kTileRw = 1024;   // tile code of the register-W 256 x 256 kernel (gemm_rw.hip)
long gemm_splitk_plan(const int* M, const int* N, const int* K, int count, long min_items,
                      int* splits);
hipError_t launch_gemm_skinny(const uint8_t* const* W, const uint16_t* const* X,
                              float* const* Y, const int* M, const int* N, const int* K,
                              int count, const int* splits, void* ws, hipStream_t stream);
hipError_t launch_gemm_swiglu(const uint8_t* Wg, const uint8_t* Wu, const uint16_t* X, float* H,
                              int M, int N, int K, hipStream_t stream);
long gemm_swiglu_launch_size(int M, int N);
hipError_t launch_rmsnorm_rows(const uint16_t* X, const uint16_t* gamma, float eps, uint16_t* Xh,
                               int M, int K, hipStream_t stream);
hipError_t launch_gemv_rmsnorm(const uint8_t* W, const uint16_t* X, const uint16_t* gamma,
                               float eps, float* Y, int N, int K, int R, hipStream_t stream);
hipError_t launch_gemv_swiglu(const uint8_t* Wg, const uint8_t* Wu, const uint16_t* X, float* H,
                              int N, int K, int R, hipStream_t stream);

hipError_t launch_kv_quant(const uint16_t* v, int8_t* q, float* scale, long nvec, int dim,
                           hipStream_t stream);
hipError_t launch_kv_dequant(const int8_t* q, const float* scale, uint16_t* v, long nvec, int dim,
                             hipStream_t stream);
long kv_grid(long nvec, int dim);

hipError_t launch_unpack_fields(const uint8_t* W, long nblocks, uint8_t* q, uint8_t* sc,
                                uint8_t* m, hipStream_t stream);
hipError_t launch_dequant_f32(const uint8_t* W, long nblocks, float* w, hipStream_t stream);
hipError_t launch_dequant_bf16(const uint8_t* W, long nblocks, uint16_t* w, hipStream_t stream);
}  // namespace jq4k

static_assert(JQ4K_GEMM_BATCH_MAX <= jq4k::kSchedMax, "one launch per grouped matmul");

// The split-K workspace of the allocation-free grouped matmul
// (jq4k_gemm_batched_noalloc, below): one copy per GPU.
static_assert(JQ4K_SCRATCH_BYTES % 256 == 0, "whole 256-byte lines");
static __device__ __align__(256) uint8_t scratch[JQ4K_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
constexpr int kQuickReturn = 1;
constexpr int kGemvMaxRows = 1024;
// blocks of W per workgroup for large single GEMVs, at most (measured best
// on the 151936 x 2560 LM head), and about, inside batched launches
// (measured best on the seven projections of a decode layer: 745
// workgroups, all resident at once)
constexpr int kGemvLargeBlocksPerWg = 240;
constexpr int kGemvBatchBlocksPerWg = 512;
// x staged as binary16 with its sums takes 608 B of LDS per 256 values
// (38 KB at the largest K); each block of W a workgroup owns adds 16 B
constexpr size_t kGemvLdsLimit = 96 * 1024;

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

// Rows per workgroup for about `per_wg` blocks of W of K-long rows (the
// nearest whole number of rows, at least `min_rows`), within N and the LDS
// budget.
int gemv_rows_for(int per_wg, int min_rows, int N, int K, int mats) {
    const int nb = K / jq4k::kQK;
    long R = (2L * per_wg / nb + 1) / 2;
    if (R < min_rows) R = min_rows;
    if (R > N) R = N;
    if (R > kGemvMaxRows) R = kGemvMaxRows;
    if (R < 1) R = 1;
    while (R > 1 && jq4k::gemv_lds_bytes(nb, static_cast<int>(R), mats) > kGemvLdsLimit) --R;
    return static_cast<int>(R);
}

// Rows spreading `blocks` blocks of W (`problems` problems, `mats` matrices
// per row) over about one workgroup per CU: for launches whose usual rows
// leave CUs idle.  A small launch is latency-bound, and every CU streaming
// part of it beats fewer, longer workgroups (the 2560 x 2560 GEMV: 4.9 ->
// 4.2 us with 11 rows instead of 16; a decode step of four dependent
// grouped launches: 33.4 -> 29.8 us; two to four workgroups per CU
// measured slower).  The rows then fill the kernel rounds (128 blocks)
// that share needs, so that no round runs nearly empty: the same time per
// workgroup, fewer workgroups (decode step 28.8 -> 28.3 us, 2560 x 2560
// GEMV 3.94 -> 3.88 us; one round fewer and more workgroups measured
// slower).
int gemv_spread_rows(long blocks, int problems, int N, int K, int mats) {
    const int nb = K / jq4k::kQK;
    const long slots = static_cast<long>(cu_count()) - problems;
    const long per_wg = slots > 0 ? (blocks + slots - 1) / slots : blocks;
    const long row_blocks = static_cast<long>(mats) * nb;
    const long rounds = (per_wg + 127) / 128;
    long R = rounds * 128 / row_blocks;
    if (R < 1) R = (per_wg + row_blocks - 1) / row_blocks;
    if (R < 1) R = 1;
    if (R > N) R = N;
    while (R > 1 && jq4k::gemv_lds_bytes(nb, static_cast<int>(R), mats) > kGemvLdsLimit) --R;
    return static_cast<int>(R);
}

// Rows per workgroup of the GEMV.  A matrix that 16-row workgroups would
// not spread over every CU takes the spread rule (gemv_spread_rows); a
// larger one as many whole rows as fit in kGemvLargeBlocksPerWg blocks of W,
// or 16 rows when that leaves CUs without a workgroup (4096 x 2560: 4.74 us
// with 16 rows, 4.82 spread).  The
// kernel's rounds take 128 blocks, so the budget is just under two rounds:
// short-lived workgroups, none paying for a nearly empty round.  Measured:
// the 151936 x 2560 LM head with 24 rows 39.6-39.9 us against 40.5-41.1 us
// with 48 (480 blocks, the earlier rule; 36 to 76 rows 40.3-41.1); a
// 9728 x 2560 projection alone 6.4 us against 8.0 with 16 rows (160 blocks,
// 1.25 rounds), and with its RMSNorm fused 6.7 against 8.6.  The LM head
// with 26 rows (260 blocks, just past two rounds) takes 46 us, with 13 rows
// (130) 64 us.  The spread rule stays better for the 2560-row projections
// (2560 x 9728: 7.05 us against 7.34 with 6 rows).  Bounded by the LDS
// budget.
int gemv_rows_per_block(int N, int K) {
    const int nb = K / jq4k::kQK;
    const long spread_blocks = static_cast<long>(N) * nb;
    if ((N + 15) / 16 < cu_count()) return gemv_spread_rows(spread_blocks, 1, N, K, 1);
    int R = kGemvLargeBlocksPerWg / nb;
    R = gemv_rows_for((R < 1 ? 1 : R) * nb, 1, N, K, 1);
    if ((N + R - 1) / R >= cu_count()) return R;
    return gemv_rows_for(16 * nb, 1, N, K, 1);
}

// Rows per workgroup inside a batched launch.  A batch that fills the GPU
// takes about kGemvBatchBlocksPerWg blocks of W per workgroup whatever the
// row length, and at least 16 rows; a smaller one is spread over the CUs.
// The decode layer: 51 rows at K = 2560, 32 at 4096, 16 at 9728, 745
// workgroups, all resident at once, 14.0 us.  Measured no better: 14 or 15
// rows at K = 9728; slower: 13 (782 workgroups, 17.0 us, with an earlier
// kernel), 52/33/14 rows (756, 15.5), more blocks for longer rows (55/36/17
// to 67/48/29, 15.3-17.1), 384 and 640 blocks, LDS padded to hold at most 3
// or 4 workgroups per CU (19.5, 15.5).
int gemv_batch_rows(int N, int K) { return gemv_rows_for(kGemvBatchBlocksPerWg, 16, N, K, 1); }

int run_gemv(const block_q4_K* W, const jq4k_bf16* X, float* Y, int N, int K, int R,
             hipStream_t stream) {
    if (R <= 0) R = gemv_rows_per_block(N, K);
    const hipError_t e = jq4k::launch_gemv(reinterpret_cast<const uint8_t*>(W), X, Y, N, K, R,
                                           stream);
    return static_cast<int>(e);
}

// MFMA tile (rows of M per workgroup) for the largest M of a launch: 64 up
// to M = 64; then 128; 256 from M = 2048 for a single matmul and from M = 512
// for a grouped launch, whose several problems fill the GPU with fewer,
// larger tiles (measured on the Qwen3-4B projections at M = 128 .. 4096).
// A 256-row launch runs the wave-specialised 256 x 128 kernel, or the
// register-W 256 x 256 one where rw_pays (below).
int mfma_tile_for(int M, bool grouped) {
    if (M <= 64) return 64;
    return M >= (grouped ? 512 : 2048) ? 256 : 128;
}

// A launch of 256-row tiles moves to the register-W kernel (gemm_rw.hip,
// one workgroup per CU) once its 256 x 256 output tiles give every CU at
// least kRwTilesPerCu of them: below that the tail of the one-per-CU kernel
// costs more than it saves (Qwen3-4B at M = 2048: the seven-projection layer,
// 3.75 tiles per CU, 422 vs 466 us; gate alone, 1.2 per CU, 147 vs 134 us;
// the LM head at M = 512, 4.6 per CU, 399 vs 475 us).
constexpr long kRwTilesPerCu = 3;

bool rw_pays(const int* M, const int* N, int count) {
    long tiles = 0;
    for (int i = 0; i < count; ++i)
        tiles += static_cast<long>((M[i] + 255) / 256) * ((N[i] + 255) / 256);
    return tiles >= kRwTilesPerCu * cu_count();
}

int run_mfma(const block_q4_K* W, const jq4k_bf16* X, float* Y, int M, int N, int K, int tile,
             hipStream_t stream) {
    if (K > JQ4K_MFMA_MAX_K) return JQ4K_EINVAL;
    if (jq4k::gemm_launch_size(&M, &N, 1, tile) > 0x7FFFFFFFL) return JQ4K_EINVAL;
    const uint8_t* w = reinterpret_cast<const uint8_t*>(W);
    return static_cast<int>(jq4k::launch_gemm_mfma(&w, &X, &Y, &M, &N, &K, 1, tile, stream));
}

// The small-M kernel (M <= 64), whole K per workgroup.
int run_skinny(const block_q4_K* W, const jq4k_bf16* X, float* Y, int M, int N, int K,
               hipStream_t stream) {
    if (M > 64 || K > JQ4K_MFMA_MAX_K) return JQ4K_EINVAL;
    if (jq4k::gemm_launch_size(&M, &N, 1, 64) > 0x7FFFFFFFL) return JQ4K_EINVAL;
    const uint8_t* w = reinterpret_cast<const uint8_t*>(W);
    return static_cast<int>(
        jq4k::launch_gemm_skinny(&w, &X, &Y, &M, &N, &K, 1, nullptr, nullptr, stream));
}

// The MFMA kernel for the shape: small-M up to M = 64, else the tile of
// mfma_tile_for.
int run_mfma_auto(const block_q4_K* W, const jq4k_bf16* X, float* Y, int M, int N, int K,
                  hipStream_t stream) {
    if (M <= 64) return run_skinny(W, X, Y, M, N, K, stream);
    int tile = mfma_tile_for(M, false);
    // A single matmul wide enough to give every CU two 256 x 128 tiles
    // takes the 256-row kernel from M = 512, as a grouped launch does
    // (the 151936-row LM head at M = 512: 562 vs 705 us with 128 rows).
    if (tile == 128 && M >= 512 &&
        static_cast<long>((M + 255) / 256) * ((N + 127) / 128) >= 2L * cu_count())
        tile = 256;
    if (tile == 256 && rw_pays(&M, &N, 1)) tile = jq4k::kTileRw;
    return run_mfma(W, X, Y, M, N, K, tile, stream);
}

// The problems of a grouped matmul, checked, with the empty ones dropped.
struct GemmBatchArgs {
    const uint8_t* W[JQ4K_GEMM_BATCH_MAX];
    const uint16_t* X[JQ4K_GEMM_BATCH_MAX];
    float* Y[JQ4K_GEMM_BATCH_MAX];
    int M[JQ4K_GEMM_BATCH_MAX], N[JQ4K_GEMM_BATCH_MAX], K[JQ4K_GEMM_BATCH_MAX];
    int live = 0, max_m = 0, tile = 0;
};

// 0 = go (a.live > 0), kQuickReturn = nothing to do, < 0 = error code.
int collect_gemm_batch(const jq4k_gemm_desc* problems, int count, GemmBatchArgs& a) {
    if (count < 0 || count > JQ4K_GEMM_BATCH_MAX) return JQ4K_EINVAL;
    if (count == 0) return kQuickReturn;
    if (problems == nullptr) return JQ4K_EINVAL;
    for (int i = 0; i < count; ++i) {
        const jq4k_gemm_desc& d = problems[i];
        const int rc = check_matmul(d.W, d.X, d.Y, d.M, d.N, d.K);
        if (rc == kQuickReturn) continue;
        if (rc != 0) return rc;
        a.W[a.live] = reinterpret_cast<const uint8_t*>(d.W);
        a.X[a.live] = d.X;
        a.Y[a.live] = d.Y;
        a.M[a.live] = d.M;
        a.N[a.live] = d.N;
        a.K[a.live] = d.K;
        a.max_m = d.M > a.max_m ? d.M : a.max_m;
        ++a.live;
    }
    if (a.live == 0) return kQuickReturn;
    for (int i = 0; i < a.live; ++i)
        if (a.K[i] > JQ4K_MFMA_MAX_K) return JQ4K_EINVAL;
    a.tile = mfma_tile_for(a.max_m, true);
    if (a.tile == 256 && rw_pays(a.M, a.N, a.live)) a.tile = jq4k::kTileRw;
    if (jq4k::gemm_launch_size(a.M, a.N, a.live, a.tile) > 0x7FFFFFFFL) return JQ4K_EINVAL;
    return 0;
}

// Split K applies to the 64-row tiles (M <= 64), whose launches are short of
// workgroups and whose long-K problems would otherwise run alone at the end.
// Returns the workspace bytes (0: no problem splits) and the K ranges.
long splitk_for(const GemmBatchArgs& a, int* splits) {
    for (int i = 0; i < a.live; ++i) splits[i] = 1;
    if (a.tile != 64) return 0;
    return jq4k::gemm_splitk_plan(a.M, a.N, a.K, a.live, 2L * cu_count(), splits);
}

// The launch of a checked batch: M <= 64 (the 64-row tile) on the small-M
// kernel of gemm_skinny.hip (split K when `splits` is given), else the MFMA
// tile the batch's largest M picks.
int launch_batch(const GemmBatchArgs& a, const int* splits, void* ws, hipStream_t stream) {
    if (a.tile == 64)
        return static_cast<int>(jq4k::launch_gemm_skinny(a.W, a.X, a.Y, a.M, a.N, a.K, a.live,
                                                         splits, ws, stream));
    return static_cast<int>(
        jq4k::launch_gemm_mfma(a.W, a.X, a.Y, a.M, a.N, a.K, a.live, a.tile, stream));
}

// KV convert: 0 = go, kQuickReturn = nothing to do, < 0 = error code.
int check_kv(const void* in, const void* out, const float* scale, long nvec, int dim,
             uintptr_t v_align, uintptr_t q_align, const void* v, const void* q) {
    if (nvec < 0 || dim < 8 || dim > JQ4K_KV_MAX_DIM || dim % 8 != 0) return JQ4K_EINVAL;
    if (nvec == 0) return kQuickReturn;
    if (nvec > 0x7FFFFFFFFFFFFFFFL / dim) return JQ4K_EINVAL;
    if (in == nullptr || out == nullptr || scale == nullptr) return JQ4K_EINVAL;
    if (misaligned(v, v_align) || misaligned(q, q_align) || misaligned(scale, 4))
        return JQ4K_EALIGN;
    if (jq4k::kv_grid(nvec, dim) > 0x7FFFFFFFL) return JQ4K_EINVAL;
    return 0;
}

int check_export(const void* W, long nblocks, const void* out, uintptr_t out_align) {
    if (nblocks < 0) return JQ4K_EINVAL;
    if (nblocks == 0) return kQuickReturn;
    if (nblocks > (0x7FFFFFFFFFFFFFFFL / jq4k::kQK)) return JQ4K_EINVAL;
    if (W == nullptr || out == nullptr) return JQ4K_EINVAL;
    if (misaligned(W, 16) || misaligned(out, out_align)) return JQ4K_EALIGN;
    return 0;
}

// ---- the allocation-free grouped matmul (jq4k_gemm_batched_noalloc) ----
// Its split-K workspace is this static device array: every GPU the library
// runs on holds one copy, at its own address, until the process ends.  Host
// code never uses the name as an address (on the host it is only a stand-in):
// hipGetSymbolAddress gives each device's address once, with that device
// current, and the kernels get that pointer.
__global__ void scratch_clear_kernel(uint4* p, long n) {
    for (long i = blockIdx.x * static_cast<long>(blockDim.x) + threadIdx.x; i < n;
         i += static_cast<long>(gridDim.x) * blockDim.x)
        p[i] = make_uint4(0u, 0u, 0u, 0u);
}

struct ScratchSlot {
    std::once_flag once;
    void* ptr = nullptr;
    int rc = 0;
};
ScratchSlot g_scratch[kMaxDevices];

// The current device's scratch address, set up on the first call there: the
// symbol's address, then one clear of the whole array on `stream` (the
// split-K counters must start at zero; every call leaves them at zero).
int device_scratch(hipStream_t stream, void** out) {
    int dev = 0;
    const hipError_t ge = hipGetDevice(&dev);
    if (ge != hipSuccess) return static_cast<int>(ge);
    if (dev < 0 || dev >= kMaxDevices) return JQ4K_EINVAL;
    ScratchSlot& s = g_scratch[dev];
    std::call_once(s.once, [&] {
        void* p = nullptr;
        hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || p == nullptr) {
            s.rc = e != hipSuccess ? static_cast<int>(e) : static_cast<int>(hipErrorInvalidSymbol);
            return;
        }
        hipLaunchKernelGGL(scratch_clear_kernel, dim3(256), dim3(256), 0, stream,
                           static_cast<uint4*>(p), static_cast<long>(JQ4K_SCRATCH_BYTES / 16));
        e = hipGetLastError();
        if (e != hipSuccess) {
            s.rc = static_cast<int>(e);
            return;
        }
        s.ptr = p;
    });
    if (s.rc != 0) return s.rc;
    *out = s.ptr;
    return 0;
}

}  // namespace

extern "C" {

int jq4k_gemv(const block_q4_K* W, const jq4k_bf16* X, float* Y, int M, int N, int K,
              hipStream_t stream) {
    if (M != 1 || K > JQ4K_GEMV_MAX_K) return JQ4K_EINVAL;
    const int rc = check_matmul(W, X, Y, M, N, K);
    if (rc != 0) return rc == kQuickReturn ? JQ4K_OK : rc;
    return run_gemv(W, X, Y, N, K, 0, stream);
}

int jq4k_gemv_rows(const block_q4_K* W, const jq4k_bf16* X, float* Y, int N, int K,
                   int rows_per_block, hipStream_t stream) {
    if (rows_per_block < 0 || K > JQ4K_GEMV_MAX_K) return JQ4K_EINVAL;
    const int rc = check_matmul(W, X, Y, 1, N, K);
    if (rc != 0) return rc == kQuickReturn ? JQ4K_OK : rc;
    if (rows_per_block > 0 &&
        jq4k::gemv_lds_bytes(K / jq4k::kQK, rows_per_block, 1) > kGemvLdsLimit)
        return JQ4K_EINVAL;
    return run_gemv(W, X, Y, N, K, rows_per_block, stream);
}

int jq4k_gemv_batched(const jq4k_gemv_desc* problems, int count, hipStream_t stream) {
    if (count < 0 || count > JQ4K_GEMV_BATCH_MAX) return JQ4K_EINVAL;
    if (count == 0) return JQ4K_OK;
    if (problems == nullptr) return JQ4K_EINVAL;
    const uint8_t* W[JQ4K_GEMV_BATCH_MAX];
    const uint16_t* X[JQ4K_GEMV_BATCH_MAX];
    float* Y[JQ4K_GEMV_BATCH_MAX];
    int N[JQ4K_GEMV_BATCH_MAX], K[JQ4K_GEMV_BATCH_MAX], R[JQ4K_GEMV_BATCH_MAX];
    int live = 0;
    long wgs = 0;
    for (int i = 0; i < count; ++i) {
        const jq4k_gemv_desc& d = problems[i];
        if (d.K > JQ4K_GEMV_MAX_K) return JQ4K_EINVAL;
        const int rc = check_matmul(d.W, d.X, d.Y, 1, d.N, d.K);
        if (rc == kQuickReturn) continue;
        if (rc != 0) return rc;
        W[live] = reinterpret_cast<const uint8_t*>(d.W);
        X[live] = d.X;
        Y[live] = d.Y;
        N[live] = d.N;
        K[live] = d.K;
        ++live;
    }
    if (live == 0) return JQ4K_OK;
    for (int i = 0; i < live; ++i) {
        R[i] = gemv_batch_rows(N[i], K[i]);
        wgs += (static_cast<long>(N[i]) + R[i] - 1) / R[i];
    }
    if (wgs < cu_count()) {
        long blocks = 0;
        for (int i = 0; i < live; ++i) blocks += static_cast<long>(N[i]) * (K[i] / jq4k::kQK);
        wgs = 0;
        for (int i = 0; i < live; ++i) {
            R[i] = gemv_spread_rows(blocks, live, N[i], K[i], 1);
            wgs += (static_cast<long>(N[i]) + R[i] - 1) / R[i];
        }
    }
    if (wgs > 0x7FFFFFFFL) return JQ4K_EINVAL;
    return static_cast<int>(jq4k::launch_gemv_batched(W, X, Y, N, K, R, live, stream));
}

int jq4k_gemm_batched(const jq4k_gemm_desc* problems, int count, hipStream_t stream) {
    GemmBatchArgs a;
    const int rc = collect_gemm_batch(problems, count, a);
    if (rc != 0) return rc == kQuickReturn ? JQ4K_OK : rc;
    return launch_batch(a, nullptr, nullptr, stream);
}

int jq4k_gemm_workspace_size(const jq4k_gemm_desc* problems, int count, size_t* bytes) {
    if (bytes == nullptr) return JQ4K_EINVAL;
    *bytes = 0;
    GemmBatchArgs a;
    const int rc = collect_gemm_batch(problems, count, a);
    if (rc != 0) return rc == kQuickReturn ? JQ4K_OK : rc;
    int splits[JQ4K_GEMM_BATCH_MAX];
    *bytes = static_cast<size_t>(splitk_for(a, splits));
    return JQ4K_OK;
}

int jq4k_gemm_batched_ws(const jq4k_gemm_desc* problems, int count, void* workspace,
                         size_t workspace_bytes, hipStream_t stream) {
    GemmBatchArgs a;
    const int rc = collect_gemm_batch(problems, count, a);
    if (rc != 0) return rc == kQuickReturn ? JQ4K_OK : rc;
    int splits[JQ4K_GEMM_BATCH_MAX];
    const long need = splitk_for(a, splits);
    if (need == 0) return launch_batch(a, nullptr, nullptr, stream);
    if (workspace == nullptr || workspace_bytes < static_cast<size_t>(need)) return JQ4K_EINVAL;
    if (misaligned(workspace, 256)) return JQ4K_EALIGN;
    if (jq4k::gemm_launch_size(a.M, a.N, a.live, a.tile, splits) > 0x7FFFFFFFL)
        return JQ4K_EINVAL;
    return launch_batch(a, splits, workspace, stream);
}

int jq4k_gemm_batched_noalloc(const jq4k_gemm_desc* problems, int count, hipStream_t stream) {
    GemmBatchArgs a;
    const int rc = collect_gemm_batch(problems, count, a);
    if (rc != 0) return rc == kQuickReturn ? JQ4K_OK : rc;
    int splits[JQ4K_GEMM_BATCH_MAX];
    const long need = splitk_for(a, splits);
    if (need == 0) return launch_batch(a, nullptr, nullptr, stream);
    if (static_cast<unsigned long>(need) > JQ4K_SCRATCH_BYTES) return JQ4K_ESCRATCH;
    if (jq4k::gemm_launch_size(a.M, a.N, a.live, a.tile, splits) > 0x7FFFFFFFL)
        return JQ4K_EINVAL;
    void* ws = nullptr;
    const int src = device_scratch(stream, &ws);
    if (src != 0) return src;
    return launch_batch(a, splits, ws, stream);
}

int jq4k_gemv_rmsnorm(const block_q4_K* W, const jq4k_bf16* X, const jq4k_bf16* gamma,
                      float eps, float* Y, int N, int K, hipStream_t stream) {
    if (K > JQ4K_GEMV_MAX_K || !(eps >= 0.0f) || eps == __builtin_inff()) return JQ4K_EINVAL;
    const int rc = check_matmul(W, X, Y, 1, N, K);
    if (rc != 0) return rc == kQuickReturn ? JQ4K_OK : rc;
    if (gamma == nullptr) return JQ4K_EINVAL;
    if (misaligned(gamma, 16)) return JQ4K_EALIGN;
    const int R = gemv_rows_per_block(N, K);
    return static_cast<int>(jq4k::launch_gemv_rmsnorm(reinterpret_cast<const uint8_t*>(W), X,
                                                      gamma, eps, Y, N, K, R, stream));
}

int jq4k_rmsnorm_bf16(const jq4k_bf16* X, const jq4k_bf16* gamma, float eps, jq4k_bf16* Xhat,
                      int M, int K, hipStream_t stream) {
    if (M < 0 || K <= 0 || K % jq4k::kQK != 0 || K > JQ4K_GEMV_MAX_K) return JQ4K_EINVAL;
    if (!(eps >= 0.0f) || eps == __builtin_inff()) return JQ4K_EINVAL;
    if (M == 0) return JQ4K_OK;
    if (X == nullptr || gamma == nullptr || Xhat == nullptr) return JQ4K_EINVAL;
    if (misaligned(X, 16) || misaligned(gamma, 16) || misaligned(Xhat, 16)) return JQ4K_EALIGN;
    return static_cast<int>(jq4k::launch_rmsnorm_rows(X, gamma, eps, Xhat, M, K, stream));
}

int jq4k_gemm_swiglu(const block_q4_K* Wg, const block_q4_K* Wu, const jq4k_bf16* X, float* H,
                     int M, int N, int K, hipStream_t stream) {
    const int rc = check_matmul(Wg, X, H, M, N, K);
    if (rc != 0) return rc == kQuickReturn ? JQ4K_OK : rc;
    if (Wu == nullptr) return JQ4K_EINVAL;
    if (misaligned(Wu, 16)) return JQ4K_EALIGN;
    const uint8_t* wg = reinterpret_cast<const uint8_t*>(Wg);
    const uint8_t* wu = reinterpret_cast<const uint8_t*>(Wu);
    if (M == 1 && K <= JQ4K_GEMV_MAX_K) {
        // R rows of each matrix per workgroup: as many whole rows as fit,
        // both matrices' blocks together, in the blocks a workgroup of a
        // grouped launch streams (the 9728 x 2560 pair: 25 rows, 500 blocks,
        // 9.2 us; 24 rows 9.2; 26 rows, 520 blocks just past four rounds,
        // 10.1-10.2; 12 rows, the single GEMV's 240 blocks, 10.9)
        const int nb = K / jq4k::kQK;
        const int fit = kGemvBatchBlocksPerWg / (2 * nb);
        int R = gemv_rows_for((fit < 1 ? 1 : fit) * nb, 8, N, K, 2);
        if ((N + R - 1) / R < cu_count())
            R = gemv_spread_rows(2L * N * (K / jq4k::kQK), 1, N, K, 2);
        return static_cast<int>(jq4k::launch_gemv_swiglu(wg, wu, X, H, N, K, R, stream));
    }
    if (K > JQ4K_MFMA_MAX_K) return JQ4K_EINVAL;
    if (jq4k::gemm_swiglu_launch_size(M, N) > 0x7FFFFFFFL) return JQ4K_EINVAL;
    return static_cast<int>(jq4k::launch_gemm_swiglu(wg, wu, X, H, M, N, K, stream));
}

int jq4k_gemm_path(const block_q4_K* W, const jq4k_bf16* X, float* Y, int M, int N, int K,
                   int path, hipStream_t stream) {
    if (path < JQ4K_PATH_AUTO || path > JQ4K_PATH_MFMA_RW) return JQ4K_EINVAL;
    if (path == JQ4K_PATH_GEMV && (M != 1 || K > JQ4K_GEMV_MAX_K)) return JQ4K_EINVAL;
    if (path == JQ4K_PATH_SKINNY && M > 64) return JQ4K_EINVAL;
    const int rc = check_matmul(W, X, Y, M, N, K);
    if (rc != 0) return rc == kQuickReturn ? JQ4K_OK : rc;
    switch (path) {
        case JQ4K_PATH_GEMV: return run_gemv(W, X, Y, N, K, 0, stream);
        case JQ4K_PATH_MFMA: return run_mfma_auto(W, X, Y, M, N, K, stream);
        case JQ4K_PATH_MFMA_T64: return run_mfma(W, X, Y, M, N, K, 64, stream);
        case JQ4K_PATH_MFMA_T128: return run_mfma(W, X, Y, M, N, K, 128, stream);
        case JQ4K_PATH_MFMA_T256: return run_mfma(W, X, Y, M, N, K, 256, stream);
        case JQ4K_PATH_SKINNY: return run_skinny(W, X, Y, M, N, K, stream);
        case JQ4K_PATH_MFMA_BIG: return run_mfma(W, X, Y, M, N, K, jq4k::kTileBig, stream);
        case JQ4K_PATH_MFMA_RW: return run_mfma(W, X, Y, M, N, K, jq4k::kTileRw, stream);
        default:
            if (M == 1 && K <= JQ4K_GEMV_MAX_K) return run_gemv(W, X, Y, N, K, 0, stream);
            return run_mfma_auto(W, X, Y, M, N, K, stream);
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

int jq4k_kv_quant_i8(const jq4k_f16* v, int8_t* q, float* scale, long nvec, int dim,
                     hipStream_t stream) {
    const int rc = check_kv(v, q, scale, nvec, dim, 16, 8, v, q);
    if (rc != 0) return rc == kQuickReturn ? JQ4K_OK : rc;
    return static_cast<int>(jq4k::launch_kv_quant(v, q, scale, nvec, dim, stream));
}

int jq4k_kv_dequant_f16(const int8_t* q, const float* scale, jq4k_f16* v, long nvec, int dim,
                        hipStream_t stream) {
    const int rc = check_kv(q, v, scale, nvec, dim, 16, 8, v, q);
    if (rc != 0) return rc == kQuickReturn ? JQ4K_OK : rc;
    return static_cast<int>(jq4k::launch_kv_dequant(q, scale, v, nvec, dim, stream));
}

const char* jq4k_strerror(int code) {
    switch (code) {
        case JQ4K_OK: return "success";
        case JQ4K_EINVAL: return "invalid argument";
        case JQ4K_EALIGN: return "misaligned pointer";
        case JQ4K_ESCRATCH: return "problems need more than the static scratch buffer";
        default:
            if (code > 0) return hipGetErrorString(static_cast<hipError_t>(code));
            return "unknown error";
    }
}

int jq4k_version(void) { return 100; }

}  // extern "C"
