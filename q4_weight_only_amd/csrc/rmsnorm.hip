// rmsnorm.hip -- RMSNorm of bf16 activation rows ahead of a prefill
// projection (M > 1): x_hat = bf16(x * r * gamma), r = 1 / sqrt(mean(x^2) +
// eps) over the row's K values (genie-ai-runtime README, "At a glance":
// fused RMSNorm + RoPE + SwiGLU kernels; the norm is Qwen3's).
//
// At M = 1 the norm is fused into the decode GEMV's x staging (gemv.hip).  At
// M > 1 a matmul workgroup sees only part of K for only some rows, and every
// column tile would repeat the row's norm, so the rows are normalised once,
// here, into a bf16 buffer that the matmul reads like any X.
//
// One workgroup of 256 threads per row.  Thread t holds 16-byte chunks t,
// t + 256, ... of the row (8 bf16 each) and of gamma, so the sum of squares,
// its reduction order (the thread's chunks in order, a butterfly over the
// wave's lanes, then the four waves as (w0 + w1) + (w2 + w3)) and the
// products are those of the fused GEMV: both paths give the same x_hat.
// HBM-bound: 2 bytes read and 2 written per value (gamma stays in L2).
#include "q4k_device.h"

namespace jq4k {

constexpr int kNormThreads = 256;
constexpr int kNormMaxChunks = 16384 / 8 / kNormThreads;   // K <= 16384

__device__ __forceinline__ float norm_bf16_lo(uint32_t v) { return __builtin_bit_cast(float, v << 16); }
__device__ __forceinline__ float norm_bf16_hi(uint32_t v) {
    return __builtin_bit_cast(float, v & 0xFFFF0000u);
}

__global__ __launch_bounds__(kNormThreads) void rmsnorm_rows_kernel(
    const uint4* X, const uint4* __restrict__ gamma, float eps, uint4* Xh, int K) {
    const int t = threadIdx.x;
    const int nxc = K / 8;   // 16-byte chunks per row
    const long base = static_cast<long>(blockIdx.x) * nxc;
    uint4 xv[kNormMaxChunks], gv[kNormMaxChunks];
    // loads never under a thread-dependent branch (past the row's end a
    // repeat of its last chunk; the count of chunks is the same for all)
#pragma unroll
    for (int j = 0; j < kNormMaxChunks; ++j) {
        if (j * kNormThreads < nxc) {
            const int g = min(t + j * kNormThreads, nxc - 1);
            xv[j] = X[base + g];
            gv[j] = gamma[g];
        }
    }
    float ss = 0.f;
#pragma unroll
    for (int j = 0; j < kNormMaxChunks; ++j)
        if (t + j * kNormThreads < nxc) {
            const uint32_t w[4] = {xv[j].x, xv[j].y, xv[j].z, xv[j].w};
#pragma unroll
            for (int e = 0; e < 4; ++e)
                ss += norm_bf16_lo(w[e]) * norm_bf16_lo(w[e]) +
                      norm_bf16_hi(w[e]) * norm_bf16_hi(w[e]);
        }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) ss += __shfl_xor(ss, o);
    __shared__ float wave_ss[kNormThreads / 64];
    if ((t & 63) == 0) wave_ss[t >> 6] = ss;
    __syncthreads();
    const float total = (wave_ss[0] + wave_ss[1]) + (wave_ss[2] + wave_ss[3]);
    const float r = rsqrtf(total / static_cast<float>(K) + eps);
#pragma unroll
    for (int j = 0; j < kNormMaxChunks; ++j)
        if (t + j * kNormThreads < nxc) {
            const uint32_t w[4] = {xv[j].x, xv[j].y, xv[j].z, xv[j].w};
            const uint32_t q[4] = {gv[j].x, gv[j].y, gv[j].z, gv[j].w};
            uint32_t o[4];
#pragma unroll
            for (int e = 0; e < 4; ++e)
                o[e] = pack_bf16x2(norm_bf16_lo(w[e]) * r * norm_bf16_lo(q[e]),
                                   norm_bf16_hi(w[e]) * r * norm_bf16_hi(q[e]));
            Xh[base + t + j * kNormThreads] = make_uint4(o[0], o[1], o[2], o[3]);
        }
}

hipError_t launch_rmsnorm_rows(const uint16_t* X, const uint16_t* gamma, float eps, uint16_t* Xh,
                               int M, int K, hipStream_t stream) {
    hipLaunchKernelGGL(rmsnorm_rows_kernel, dim3(static_cast<unsigned>(M)), dim3(kNormThreads), 0,
                       stream, reinterpret_cast<const uint4*>(X),
                       reinterpret_cast<const uint4*>(gamma), eps, reinterpret_cast<uint4*>(Xh),
                       K);
    return hipGetLastError();
}

}  // namespace jq4k
