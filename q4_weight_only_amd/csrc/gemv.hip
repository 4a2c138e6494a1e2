// gemv.hip -- the M = 1 (decode) Q4_K GEMV for gfx950.
//
// y[n] = sum_k w[n][k] x[k], weights dequantised in registers and never
// materialised (genie-ai-runtime README, "At a glance": INT4 dequant-fused
// GEMV).  HBM-bound: each weight byte is read once (0.5625 B per weight).
//
// Work decomposition.  A workgroup owns R consecutive rows, i.e. R*nb
// consecutive blocks of W (nb = K/256) -- one contiguous span of memory.  The
// span is cut into tasks of one quarter block each (header + 32 quant bytes
// = 64 weights, sub-blocks 2c and 2c+1); 256 threads sweep the tasks in
// rounds, so lanes 4j..4j+3 of a round take the four quarters of one block
// and every round reads 64 consecutive blocks.  A thread's quarter c = t & 3
// never changes.
//
// Arithmetic per quarter.  With s = a sub-block, the kernel uses
//   sum_{k in s} w_k x_k = d*sc_s * sum (q_k x_k) - dmin*m_s * X_s,
//   X_s = sum_{k in s} x_k,
// and forms sum q_k x_k as sum (128 + q_k) x_k - 128 X_s: a byte permute puts
// each 4-bit code q under the bf16 exponent of 128 (0x43 in the high byte
// gives the exact bf16 value 128 + q), and v_dot2_f32_bf16 multiplies two
// such codes by two bf16 activations per instruction with fp32 accumulation.
// X_s is computed once per workgroup, while x is staged in LDS.  Per 8 weights:
// 3 mask/shift, 4 permutes, 4 dot2 -- no per-weight float conversion.
//
// Reduction.  The four lanes of a block are summed with two DPP quad
// permutes; one value per block goes to LDS; after all rounds each row sums
// its nb block values in order (deterministic, no atomics).
//
// LDS layout of x.  x is stored as 16-byte chunks, chunk g = 32 kb + 8 c + i
// (i = 0..3 the even sub-block, 4..7 the odd one), in groups of 8 per
// (block, quarter) at a stride of 9 chunks (x_group_base), which keeps the
// reads free of bank conflicts and costs no address arithmetic per chunk.
#include "q4k_device.h"

namespace jq4k {

constexpr int kGemvThreads = 256;
constexpr int kGemvBatchMax = 16;  // problems per batched launch

size_t gemv_lds_bytes(int nb, int R);

// x in LDS: the 8 chunks of (block kb, quarter c) -- chunk g = 32 kb + 8 c
// + i of x, i = 0..3 the even sub-block, 4..7 the odd one -- sit at 9 (4 kb
// + c) + i.  The stride of 9 chunks spreads the groups over the banks: the
// 64 lanes of a round read one chunk index i of 64 consecutive groups, and
// 9 m mod 16 takes every 16-byte slot exactly four times, the conflict-free
// case of ds_read_b128.  A thread's 8 reads are one base address plus
// immediate offsets.
constexpr int kXGroupStride = 9;
__device__ __forceinline__ int x_group_base(int kb, int c) { return (4 * kb + c) * kXGroupStride; }
__device__ __forceinline__ int x_chunk_phys(int g) { return (g >> 3) * kXGroupStride + (g & 7); }

__device__ __forceinline__ float bf16_lo(uint32_t v) { return __builtin_bit_cast(float, v << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t v) { return __builtin_bit_cast(float, v & 0xFFFF0000u); }

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                           __builtin_bit_cast(bf16x2_t, b), c, false);
}

// 128 + q as bf16 for bytes 0,1 (SEL01) or 2,3 (SEL23) of a quant word
// whose bytes hold one code each: result lanes (128 + q_lo, 128 + q_hi).
constexpr uint32_t kBf16Exp128 = 0x43434343u;
constexpr uint32_t kSel01 = 0x04010400u;
constexpr uint32_t kSel23 = 0x04030402u;

__device__ __forceinline__ float quant_dot8(uint32_t q4, uint32_t xa, uint32_t xb, float acc) {
    acc = dot2_bf16(__builtin_amdgcn_perm(kBf16Exp128, q4, kSel01), xa, acc);
    acc = dot2_bf16(__builtin_amdgcn_perm(kBf16Exp128, q4, kSel23), xb, acc);
    return acc;
}

__device__ __forceinline__ float quad_sum(float v) {
    // quad_perm [1,0,3,2] then [2,3,0,1]
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                                       0, __builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, false));
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                                       0, __builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, false));
    return v;
}

struct QuarterLoad {
    uint4 hdr, qa, qb;
};

__device__ __forceinline__ QuarterLoad load_quarter(const uint8_t* blk, int c) {
    QuarterLoad r;
    r.hdr = load16(blk);
    r.qa = load16(blk + 16 + 32 * c);
    r.qb = load16(blk + 32 + 32 * c);
    return r;
}

// Contribution of one quarter block to its row: 64 weights.
__device__ __forceinline__ float quarter_dot(const QuarterLoad& ld, int c, const uint4* xs,
                                             int kb, float2 xsum) {
    const float d = half_bits_to_float(ld.hdr.x & 0xFFFFu);
    const float dmin = half_bits_to_float(ld.hdr.x >> 16);
    uint32_t scp, mp;
    scale_min_pair(static_cast<uint32_t>(c), ld.hdr.y, ld.hdr.z, ld.hdr.w, &scp, &mp);

    float acc0 = -128.f * xsum.x;  // -128 X_(2c)
    float acc1 = -128.f * xsum.y;  // -128 X_(2c+1)
    const uint32_t qw[8] = {ld.qa.x, ld.qa.y, ld.qa.z, ld.qa.w,
                            ld.qb.x, ld.qb.y, ld.qb.z, ld.qb.w};
    const uint4* xg = xs + x_group_base(kb, c);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint4 xl = xg[i];
        const uint4 xh = xg[4 + i];
        const uint32_t v0 = qw[2 * i], v1 = qw[2 * i + 1];
        acc0 = quant_dot8(low_quants(v0), xl.x, xl.y, acc0);
        acc0 = quant_dot8(low_quants(v1), xl.z, xl.w, acc0);
        acc1 = quant_dot8(high_quants(v0), xh.x, xh.y, acc1);
        acc1 = quant_dot8(high_quants(v1), xh.z, xh.w, acc1);
    }
    const float sc0 = ubyte_to_float<0>(scp), sc1 = ubyte_to_float<1>(scp);
    const float m0 = ubyte_to_float<0>(mp), m1 = ubyte_to_float<1>(mp);
    const float qx = sc0 * acc0 + sc1 * acc1;
    const float mx = m0 * xsum.x + m1 * xsum.y;
    return d * qx - dmin * mx;
}

// LDS: x chunks (nb*36 x 16 B), per-sub-block sums X_s (nb*8 floats, as a
// float2 (even, odd) per (kb, quarter)), per-block partials (R*nb floats per
// matrix).
constexpr int kGemvDepth = 2;  // quarter tasks in flight per thread (2 measured best: 74 VGPRs, 6 waves per SIMD)
constexpr int kGemvMaxK = 16384;
constexpr int kGemvMaxXChunksPerThread = kGemvMaxK / 8 / kGemvThreads;

// One workgroup's share of a GEMV: rows [tile * R, tile * R + R) of W.
// kPair: the same rows of a second matrix W2 follow in the task list (the
// gate and up projections of an MLP), and the row's output is
// silu(gate) * up (SwiGLU) instead of the dot product.
// kNorm: x is RMS-normalised while it is staged, x_hat = bf16(x / sqrt(
// mean(x^2) + eps) * gamma) (RMSNorm ahead of the projection); the sum of
// squares is reduced in a fixed order (lane butterfly, then the four waves).
template <bool kPair, bool kNorm = false>
__device__ __forceinline__ void gemv_tile(const uint8_t* __restrict__ W,
                                          const uint8_t* __restrict__ W2,
                                          const uint4* __restrict__ X, float* __restrict__ Y,
                                          int N, int nb, int R, long tile, uint4* smem,
                                          const uint4* __restrict__ gamma = nullptr,
                                          float eps = 0.f) {
    uint4* xs = smem;
    float2* xsum = reinterpret_cast<float2*>(xs + nb * 4 * kXGroupStride);
    float* part = reinterpret_cast<float*>(xsum + nb * 4);

    const int t = threadIdx.x;
    const int c = t & 3;
    const long row0 = tile * R;
    const int rows = static_cast<int>(min(static_cast<long>(R), N - row0));
    const int nblk = rows * nb;                       // blocks per matrix
    const int ntask = (kPair ? 2 : 1) * nblk * 4;
    const uint8_t* Wt = W + row0 * nb * kBlockBytes;
    const uint8_t* Wt2 = kPair ? W2 + row0 * nb * kBlockBytes : nullptr;
    // block b of the task list: W's span, then (kPair) W2's
    auto blk_ptr = [&](int b) {
        if (kPair && b >= nblk) return Wt2 + static_cast<long>(b - nblk) * kBlockBytes;
        return Wt + static_cast<long>(b) * kBlockBytes;
    };
    const int b0 = t >> 2;  // this thread's first block; +64 per round

    // Memory requests in the order they are needed (vmcnt retires in order):
    // x first, then the first kGemvDepth rounds of weights, so that staging
    // x waits only for x and each round waits only for its own weights.
    const int nxc = nb * 32;  // 16-byte chunks of x, at most 2048 (K <= 16384)
    uint4 xv[kGemvMaxXChunksPerThread];
    uint4 gv[kNorm ? kGemvMaxXChunksPerThread : 1];
    // Every load below is unconditional, past the end a repeat of the last
    // chunk or block: with loads under branches the compiler's count of
    // loads in flight turns pessimistic at the joins and it waits for all
    // of them, which undoes the prefetch.
    const int nround = (ntask + kGemvThreads - 1) / kGemvThreads;   // same for every thread
    const int nblk_all = ntask >> 2;
    auto round_block = [&](int round) { return min(b0 + 64 * round, nblk_all - 1); };
#pragma unroll
    for (int j = 0; j < kGemvMaxXChunksPerThread; ++j) {
        // j beyond the chunks of the largest K: no load at all (compile-time)
        if (j * kGemvThreads < nxc) {
            const int g = min(t + j * kGemvThreads, nxc - 1);
            xv[j] = X[g];
            if constexpr (kNorm) gv[j] = gamma[g];
        }
    }
    QuarterLoad ld[kGemvDepth];
#pragma unroll
    for (int u = 0; u < kGemvDepth; ++u) ld[u] = load_quarter(blk_ptr(round_block(u)), c);

    if constexpr (kNorm) {
        float ss = 0.f;
#pragma unroll
        for (int j = 0; j < kGemvMaxXChunksPerThread; ++j)
            if (t + j * kGemvThreads < nxc) {
                const uint4 v = xv[j];
                const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    ss += bf16_lo(w[e]) * bf16_lo(w[e]) + bf16_hi(w[e]) * bf16_hi(w[e]);
            }
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) ss += __shfl_xor(ss, o);
        __shared__ float wave_ss[kGemvThreads / 64];
        if ((t & 63) == 0) wave_ss[t >> 6] = ss;
        __syncthreads();
        const float total = (wave_ss[0] + wave_ss[1]) + (wave_ss[2] + wave_ss[3]);
        const float r = rsqrtf(total / static_cast<float>(nb * kQK) + eps);
#pragma unroll
        for (int j = 0; j < kGemvMaxXChunksPerThread; ++j)
            if (t + j * kGemvThreads < nxc) {
                const uint32_t w[4] = {xv[j].x, xv[j].y, xv[j].z, xv[j].w};
                const uint32_t q[4] = {gv[j].x, gv[j].y, gv[j].z, gv[j].w};
                uint32_t o[4];
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    o[e] = pack_bf16x2(bf16_lo(w[e]) * r * bf16_lo(q[e]),
                                       bf16_hi(w[e]) * r * bf16_hi(q[e]));
                xv[j] = make_uint4(o[0], o[1], o[2], o[3]);
            }
    }

    // Stage x; each quad of lanes holds one half sub-block (4 chunks of 8),
    // so two DPP steps give X_s for every sub-block.
#pragma unroll
    for (int j = 0; j < kGemvMaxXChunksPerThread; ++j) {
        const int g = t + j * kGemvThreads;
        if (g < nxc) {
            const uint4 v = xv[j];
            xs[x_chunk_phys(g)] = v;
            float sum = ((bf16_lo(v.x) + bf16_hi(v.x)) + (bf16_lo(v.y) + bf16_hi(v.y))) +
                        ((bf16_lo(v.z) + bf16_hi(v.z)) + (bf16_lo(v.w) + bf16_hi(v.w)));
            sum = quad_sum(sum);
            if ((g & 3) == 0) reinterpret_cast<float*>(xsum)[g >> 2] = sum;
        }
    }
    __syncthreads();

    // A round past the thread's last task (the last round of a span whose
    // task count is not a multiple of 256) computes on a repeated block and
    // stores nothing; the four lanes of a block agree, so the quad sum sees
    // only its own block.  The loop runs whole groups of kGemvDepth rounds
    // without a branch; the remaining rounds follow it, without prefetch.
    const int kb_step = 64 % nb;
    int kb = b0 % nb;
    auto task = [&](int round, QuarterLoad& l, bool prefetch) {
        const int b = b0 + 64 * round;
        const float2 xsm = xsum[kb * 4 + c];
        float p = quarter_dot(l, c, xs, kb, xsm);
        p = quad_sum(p);
        if (c == 0 && b < nblk_all) part[b] = p;
        if (prefetch) l = load_quarter(blk_ptr(round_block(round + kGemvDepth)), c);
        kb += kb_step;
        if (kb >= nb) kb -= nb;
    };
    int r0 = 0;
    for (; r0 + kGemvDepth <= nround; r0 += kGemvDepth) {
#pragma unroll
        for (int u = 0; u < kGemvDepth; ++u) task(r0 + u, ld[u], true);
    }
#pragma unroll
    for (int u = 0; u + 1 < kGemvDepth; ++u)
        if (r0 + u < nround) task(r0 + u, ld[u], false);
    __syncthreads();
    for (int r = t; r < rows; r += kGemvThreads) {
        float s = 0.f;
        for (int j = 0; j < nb; ++j) s += part[r * nb + j];
        if constexpr (kPair) {
            float u = 0.f;
            for (int j = 0; j < nb; ++j) u += part[nblk + r * nb + j];
            s = silu(s) * u;
        }
        Y[row0 + r] = s;
    }
}

__global__ __launch_bounds__(kGemvThreads) void q4k_gemv_kernel(
    const uint8_t* __restrict__ W, const uint4* __restrict__ X, float* __restrict__ Y,
    int N, int nb, int R) {
    extern __shared__ uint4 smem[];
    gemv_tile<false>(W, nullptr, X, Y, N, nb, R, blockIdx.x, smem);
}

// RMSNorm ahead of the projection at M = 1: Y = W . x_hat.
__global__ __launch_bounds__(kGemvThreads) void q4k_gemv_rmsnorm_kernel(
    const uint8_t* __restrict__ W, const uint4* __restrict__ X, const uint4* __restrict__ gamma,
    float eps, float* __restrict__ Y, int N, int nb, int R) {
    extern __shared__ uint4 smem[];
    gemv_tile<false, true>(W, nullptr, X, Y, N, nb, R, blockIdx.x, smem, gamma, eps);
}

// SwiGLU of a gate/up pair at M = 1: H[n] = silu(Wg[n] . x) * (Wu[n] . x).
__global__ __launch_bounds__(kGemvThreads) void q4k_gemv_swiglu_kernel(
    const uint8_t* __restrict__ Wg, const uint8_t* __restrict__ Wu, const uint4* __restrict__ X,
    float* __restrict__ H, int N, int nb, int R) {
    extern __shared__ uint4 smem[];
    gemv_tile<true>(Wg, Wu, X, H, N, nb, R, blockIdx.x, smem);
}

// Several independent GEMVs in one launch: workgroups [first[p], first[p+1])
// belong to problem p.  The descriptors travel in the kernel arguments.
struct GemvProblem {
    const uint8_t* W;
    const uint4* X;
    float* Y;
    int N, nb, R;
};

struct GemvBatch {
    GemvProblem p[kGemvBatchMax];
    int first[kGemvBatchMax + 1];
    int count;
};

__global__ __launch_bounds__(kGemvThreads) void q4k_gemv_batched_kernel(const GemvBatch batch) {
    extern __shared__ uint4 smem[];
    const int wg = blockIdx.x;
    int p = 0;
    while (p + 1 < batch.count && wg >= batch.first[p + 1]) ++p;
    const GemvProblem& pr = batch.p[p];
    gemv_tile<false>(pr.W, nullptr, pr.X, pr.Y, pr.N, pr.nb, pr.R, wg - batch.first[p], smem);
}

hipError_t launch_gemv_batched(const uint8_t* const* W, const uint16_t* const* X,
                               float* const* Y, const int* N, const int* K, const int* R,
                               int count, hipStream_t stream) {
    GemvBatch b = {};
    size_t lds = 0;
    int total = 0;
    b.count = count;
    // Problems with the longest rows first (largest K, stable): their
    // workgroups stage the most x before their first weights, and started
    // first they no longer form the tail (decode layer: 15.3 -> 14.9 us with
    // the down projection, K = 9728, first).  Each problem's results do not
    // depend on the order.
    int ord[kGemvBatchMax];
    for (int i = 0; i < count; ++i) ord[i] = i;
    for (int i = 1; i < count; ++i)
        for (int j = i; j > 0 && K[ord[j]] > K[ord[j - 1]]; --j) {
            const int o = ord[j];
            ord[j] = ord[j - 1];
            ord[j - 1] = o;
        }
    for (int slot = 0; slot < count; ++slot) {
        const int i = ord[slot];
        const int nb = K[i] / kQK;
        b.p[slot] = {W[i], reinterpret_cast<const uint4*>(X[i]), Y[i], N[i], nb, R[i]};
        b.first[slot] = total;
        total += static_cast<int>((static_cast<long>(N[i]) + R[i] - 1) / R[i]);
        lds = gemv_lds_bytes(nb, R[i]) > lds ? gemv_lds_bytes(nb, R[i]) : lds;
    }
    b.first[count] = total;
    hipLaunchKernelGGL(q4k_gemv_batched_kernel, dim3(total), dim3(kGemvThreads), lds, stream, b);
    return hipGetLastError();
}

size_t gemv_lds_bytes(int nb, int R) {
    return static_cast<size_t>(nb) * 4 * kXGroupStride * 16 + static_cast<size_t>(nb) * 4 * 8 +
           static_cast<size_t>(R) * nb * 4;
}

hipError_t launch_gemv_rmsnorm(const uint8_t* W, const uint16_t* X, const uint16_t* gamma,
                               float eps, float* Y, int N, int K, int R, hipStream_t stream) {
    const int nb = K / kQK;
    const unsigned grid = static_cast<unsigned>((static_cast<long>(N) + R - 1) / R);
    hipLaunchKernelGGL(q4k_gemv_rmsnorm_kernel, dim3(grid), dim3(kGemvThreads),
                       gemv_lds_bytes(nb, R), stream, W, reinterpret_cast<const uint4*>(X),
                       reinterpret_cast<const uint4*>(gamma), eps, Y, N, nb, R);
    return hipGetLastError();
}

// R rows of each matrix per workgroup; the partials of both sit in LDS
// (gemv_lds_bytes(nb, 2 R)).
hipError_t launch_gemv_swiglu(const uint8_t* Wg, const uint8_t* Wu, const uint16_t* X, float* H,
                              int N, int K, int R, hipStream_t stream) {
    const int nb = K / kQK;
    const unsigned grid = static_cast<unsigned>((static_cast<long>(N) + R - 1) / R);
    hipLaunchKernelGGL(q4k_gemv_swiglu_kernel, dim3(grid), dim3(kGemvThreads),
                       gemv_lds_bytes(nb, 2 * R), stream, Wg, Wu,
                       reinterpret_cast<const uint4*>(X), H, N, nb, R);
    return hipGetLastError();
}

hipError_t launch_gemv(const uint8_t* W, const uint16_t* X, float* Y, int N, int K, int R,
                       hipStream_t stream) {
    const int nb = K / kQK;
    const unsigned grid = static_cast<unsigned>((static_cast<long>(N) + R - 1) / R);
    hipLaunchKernelGGL(q4k_gemv_kernel, dim3(grid), dim3(kGemvThreads), gemv_lds_bytes(nb, R),
                       stream, W, reinterpret_cast<const uint4*>(X), Y, N, nb, R);
    return hipGetLastError();
}

}  // namespace jq4k
