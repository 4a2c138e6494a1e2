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
// rounds.  Lane l of wave w takes quarter c = l / 16 of block 16 w + l % 16
// (plus 64 per round), so every round reads 64 consecutive blocks and a
// lane's quarter never changes.
//
// Arithmetic.  Each weight is formed in fp32, d*sc*q - dmin*m rounded once
// (v_fma_mix_f32 on the quants read as binary16 subnormals), then rounded to
// binary16, and x is staged as binary16 with a power-of-two scale per
// block of 256 values (2^-s_kb, chosen from the block's largest exponent so
// that no value overflows).  The products then go through the matrix cores:
// v_mfma_f32_16x16x32_f16 with A = the x of 16 blocks (row m = block m of
// the wave) and B = their weights (column n = block n), so that the diagonal
// D[j][j] sums block j's 256 products over the eight instructions of a
// round; the other 240 entries are not used.  The lanes of quarter
// c = j / 4 hold D[j][j] (accumulator j % 4) and store it, times 2^s_kb, as
// the block's partial.  No offset or factored form is involved, so the
// rounding error is relative to sum |w * x|: at most 2^-11 per weight from
// the binary16 rounding, plus fp32 accumulation over 256 products and nb
// partials (the bound is stated with the header's numerics).
//
// Reduction.  One partial per block in LDS; after all rounds each row sums
// its nb block values in order (deterministic, no atomics).
//
// LDS layout of x.  Chunk (kb, c, t) -- 16 bytes, the binary16 values
// x[256 kb + 64 c + 4 t + 0..3] then x[256 kb + 64 c + 32 + 4 t + 0..3], the
// A operand of instruction t for quarter c -- sits at 9 (c nb + kb) + t.  The
// stride of 9 chunks per (quarter, block) keeps the reads free of bank
// conflicts and costs no address arithmetic per chunk.
#include "q4k_device.h"

namespace jq4k {

constexpr int kGemvThreads = 256;
constexpr int kGemvBatchMax = 16;  // problems per batched launch

typedef __attribute__((ext_vector_type(8))) _Float16 half8_t;
typedef __attribute__((ext_vector_type(4))) float float4_t;
typedef __attribute__((ext_vector_type(2))) unsigned short u16x2_t;

size_t gemv_lds_bytes(int nb, int R);

// x in LDS (see the layout above): the 16 lanes of one quarter c read chunk
// t of 16 consecutive blocks (consecutive groups, wrapping at the end of a
// row), and 9 m mod 16 gives 16 consecutive groups 16 different 16-byte
// slots of the 64 banks, the conflict-free case of ds_read_b128.
constexpr int kXGroupStride = 9;
__device__ __forceinline__ int x_group_base(int kb, int c, int nb) {
    return (c * nb + kb) * kXGroupStride;
}

__device__ __forceinline__ float bf16_lo(uint32_t v) { return __builtin_bit_cast(float, v << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t v) { return __builtin_bit_cast(float, v & 0xFFFF0000u); }

// Largest biased exponent field (bits 7..14) among the 8 bf16 values of a
// chunk; packed 16-bit maxima.
__device__ __forceinline__ int max_exponent8(uint4 v) {
    constexpr uint32_t kExp = 0x7F807F80u;
    const u16x2_t a = __builtin_elementwise_max(__builtin_bit_cast(u16x2_t, v.x & kExp),
                                                __builtin_bit_cast(u16x2_t, v.y & kExp));
    const u16x2_t b = __builtin_elementwise_max(__builtin_bit_cast(u16x2_t, v.z & kExp),
                                                __builtin_bit_cast(u16x2_t, v.w & kExp));
    const u16x2_t m = __builtin_elementwise_max(a, b);
    return static_cast<int>(max(static_cast<uint32_t>(m[0]), static_cast<uint32_t>(m[1])) >> 7);
}

// Maximum over the 32 lanes of each half wave: row-local DPP steps (lanes
// 0..15 of a row), then one swizzle across the half wave's two rows.
__device__ __forceinline__ int half_wave_max(int v) {
    v = max(v, __builtin_amdgcn_update_dpp(0, v, 0xB1, 0xF, 0xF, false));   // quad_perm [1,0,3,2]
    v = max(v, __builtin_amdgcn_update_dpp(0, v, 0x4E, 0xF, 0xF, false));   // quad_perm [2,3,0,1]
    v = max(v, __builtin_amdgcn_update_dpp(0, v, 0x124, 0xF, 0xF, false));  // row_ror:4
    v = max(v, __builtin_amdgcn_update_dpp(0, v, 0x128, 0xF, 0xF, false));  // row_ror:8
    // ds_swizzle, bit-mask mode: lane ^ 16 within each group of 32
    return max(v, __builtin_amdgcn_ds_swizzle(v, (0x10 << 10) | 0x1F));
}

// The scale exponent of a block of x whose largest exponent field is e:
// x * 2^-s stays below 2^15 in magnitude (binary16 overflows at 65520), and
// 2^-s is a normal fp32 (s in [-126, 114]; e = 255 is Inf or NaN, which
// propagate).  Values below 2^(s-14) become binary16 subnormals: they lose
// at most 2^(s-25) = 2^(e-166), i.e. less than 2^-39 of the block's largest
// magnitude.
__device__ __forceinline__ int block_shift(int e) { return min(max(e - 141, -126), 114); }

// Two bf16 values (one word) times 2^-s (exact in fp32: a power of two),
// each rounded once to binary16.
__device__ __forceinline__ uint32_t bf16x2_to_f16x2(uint32_t w, float scale) {
    return pack_f16x2(bf16_lo(w) * scale, bf16_hi(w) * scale);
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

// D[j][j] of the round's 16 x 16 product for this lane's block j = lane % 16
// (meaningful in the lanes of quarter j / 4): 64 weights of quarter c times
// the matching staged x, summed over the four quarters by the instruction.
__device__ __forceinline__ float4_t quarter_mfma(const QuarterLoad& ld, int c, const uint4* xg) {
    const QuarterScales s = quarter_scales(ld.hdr, static_cast<uint32_t>(c));
    const uint32_t qw[8] = {ld.qa.x, ld.qa.y, ld.qa.z, ld.qa.w,
                            ld.qb.x, ld.qb.y, ld.qb.z, ld.qb.w};
    float4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        uint32_t h[4];
        dequant_dword_f16(qw[i], s, h);
        const uint4 xa = xg[i];
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(
            __builtin_bit_cast(half8_t, xa),
            __builtin_bit_cast(half8_t, make_uint4(h[0], h[1], h[2], h[3])), acc, 0, 0, 0);
    }
    return acc;
}

// LDS: x chunks (nb*36 x 16 B), the scale exponent s_kb of every block (nb
// ints, padded to 16 B), per-block partials (R*nb floats per matrix).
constexpr int kGemvDepth = 3;  // quarter tasks in flight per thread (3 measured best)
constexpr int kGemvMaxK = 16384;
constexpr int kGemvMaxXChunksPerThread = kGemvMaxK / 8 / kGemvThreads;

__host__ __device__ constexpr int gemv_shift_words(int nb) { return (nb + 3) & ~3; }

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
    int* xsh = reinterpret_cast<int*>(xs + nb * 4 * kXGroupStride);
    float* part = reinterpret_cast<float*>(xsh + gemv_shift_words(nb));

    const int t = threadIdx.x;
    const int lane = t & 63;
    const int c = lane >> 4, j = lane & 15;
    const bool diag = c == (j >> 2);        // this lane stores block j's partial
    const bool sel1 = (j & 1) != 0, sel2 = (j & 2) != 0;   // ... from accumulator j % 4
    const long row0 = tile * R;
    const int rows = static_cast<int>(min(static_cast<long>(R), N - row0));
    const int nblk = rows * nb;                       // blocks per matrix
    const int nblk_all = (kPair ? 2 : 1) * nblk;
    const uint8_t* Wt = W + row0 * nb * kBlockBytes;
    const uint8_t* Wt2 = kPair ? W2 + row0 * nb * kBlockBytes : nullptr;
    // block b of the task list: W's span, then (kPair) W2's
    auto blk_ptr = [&](int b) {
        if (kPair && b >= nblk) return Wt2 + static_cast<long>(b - nblk) * kBlockBytes;
        return Wt + static_cast<long>(b) * kBlockBytes;
    };
    const int b0 = 16 * (t >> 6) + j;  // this lane's first block; +64 per round

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
    const int nround = (nblk_all + 63) / 64;   // same for every thread
    auto round_block = [&](int round) { return min(b0 + 64 * round, nblk_all - 1); };
#pragma unroll
    for (int q = 0; q < kGemvMaxXChunksPerThread; ++q) {
        // q beyond the chunks of the largest K: no load at all (compile-time)
        if (q * kGemvThreads < nxc) {
            const int g = min(t + q * kGemvThreads, nxc - 1);
            xv[q] = X[g];
            if constexpr (kNorm) gv[q] = gamma[g];
        }
    }
    QuarterLoad ld[kGemvDepth];
#pragma unroll
    for (int u = 0; u < kGemvDepth; ++u) ld[u] = load_quarter(blk_ptr(round_block(u)), c);

    if constexpr (kNorm) {
        float ss = 0.f;
#pragma unroll
        for (int q = 0; q < kGemvMaxXChunksPerThread; ++q)
            if (t + q * kGemvThreads < nxc) {
                const uint4 v = xv[q];
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
        for (int q = 0; q < kGemvMaxXChunksPerThread; ++q)
            if (t + q * kGemvThreads < nxc) {
                const uint32_t w[4] = {xv[q].x, xv[q].y, xv[q].z, xv[q].w};
                const uint32_t gm[4] = {gv[q].x, gv[q].y, gv[q].z, gv[q].w};
                uint32_t o[4];
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    o[e] = pack_bf16x2(bf16_lo(w[e]) * r * bf16_lo(gm[e]),
                                       bf16_hi(w[e]) * r * bf16_hi(gm[e]));
                xv[q] = make_uint4(o[0], o[1], o[2], o[3]);
            }
    }

    // Stage x as binary16.  Chunk g (x[8g .. 8g+7]) belongs to block
    // kb = g / 32, quarter c = (g / 8) % 4, and is piece gq = g % 8 of the
    // quarter: pieces 0..3 are even-sub-block values (bytes 0..7 of chunks
    // t = 2 gq, 2 gq + 1), pieces 4..7 odd ones (bytes 8..15 of chunks
    // t = 2 (gq - 4), + 1).  The 32 chunks of a block sit in 32 consecutive
    // lanes (half a wave), which reduce the block's largest exponent among
    // themselves; a half wave past the end of x holds repeats and stores
    // nothing.
#pragma unroll
    for (int q = 0; q < kGemvMaxXChunksPerThread; ++q) {
        if (q * kGemvThreads < nxc) {
            const int g = t + q * kGemvThreads;
            const uint4 v = xv[q];
            const int e = half_wave_max(max_exponent8(v));
            const int sh = block_shift(e);
            const float scale = __builtin_bit_cast(float, static_cast<uint32_t>(127 - sh) << 23);
            const uint32_t h0 = bf16x2_to_f16x2(v.x, scale), h1 = bf16x2_to_f16x2(v.y, scale);
            const uint32_t h2 = bf16x2_to_f16x2(v.z, scale), h3 = bf16x2_to_f16x2(v.w, scale);
            if (g < nxc) {
                const int kb = g >> 5, gq = g & 7;
                const int t0 = 2 * (gq & 3);
                uint2* dst = reinterpret_cast<uint2*>(xs + x_group_base(kb, (g >> 3) & 3, nb) + t0) +
                             (gq >> 2);
                dst[0] = make_uint2(h0, h1);
                dst[2] = make_uint2(h2, h3);
                if ((g & 31) == 0) xsh[kb] = sh;
            }
        }
    }
    __syncthreads();

    // A round past the thread's last task (the last round of a span whose
    // block count is not a multiple of 64) computes on a repeated block and
    // stores nothing; the four lanes of a block agree, so the instruction's
    // sum over quarters sees only its own block.  The loop runs whole groups
    // of kGemvDepth rounds without a branch; the remaining rounds follow it,
    // without prefetch.
    const int kb_step = 64 % nb;
    int kb = b0 % nb;
    auto task = [&](int round, QuarterLoad& l, bool prefetch) {
        const int b = b0 + 64 * round;
        const float4_t acc = quarter_mfma(l, c, xs + x_group_base(kb, c, nb));
        const float p01 = sel1 ? acc[1] : acc[0];
        const float p23 = sel1 ? acc[3] : acc[2];
        const float p = __builtin_amdgcn_ldexpf(sel2 ? p23 : p01, xsh[kb]);
        if (diag && b < nblk_all) part[b] = p;
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
        for (int i = 0; i < nb; ++i) s += part[r * nb + i];
        if constexpr (kPair) {
            float u = 0.f;
            for (int i = 0; i < nb; ++i) u += part[nblk + r * nb + i];
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
    return static_cast<size_t>(nb) * 4 * kXGroupStride * 16 +
           static_cast<size_t>(gemv_shift_words(nb)) * 4 + static_cast<size_t>(R) * nb * 4;
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
