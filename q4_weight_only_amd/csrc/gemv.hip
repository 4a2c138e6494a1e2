// gemv.hip -- the M = 1 (decode) Q4_K GEMV for gfx950.
//
// y[n] = sum_k w[n][k] x[k], w = d*sc_s*q - dmin*m_s (genie-ai-runtime
// README, "At a glance": INT4 dequant-fused GEMV).  HBM-bound: every byte of
// W is read once (0.5625 B per weight); no weight is ever formed.
//
// Arithmetic: the factored form, certified per row.  Sub-block s of a block
// adds ds_s * S1_s - dm_s * S0_s to its row, with ds = d*sc and dm = dmin*m
// (exact in fp32: at most 11 + 6 significant bits), S1 = sum q x over the
// sub-block's 32 weights and S0 = sum x.  The 4-bit codes go into
// v_dot2_f32_f16 as they sit in the block: a nibble masked in place in a
// 16-bit half reads as the binary16 subnormal q * 2^-24 (low nibble) or
// q * 2^-20 (high nibble), exactly.  x is staged as binary16 times 2^-sh per
// block of 256 values (sh from the block's largest exponent), so every
// product q * x is exact and each dot2 step sums two of them into fp32.
//
// The factored form loses accuracy where ds*S1 and dm*S0 cancel (weights
// near zero against large scales), so every row also carries a bound on its
// own rounding error and a lower bound on sum |w x|, and a row whose bound
// does not certify the accuracy contract is recomputed exactly (below).
// Rows of randomly drawn blocks certify with a margin of about 8.
//
// Work decomposition.  A workgroup owns R consecutive rows, R*nb
// consecutive blocks of W: one contiguous span of memory (for a gate/up
// pair, the span of the second matrix follows the first's in the task
// list).  The span is cut into tasks of one half block (the header and the
// 64 code bytes of sub-blocks 4h .. 4h+3: 128 weights); the 256 threads
// sweep the tasks in rounds, lanes 2j and 2j+1 of a round taking the two
// halves of one block, so every round reads 128 consecutive blocks.  A
// thread's half h = t & 1 never changes; the next round's loads are in
// flight while a round is computed (two sets of 20 registers take the
// rounds in turn: 79 VGPRs, six waves per SIMD; two rounds in flight, or
// three for small launches, measured slower).
//
// Per half block, each sub-block gives r = ds S1 - dm S0 (one fma after the
// exact dm S0 rounding), and the half adds its four r (the output), their
// magnitudes (L: at most sum |w x|) and the error scale B = sum over its
// sub-blocks of (15 |ds| + |dm|) T0, T0 = sum |x|, which bounds
// sum (|ds| q + |dm|) |x| and with it every rounding error.  S0 and T0 are
// staged with x.  The two halves' sums are added with one DPP step (the same
// bits in both lanes), scaled by 2^sh_kb and left in LDS per block; each row
// then adds its nb blocks in order.  A row's sums therefore do not depend on
// R or on the launch: the same bits for every grouping of the rows (no
// atomics on values).
//
// Certificate.  With u = 2^-24, every rounding error of the row is at most
// E = (192 + nb) u B: the dot2 chains (16 steps of two exact products per
// sub-block, at most two roundings a step: 32u; the budget allows 128u),
// the staged S0 and T0 (9 additions), the combine (3 roundings) and the
// row's sums (fewer than 8 + nb additions deep).  The row is accepted when
//     E <= 1.9e-3 * max(L - 2E, |y| - E) + 0.99e-5,
// the slack to 2e-3 and 1e-5 covering w against the fp32 weight (u |w|) and
// the rounding of E itself.  Otherwise -- and for every row when some x is
// not exact in its staged binary16 (values below 2^-31 of their block's
// largest magnitude, Inf, NaN) -- one wave recomputes the row: each fp32
// weight (d*sc*q - dmin*m rounded once) times x, summed in fp64, rounded
// once to fp32.
//
// LDS layout of the staged x.  Chunk g holds the binary16 x[8g .. 8g+7] in
// the order 0, 2, 1, 3, 4, 6, 5, 7 (the order of the codes as masked from
// two consecutive code dwords: bytes 0, 2, 1, 3 of each).  The 16 chunks a
// half-block task reads (g = 32 kb + 16 h + i: sub-block 4h + i / 4) sit at
// 19 (2 kb + h) + i, followed by two chunks of that half's S0 and T0.  The
// lanes of a round read one chunk index i of consecutive groups, and the odd
// stride of 19 spreads them over the banks without conflicts; a thread's
// reads are one base address plus immediate offsets.
#include "q4k_device.h"

namespace jq4k {

constexpr int kGemvThreads = 256;
constexpr int kGemvBatchMax = 16;  // problems per batched launch
constexpr int kGemvMaxK = 16384;
constexpr int kGemvMaxXChunksPerThread = kGemvMaxK / 8 / kGemvThreads;
constexpr int kXGroupStride = 19;  // LDS chunks per (block, half): 16 of x, S0, T0, one spare
constexpr int kRoundBlocks = kGemvThreads / 2;   // blocks per round

typedef __attribute__((ext_vector_type(4))) float float4_t;
typedef __attribute__((ext_vector_type(2))) unsigned short u16x2_t;
typedef __attribute__((ext_vector_type(2))) _Float16 half2_t;

__host__ __device__ constexpr int gemv_shift_words(int nb) { return (nb + 3) & ~3; }
__device__ __forceinline__ int x_group_base(int kb, int h) { return (2 * kb + h) * kXGroupStride; }
__device__ __forceinline__ int x_chunk_phys(int g) { return (g >> 4) * kXGroupStride + (g & 15); }

// LDS of a workgroup with R rows of each of `mats` matrices (bytes):
//   staged x              nb * 2 groups of 19 chunks of 16 B: 16 chunks of x,
//                         then S0 and T0 of the half's four sub-blocks
//   sh                    per block, one int (padded to 16 B)
//   block partials        mats * R * nb + 1 float4 {y, L, B, -} (the last slot
//                         takes the stores of lanes past the last block)
//   row results           mats * R floats
//   recompute list        1 + mats * R ints (count, then rows)
__host__ __device__ constexpr size_t gemv_lds_layout(int nb, int R, int mats) {
    return static_cast<size_t>(nb) * 2 * kXGroupStride * 16 +
           static_cast<size_t>(gemv_shift_words(nb)) * 4 +
           (static_cast<size_t>(mats) * R * nb + 1) * 16 + static_cast<size_t>(mats) * R * 4 +
           (1 + static_cast<size_t>(mats) * R) * 4;
}

size_t gemv_lds_bytes(int nb, int R, int mats) { return gemv_lds_layout(nb, R, mats); }

__device__ __forceinline__ float bf16_lo(uint32_t v) { return __builtin_bit_cast(float, v << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t v) { return __builtin_bit_cast(float, v & 0xFFFF0000u); }

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

// Sum over the four lanes of a quad, the same bits in all four: each lane
// adds its partner's value, then the other pair's sum (fp32 addition
// commutes, so the four results agree).
__device__ __forceinline__ float quad_sum(float v) {
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                                       0, __builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, false));
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                                       0, __builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, false));
    return v;
}

// Sum over the two lanes of a pair, the same bits in both (fp32 addition
// commutes).
__device__ __forceinline__ float pair_sum(float v) {
    const int i = __builtin_bit_cast(int, v);
    return v + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(i, i, 0xB1, 0xF, 0xF, true));
}

// The scale exponent of a block of x whose largest exponent field is e:
// x * 2^-sh stays below 2^15 in magnitude (binary16 overflows at 65520),
// and 2^-sh is a normal fp32 (sh in [-126, 114]; e = 255 is Inf or NaN).
__device__ __forceinline__ int block_shift(int e) { return min(max(e - 141, -126), 114); }
__device__ __forceinline__ float pow2f(int e) {
    return __builtin_bit_cast(float, static_cast<uint32_t>(127 + e) << 23);
}

// Two binary16 codes (as masked in place) times two staged binary16 x, added
// to an fp32 sum.
__device__ __forceinline__ float dot2_codes(uint32_t codes, uint32_t x, float acc) {
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, codes),
                                  __builtin_bit_cast(half2_t, x), acc, false);
}

struct HalfLoad {
    uint4 hdr;     // d, dmin, scales
    uint4 q[4];    // code bytes 64 h .. 64 h + 63: quarters 2h and 2h+1
};

__device__ __forceinline__ HalfLoad load_half(const uint8_t* blk, int h) {
    HalfLoad r;
    r.hdr = load16(blk);
#pragma unroll
    for (int k = 0; k < 4; ++k) r.q[k] = load16(blk + 16 + 64 * h + 16 * k);
    return r;
}

// S1 of one sub-block (32 weights) from its 8 code dwords' nibbles (low
// nibbles: mask 0x000F000F, codes q 2^-24; high: 0x00F000F0, q 2^-20) and
// its 4 chunks of staged x.
template <uint32_t kMask>
__device__ __forceinline__ float sub_block_sum(const uint4& qa, const uint4& qb, const uint4* xc) {
    const uint32_t qw[8] = {qa.x, qa.y, qa.z, qa.w, qb.x, qb.y, qb.z, qb.w};
    float acc = 0.f;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const uint4 x = xc[p];
        const uint32_t v = qw[2 * p], u = qw[2 * p + 1];
        acc = dot2_codes(v & kMask, x.x, acc);
        acc = dot2_codes((v >> 8) & kMask, x.y, acc);
        acc = dot2_codes(u & kMask, x.z, acc);
        acc = dot2_codes((u >> 8) & kMask, x.w, acc);
    }
    return acc;
}

// One row recomputed by one wave, lane l taking sub-block l / 8, weights
// 4 (l % 8) .. + 3 of every block: each fp32 weight (one rounding of
// d*sc*q - dmin*m) times x, summed in fp64 (the products of a 24-bit weight
// and an 8-bit activation are exact there), the lanes' sums combined in a
// fixed butterfly and rounded once to fp32.  kNorm: x is the normalised
// activation, recomputed exactly as it was staged.
template <bool kNorm>
__device__ float exact_row(const uint8_t* rowp, int nb, const uint4* __restrict__ X,
                           const uint4* __restrict__ gamma, float rnorm, int lane) {
    const int s = lane >> 3, i0 = 4 * (lane & 7);
    const uint16_t* Xh = reinterpret_cast<const uint16_t*>(X);
    const uint16_t* Gh = reinterpret_cast<const uint16_t*>(gamma);
    double acc = 0.0;
    for (int kb = 0; kb < nb; ++kb) {
        const uint8_t* blk = rowp + static_cast<long>(kb) * kBlockBytes;
        const uint4 hdr = load16(blk);
        const uint32_t qd = *reinterpret_cast<const uint32_t*>(blk + 16 + 32 * (s >> 1) + i0);
        const uint2 xw = *reinterpret_cast<const uint2*>(Xh + kQK * kb + 32 * s + i0);
        float xs[4] = {bf16_lo(xw.x), bf16_hi(xw.x), bf16_lo(xw.y), bf16_hi(xw.y)};
        if constexpr (kNorm) {
            const uint2 gw = *reinterpret_cast<const uint2*>(Gh + kQK * kb + 32 * s + i0);
            const uint32_t o0 = pack_bf16x2(xs[0] * rnorm * bf16_lo(gw.x),
                                            xs[1] * rnorm * bf16_hi(gw.x));
            const uint32_t o1 = pack_bf16x2(xs[2] * rnorm * bf16_lo(gw.y),
                                            xs[3] * rnorm * bf16_hi(gw.y));
            xs[0] = bf16_lo(o0);
            xs[1] = bf16_hi(o0);
            xs[2] = bf16_lo(o1);
            xs[3] = bf16_hi(o1);
        }
        const float d = half_bits_to_float(hdr.x & 0xFFFFu);
        const float dmin = half_bits_to_float(hdr.x >> 16);
        uint32_t scp, mp;
        scale_min_pair(static_cast<uint32_t>(s >> 1), hdr.y, hdr.z, hdr.w, &scp, &mp);
        const uint32_t odd = static_cast<uint32_t>(s & 1);
        const float ds = d * static_cast<float>((scp >> (8 * odd)) & 0xFFu);
        const float dm = dmin * static_cast<float>((mp >> (8 * odd)) & 0xFFu);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const uint32_t q = (qd >> (8 * e + 4 * odd)) & 0xFu;
            const float w = __builtin_fmaf(ds, static_cast<float>(q), -dm);
            acc = __builtin_fma(static_cast<double>(w), static_cast<double>(xs[e]), acc);
        }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) acc += __shfl_xor(acc, o);
    return static_cast<float>(acc);
}

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
    constexpr int kMats = kPair ? 2 : 1;
    const int t = threadIdx.x;
    const int lane = t & 63;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
    const int h = t & 1;
    const long row0 = tile * R;
    const int rows = static_cast<int>(min(static_cast<long>(R), N - row0));
    const int nblk = rows * nb;                 // blocks per matrix here
    const int nblk_all = kMats * nblk;

    uint4* xs = smem;
    int* xsh = reinterpret_cast<int*>(xs + nb * 2 * kXGroupStride);
    float4_t* part = reinterpret_cast<float4_t*>(xsh + gemv_shift_words(nb));
    const int spare = kMats * R * nb;           // the partials' spare slot
    float* yrow = reinterpret_cast<float*>(part + spare + 1);
    int* flist = reinterpret_cast<int*>(yrow + kMats * R);

    const uint8_t* Wt = W + row0 * nb * kBlockBytes;
    const uint8_t* Wt2 = kPair ? W2 + row0 * nb * kBlockBytes : nullptr;
    // block b of the task list: W's span, then (kPair) W2's (a single
    // matrix: a 32-bit offset from the workgroup's base)
    auto blk_ptr = [&](int b) {
        if constexpr (kPair) {
            if (b >= nblk) return Wt2 + static_cast<long>(b - nblk) * kBlockBytes;
            return Wt + static_cast<long>(b) * kBlockBytes;
        } else {
            return Wt + static_cast<uint32_t>(b) * static_cast<uint32_t>(kBlockBytes);
        }
    };
    const int b0 = t >> 1;  // this thread's first block; + kRoundBlocks per round

    // Memory requests in the order they are needed (vmcnt retires in order):
    // x first, then the first round of weights, so that staging x waits only
    // for x and each round waits only for its own weights.
    // Every load is unconditional, past the end a repeat of the last chunk
    // or block: with loads under branches the compiler's count of loads in
    // flight turns pessimistic at the joins and it waits for all of them,
    // which undoes the prefetch.
    const int nxc = nb * 32;  // 16-byte chunks of x, at most 2048 (K <= 16384)
    const int nround = (nblk_all + kRoundBlocks - 1) / kRoundBlocks;   // the same for every thread
    auto round_block = [&](int round) { return min(b0 + kRoundBlocks * round, nblk_all - 1); };
    uint4 xv[kGemvMaxXChunksPerThread];
    uint4 gv[kNorm ? kGemvMaxXChunksPerThread : 1];
#pragma unroll
    for (int q = 0; q < kGemvMaxXChunksPerThread; ++q) {
        // q beyond the chunks of the largest K: no load at all (compile-time)
        if (q * kGemvThreads < nxc) {
            const int g = min(t + q * kGemvThreads, nxc - 1);
            xv[q] = X[g];
            if constexpr (kNorm) gv[q] = gamma[g];
        }
    }
    HalfLoad la = load_half(blk_ptr(round_block(0)), h);

    if (t == 0) flist[0] = 0;

    float rnorm = 0.f;
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
        if (lane == 0) wave_ss[wave] = ss;
        __syncthreads();
        const float total = (wave_ss[0] + wave_ss[1]) + (wave_ss[2] + wave_ss[3]);
        rnorm = rsqrtf(total / static_cast<float>(nb * kQK) + eps);
#pragma unroll
        for (int q = 0; q < kGemvMaxXChunksPerThread; ++q)
            if (t + q * kGemvThreads < nxc) {
                const uint32_t w[4] = {xv[q].x, xv[q].y, xv[q].z, xv[q].w};
                const uint32_t gm[4] = {gv[q].x, gv[q].y, gv[q].z, gv[q].w};
                uint32_t o[4];
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    o[e] = pack_bf16x2(bf16_lo(w[e]) * rnorm * bf16_lo(gm[e]),
                                       bf16_hi(w[e]) * rnorm * bf16_hi(gm[e]));
                xv[q] = make_uint4(o[0], o[1], o[2], o[3]);
            }
    }

    // Stage x.  Chunk g (x[8g .. 8g+7]) is piece p = g % 4 of sub-block
    // s = (g / 4) % 8 of block kb = g / 32.  The 32 chunks of a block sit in
    // 32 consecutive lanes (half a wave), which reduce the block's largest
    // magnitude among themselves, and the 4 chunks of a sub-block in a quad,
    // which sums its S0 and T0; a half wave past the end of x holds repeats
    // and stores nothing.  A bf16 value is exact in the staged binary16 when
    // its exponent field is at least the block's largest minus 31 (its last
    // significant bit then lands at or above 2^-24 after the scaling), or
    // when it is zero; smaller non-zero values (and Inf, NaN) set `inexact`.
    int inexact = 0;
#pragma unroll
    for (int q = 0; q < kGemvMaxXChunksPerThread; ++q) {
        if (q * kGemvThreads < nxc) {
            const int g = t + q * kGemvThreads;
            const uint4 v = xv[q];
            const uint4 mag = make_uint4(v.x & 0x7FFF7FFFu, v.y & 0x7FFF7FFFu, v.z & 0x7FFF7FFFu,
                                         v.w & 0x7FFF7FFFu);
            const u16x2_t mx = __builtin_elementwise_max(
                __builtin_elementwise_max(__builtin_bit_cast(u16x2_t, mag.x),
                                          __builtin_bit_cast(u16x2_t, mag.y)),
                __builtin_elementwise_max(__builtin_bit_cast(u16x2_t, mag.z),
                                          __builtin_bit_cast(u16x2_t, mag.w)));
            // magnitude bits minus one: zero wraps to the largest value
            const u16x2_t one = {1, 1};
            const u16x2_t mn = __builtin_elementwise_min(
                __builtin_elementwise_min(__builtin_bit_cast(u16x2_t, mag.x) - one,
                                          __builtin_bit_cast(u16x2_t, mag.y) - one),
                __builtin_elementwise_min(__builtin_bit_cast(u16x2_t, mag.z) - one,
                                          __builtin_bit_cast(u16x2_t, mag.w) - one));
            const int e = half_wave_max(
                static_cast<int>(max(static_cast<uint32_t>(mx[0]), static_cast<uint32_t>(mx[1])) >> 7));
            const int low = static_cast<int>(min(static_cast<uint32_t>(mn[0]), static_cast<uint32_t>(mn[1])));
            const int bad = (e == 255) | (low < ((e - 31) << 7) - 1);
            const int sh = block_shift(e);
            const float scale = pow2f(-sh);
            const float x[8] = {bf16_lo(v.x), bf16_hi(v.x), bf16_lo(v.y), bf16_hi(v.y),
                                bf16_lo(v.z), bf16_hi(v.z), bf16_lo(v.w), bf16_hi(v.w)};
            float f[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) f[i] = x[i] * scale;
            const uint32_t h0 = pack_f16x2(f[0], f[2]), h1 = pack_f16x2(f[1], f[3]);
            const uint32_t h2 = pack_f16x2(f[4], f[6]), h3 = pack_f16x2(f[5], f[7]);
            const half2_t ones = {static_cast<_Float16>(1.0f), static_cast<_Float16>(1.0f)};
            float s0 = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, h0), ones, 0.f, false);
            s0 = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, h1), ones, s0, false);
            s0 = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, h2), ones, s0, false);
            s0 = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, h3), ones, s0, false);
            float t0 = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, h0 & 0x7FFF7FFFu), ones,
                                              0.f, false);
            t0 = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, h1 & 0x7FFF7FFFu), ones, t0,
                                        false);
            t0 = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, h2 & 0x7FFF7FFFu), ones, t0,
                                        false);
            t0 = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, h3 & 0x7FFF7FFFu), ones, t0,
                                        false);
            s0 = quad_sum(s0);
            t0 = quad_sum(t0);
            if (g < nxc) {
                inexact |= bad;
                xs[x_chunk_phys(g)] = make_uint4(h0, h1, h2, h3);
                if ((g & 3) == 0) {
                    // sub-block s: slot s % 4 of the S0 and T0 chunks of
                    // group (block, half s / 4)
                    float* z = reinterpret_cast<float*>(xs + x_chunk_phys(g | 15) + 1);
                    const int s = (g >> 2) & 7;
                    z[s & 3] = s0;
                    z[4 + (s & 3)] = t0;
                }
                if ((g & 31) == 0) xsh[g >> 5] = sh;
            }
        }
    }
    const bool x_inexact = __syncthreads_or(inexact) != 0;

    // The tasks.  A round past the thread's last task (the last round of a
    // span whose block count is not a multiple of kRoundBlocks) computes on
    // a repeated block and stores into the spare slot; the two lanes of a
    // block agree, so the pair sums see only their own block.
    const int kb_step = kRoundBlocks % nb;
    int kb = b0 % nb;
    int gq = x_group_base(kb, h);   // the LDS chunk of group (kb, h)
    // scale bytes of sub-blocks 4h + 0..3 (Q4_K packing): half 0 the low six
    // bits of scales[j] and scales[4+j]; half 1 the nibbles of scales[8+j]
    // plus bits 6..7 of scales[j] and scales[4+j] as bits 4..5
    const uint32_t low_mask = h ? 0x0F0F0F0Fu : 0x3F3F3F3Fu;
    const uint32_t top_mask = h ? 0x30303030u : 0u;
    auto task = [&](int round, const HalfLoad& l) {
        const int b = b0 + kRoundBlocks * round;
        const uint4* xg = xs + gq;
        // S1 of sub-blocks 4h + j, scaled by 2^-sh like x: even j from the
        // low nibbles of quarter 2h + j / 2, odd j from its high nibbles
        float s1[4];
        s1[0] = sub_block_sum<0x000F000Fu>(l.q[0], l.q[1], xg);
        s1[1] = sub_block_sum<0x00F000F0u>(l.q[0], l.q[1], xg + 4);
        s1[2] = sub_block_sum<0x000F000Fu>(l.q[2], l.q[3], xg + 8);
        s1[3] = sub_block_sum<0x00F000F0u>(l.q[2], l.q[3], xg + 12);
        const float4_t S0 = *reinterpret_cast<const float4_t*>(xg + 16);
        const float4_t T0 = *reinterpret_cast<const float4_t*>(xg + 17);
        const int sh = xsh[kb];
        const uint4 hd = l.hdr;
        const float d = half_bits_to_float(hd.x & 0xFFFFu);
        const float dmin = half_bits_to_float(hd.x >> 16);
        const uint32_t sc_src = h ? hd.w : hd.y;
        const uint32_t m_src = h ? hd.w >> 4 : hd.z;
        const uint32_t scb = (sc_src & low_mask) | ((hd.y >> 2) & top_mask);
        const uint32_t mb = (m_src & low_mask) | ((hd.z >> 2) & top_mask);
        const float sc[4] = {ubyte_to_float<0>(scb), ubyte_to_float<1>(scb),
                             ubyte_to_float<2>(scb), ubyte_to_float<3>(scb)};
        const float mm[4] = {ubyte_to_float<0>(mb), ubyte_to_float<1>(mb),
                             ubyte_to_float<2>(mb), ubyte_to_float<3>(mb)};
        const float dE = d * 0x1p24f, dO = d * 0x1p20f;
        float r[4];
#pragma unroll
        for (int j = 0; j < 4; ++j)
            r[j] = __builtin_fmaf(((j & 1) ? dO : dE) * sc[j], s1[j], -((dmin * mm[j]) * S0[j]));
        const float bq = (15.0f * fabsf(d)) * ((sc[0] * T0[0] + sc[1] * T0[1]) +
                                               (sc[2] * T0[2] + sc[3] * T0[3])) +
                         fabsf(dmin) * ((mm[0] * T0[0] + mm[1] * T0[1]) +
                                        (mm[2] * T0[2] + mm[3] * T0[3]));
        // the block's sums (the two halves added, the same bits in both
        // lanes), scaled by 2^sh; half 0 stores {y, L}, half 1 B
        const float y = pair_sum((r[0] + r[1]) + (r[2] + r[3]));
        const float L = pair_sum((fabsf(r[0]) + fabsf(r[1])) + (fabsf(r[2]) + fabsf(r[3])));
        const float B = pair_sum(bq);
        const int slot = b < nblk_all ? b : spare;
        float2* dst = reinterpret_cast<float2*>(part + slot) + h;
        *dst = h ? make_float2(__builtin_amdgcn_ldexpf(B, sh), 0.f)
                 : make_float2(__builtin_amdgcn_ldexpf(y, sh), __builtin_amdgcn_ldexpf(L, sh));
        kb += kb_step;
        gq += kb_step * 2 * kXGroupStride;
        if (kb >= nb) {
            kb -= nb;
            gq -= nb * 2 * kXGroupStride;
        }
    };
    // Two register sets take the rounds in turn: the next round's loads go
    // into one while the other is computed (one round in flight), and no
    // set is copied into the other.  A set is reloaded only after its round
    // is computed (the scheduling barrier keeps the load there; moved above
    // the round it would need a third set).  The last round's reload asks
    // for a repeated block.
    int r0 = 0;
    for (; r0 + 2 <= nround; r0 += 2) {
        const HalfLoad lb = load_half(blk_ptr(round_block(r0 + 1)), h);
        task(r0, la);
        __builtin_amdgcn_sched_barrier(0);
        la = load_half(blk_ptr(round_block(r0 + 2)), h);
        task(r0 + 1, lb);
    }
    if (r0 < nround) task(r0, la);
    __syncthreads();

    // Rows: the blocks' sums in order, the certificate, and the list of rows
    // to recompute (the list's order does not matter: a row's recomputation
    // is the same whichever wave runs it).  Row q of the task list (W's rows,
    // then W2's) owns blocks q nb .. q nb + nb - 1.
    const float kE = (192.0f + static_cast<float>(nb)) * 0x1p-24f;
    for (int q = t; q < kMats * rows; q += kGemvThreads) {
        const float4_t* pr = part + q * nb;
        float y = 0.f, L = 0.f, B = 0.f;
        for (int j = 0; j < nb; ++j) {
            const float4_t v = pr[j];
            y += v[0];
            L += v[1];
            B += v[2];
        }
        const float E = kE * B;
        const float lb = fmaxf(L - 2.0f * E, fabsf(y) - E);
        yrow[q] = y;
        if (x_inexact || !(E <= 1.9e-3f * lb + 0.99e-5f)) flist[1 + atomicAdd(flist, 1)] = q;
    }
    __syncthreads();
    const int nredo = flist[0];
    for (int e = wave; e < nredo; e += kGemvThreads / 64) {
        const int q = flist[1 + e];
        const int mat = (kPair && q >= rows) ? 1 : 0;
        const int qq = q - mat * rows;
        const uint8_t* rp = (mat ? W2 : W) + (row0 + qq) * nb * kBlockBytes;
        const float y = exact_row<kNorm>(rp, nb, X, gamma, rnorm, lane);
        if (lane == 0) yrow[q] = y;
    }
    __syncthreads();
    for (int q = t; q < rows; q += kGemvThreads) {
        if constexpr (kPair)
            Y[row0 + q] = silu(yrow[q]) * yrow[rows + q];
        else
            Y[row0 + q] = yrow[q];
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
    // first they do not form the tail.  Each problem's results do not
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
        const size_t need = gemv_lds_bytes(nb, R[i], 1);
        lds = need > lds ? need : lds;
    }
    b.first[count] = total;
    hipLaunchKernelGGL(q4k_gemv_batched_kernel, dim3(total), dim3(kGemvThreads), lds, stream, b);
    return hipGetLastError();
}

hipError_t launch_gemv_rmsnorm(const uint8_t* W, const uint16_t* X, const uint16_t* gamma,
                               float eps, float* Y, int N, int K, int R, hipStream_t stream) {
    const int nb = K / kQK;
    const unsigned grid = static_cast<unsigned>((static_cast<long>(N) + R - 1) / R);
    hipLaunchKernelGGL(q4k_gemv_rmsnorm_kernel, dim3(grid), dim3(kGemvThreads),
                       gemv_lds_bytes(nb, R, 1), stream, W, reinterpret_cast<const uint4*>(X),
                       reinterpret_cast<const uint4*>(gamma), eps, Y, N, nb, R);
    return hipGetLastError();
}

// R rows of each matrix per workgroup.
hipError_t launch_gemv_swiglu(const uint8_t* Wg, const uint8_t* Wu, const uint16_t* X, float* H,
                              int N, int K, int R, hipStream_t stream) {
    const int nb = K / kQK;
    const unsigned grid = static_cast<unsigned>((static_cast<long>(N) + R - 1) / R);
    hipLaunchKernelGGL(q4k_gemv_swiglu_kernel, dim3(grid), dim3(kGemvThreads),
                       gemv_lds_bytes(nb, R, 2), stream, Wg, Wu,
                       reinterpret_cast<const uint4*>(X), H, N, nb, R);
    return hipGetLastError();
}

hipError_t launch_gemv(const uint8_t* W, const uint16_t* X, float* Y, int N, int K, int R,
                       hipStream_t stream) {
    const int nb = K / kQK;
    const unsigned grid = static_cast<unsigned>((static_cast<long>(N) + R - 1) / R);
    hipLaunchKernelGGL(q4k_gemv_kernel, dim3(grid), dim3(kGemvThreads),
                       gemv_lds_bytes(nb, R, 1), stream, W, reinterpret_cast<const uint4*>(X), Y,
                       N, nb, R);
    return hipGetLastError();
}

}  // namespace jq4k
