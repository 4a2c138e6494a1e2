// gemv.hip -- the M = 1 (decode) Q4_K GEMV for gfx950.
//
// y[n] = sum_k w[n][k] x[k], w = d*sc_s*q - dmin*m_s (genie-ai-runtime
// README, "At a glance": INT4 dequant-fused GEMV).  HBM-bound: every byte of
// W is read once (0.5625 B per weight); no weight is ever formed.
//
// Arithmetic: the factored form on the matrix cores, certified per row.
// Sub-block s of a block adds ds_s * S1_s - dm_s * S0_s to its row, with
// ds = d*sc and dm = dmin*m (exact in fp32: at most 11 + 6 significant
// bits), S1 = sum q x over the sub-block's 32 weights and S0 = sum x.  The
// 4-bit codes go into v_mfma_f32_16x16x32_f16 as they sit in the block: a
// nibble masked in place in a 16-bit half reads as the binary16 subnormal
// q * 2^-24 (low nibble) or q * 2^-20 (high nibble), exactly.  x is staged
// as binary16 times 2^-sh per block of 256 values (sh from the block's
// largest exponent), so every product q * x is exact and the matrix cores
// sum them in fp32.
//
// The factored form loses accuracy where ds*S1 and dm*S0 cancel (weights
// near zero against large scales), so every row also carries a bound on its
// own rounding error and a lower bound on sum |w x|, and a row whose bound
// does not certify the accuracy contract is recomputed exactly (below).
// Rows of randomly drawn blocks certify with a margin of about 8.
//
// Matrix-core tile: 16 rows of W at one block column kb.  B column n is
// block (row n, kb); lane 16c + n holds 8 codes of its quarter c (the
// quarter's code bytes pair sub-blocks 2c and 2c+1).  Row m < 8 of A is
// sub-block m of x: lane 16c + m supplies its values where sub-block m is
// the one k-group c covers in the instruction (2c for the instructions on
// low nibbles, 2c+1 for high) and zeros otherwise; rows 8..15 are zero.
// Eight instructions per tile (4 code pairs x low/high nibbles) leave
// D[s][n] = S1_s of block n (scaled) in lane 16 (s / 4) + n, accumulator
// s % 4: lanes 0..31 ("S lanes") hold sub-blocks 0..3 / 4..7 of block n.
//
// Per tile, every S lane combines its four sub-blocks: a = dm S0,
// r = ds D - a, and sums r (the output) and |r| (L: sum over sub-blocks of
// |sum w x| <= sum |w x|).  Lanes 32..63 ("T lanes", D = 0) sum the error
// scale B = sum over sub-blocks of (15 |ds| + |dm|) T0 with T0 = sum |x|,
// which bounds sum (|ds| q + |dm|) |x| and with it every rounding error.
// S0 and T0 are staged with x.  Each tile's sums are scaled by 2^sh_kb.
//
// Certificate.  With u = 2^-24, every rounding error of the row is at most
// E = (192 + nb) u B: the matrix cores' fp32 sums (at most 2u per addition
// of 32 exact products: 64u, taken twice), the staged S0 and T0 (9
// additions), the combine (3 roundings) and the row's sums (fewer than
// 8 + nb additions deep).  The row is accepted when
//     E <= 1.9e-3 * max(L - 2E, |y| - E) + 0.99e-5,
// the slack to 2e-3 and 1e-5 covering w against the fp32 weight (u |w|) and
// the rounding of E itself.  Otherwise -- and for every row when some x is
// not exact in its staged binary16 (values below 2^-31 of their block's
// largest magnitude, Inf, NaN) -- one wave recomputes the row: each fp32
// weight (d*sc*q - dmin*m rounded once) times x, summed in fp64, rounded
// once to fp32.
//
// Work decomposition.  A workgroup owns R consecutive rows (ceil(R/16)
// groups of 16) of each of its matrices.  Its tiles (group g, column kb) are
// numbered g*nb + kb and wave w takes tiles w, w+4, w+8, ..., so the four
// waves sweep the same 16 rows at neighbouring columns; three tiles per lane
// are in flight.  Within a group a wave's tiles share kb mod 4 (its
// "class"); each lane sums its tiles of the group in order and leaves the
// sums in LDS under (row, class), and each row adds its four classes in
// order: deterministic, and the same bits whatever R or the launch (no
// atomics on values).
//
// LDS layout of the staged x, per block kb (40 chunks of 16 B): chunk
// 5 s + p holds the binary16 x of sub-block s, values 8p + {0,2,1,3,4,6,5,7}
// (the order of the codes as masked from two consecutive code dwords: bytes
// 0, 2, 1, 3 of each); the stride of 5 puts the four sub-blocks an
// instruction reads on different banks.
#include "q4k_device.h"

namespace jq4k {

constexpr int kGemvThreads = 256;
constexpr int kGemvBatchMax = 16;  // problems per batched launch
constexpr int kGemvDepth = 3;      // tiles in flight per lane
constexpr int kGemvMaxK = 16384;
constexpr int kGemvMaxXChunksPerThread = kGemvMaxK / 8 / kGemvThreads;
constexpr int kSubChunks = 5;   // LDS chunk stride of a sub-block's 4 chunks of x
constexpr int kXaChunks = 40;   // LDS chunks per block of x (8 sub-blocks)

typedef __attribute__((ext_vector_type(8))) _Float16 half8_t;
typedef __attribute__((ext_vector_type(4))) float float4_t;
typedef __attribute__((ext_vector_type(2))) unsigned short u16x2_t;
typedef __attribute__((ext_vector_type(2))) _Float16 half2_t;

__host__ __device__ constexpr int gemv_shift_words(int nb) { return (nb + 3) & ~3; }
__host__ __device__ constexpr int gemv_groups(int R) { return (R + 15) >> 4; }

// LDS of a workgroup with R rows of each of `mats` matrices (bytes):
//   staged x              nb * 40 chunks
//   zeros                 4 chunks (the A values of inactive lanes)
//   S0[8], T0[8]          per block, 16 floats
//   sh                    per block, one int (padded to 16 B)
//   row partials          mats * 16 ceil(R/16) rows x 4 classes x 4 lane slots x 2 floats
//   row results           mats * R floats
//   recompute list        1 + mats * R ints (count, then rows)
__host__ __device__ constexpr size_t gemv_lds_layout(int nb, int R, int mats) {
    return static_cast<size_t>(nb) * kXaChunks * 16 + 64 + static_cast<size_t>(nb) * 64 +
           static_cast<size_t>(gemv_shift_words(nb)) * 4 +
           static_cast<size_t>(mats) * gemv_groups(R) * 16 * 16 * 8 +
           static_cast<size_t>(mats) * R * 4 + (1 + static_cast<size_t>(mats) * R) * 4;
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

// The scale exponent of a block of x whose largest exponent field is e:
// x * 2^-sh stays below 2^15 in magnitude (binary16 overflows at 65520),
// and 2^-sh is a normal fp32 (sh in [-126, 114]; e = 255 is Inf or NaN).
__device__ __forceinline__ int block_shift(int e) { return min(max(e - 141, -126), 114); }
__device__ __forceinline__ float pow2f(int e) {
    return __builtin_bit_cast(float, static_cast<uint32_t>(127 + e) << 23);
}

struct TileLoad {
    uint4 hdr, qa, qb;   // header; code dwords 0..3 and 4..7 of the lane's quarter
};

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
// kPair: the same rows of a second matrix W2 follow in the tile list (the
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
    const long row0 = tile * R;
    const int rows = static_cast<int>(min(static_cast<long>(R), N - row0));
    const int G = gemv_groups(rows);            // row groups per matrix here
    const int Gt = kMats * G;
    const int Gl = gemv_groups(R);              // ... in a full workgroup (LDS carve)

    uint4* xa = smem;
    uint4* zero4 = xa + nb * kXaChunks;
    float* zs = reinterpret_cast<float*>(zero4 + 4);
    int* xsh = reinterpret_cast<int*>(zs + nb * 16);
    float2* part = reinterpret_cast<float2*>(xsh + gemv_shift_words(nb));
    float* yrow = reinterpret_cast<float*>(part + kMats * Gl * 16 * 16);
    int* flist = reinterpret_cast<int*>(yrow + kMats * R);

    // Lane roles.  As an A/B lane: k-group c, row / column m of the tile.
    const int c = lane >> 4, m = lane & 15;
    const bool act_lo = m == 2 * c, act_hi = m == 2 * c + 1;   // rows 8..15: never
    const int zero_chunk = nb * kXaChunks;
    const int alo_base = act_lo ? kSubChunks * m : zero_chunk;
    const int ahi_base = act_hi ? kSubChunks * m : zero_chunk;
    const int alo_stride = act_lo ? kXaChunks : 0;
    const int ahi_stride = act_hi ? kXaChunks : 0;
    // As a D lane: S (lanes 0..31: D = S1) or T (32..63: D = 0), sub-blocks
    // 4 half + 0..3 of block (row m, kb)
    const bool laneT = lane >= 32;
    const bool half = ((lane >> 4) & 1) != 0;
    const int zoff = (laneT ? 8 : 0) + (half ? 4 : 0);
    // scale bytes of sub-blocks 4 half + 0..3 (Q4_K packing): half 0 the low
    // six bits of scales[i] and scales[4+i]; half 1 the nibbles of
    // scales[8+i] plus bits 6..7 of scales[i] and scales[4+i] as bits 4..5.
    // One branch-free formula with lane-constant masks.
    const uint32_t low_mask = half ? 0x0F0F0F0Fu : 0x3F3F3F3Fu;
    const uint32_t top_mask = half ? 0x30303030u : 0u;
    const int qoff = 16 + 32 * c;

    // x first, then the first tiles of weights (vmcnt retires in order), so
    // that staging x waits only for x.
    const int nxc = nb * 32;  // 16-byte chunks of x, at most 2048 (K <= 16384)
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

    // This wave's tiles: w, w + 4, ... of the Gt * nb.  Loads past the last
    // tile repeat it (every load below is unconditional: with loads under
    // branches the compiler's count of loads in flight turns pessimistic at
    // the joins and it waits for all of them, which undoes the prefetch).
    const int ntiles = Gt * nb;
    const int mine = ntiles > wave ? (ntiles - wave + 3) >> 2 : 0;
    auto group_row = [&](int g) {
        const bool second = kPair && g >= G;
        const int gg = second ? g - G : g;
        const long r = row0 + min(16 * gg + m, rows - 1);
        return (second ? W2 : W) + r * nb * kBlockBytes + qoff;
    };
    int pi = 0, pg = 0, pkb = wave;
    while (pkb >= nb) {
        pkb -= nb;
        ++pg;
    }
    const uint8_t* prow = group_row(pg);
    auto issue = [&](TileLoad& l) {
        const uint8_t* p = prow + pkb * kBlockBytes;
        l.qa = load16(p);
        l.qb = load16(p + 16);
        l.hdr = load16(p - qoff);
        if (pi + 1 < mine) {
            ++pi;
            pkb += 4;
            const int g0 = pg;
            while (pkb >= nb) {
                pkb -= nb;
                ++pg;
            }
            if (pg != g0) prow = group_row(pg);
        }
    };
    // Two tiles go out before x is staged, the third after: a smaller first
    // burst of weight loads lets x (queued behind it) arrive sooner
    // (measured: 2 best of 0..3 on the decode layer and the LM head).
    constexpr int kEarly = 2;
    TileLoad ld[kGemvDepth];
    if (mine > 0) {
#pragma unroll
        for (int u = 0; u < kEarly; ++u) issue(ld[u]);
    }

    // LDS that is read before it is written: the zeros, the partials (a
    // class without blocks, when nb < 4, stays zero) and the list's count.
    if (t < 4) zero4[t] = make_uint4(0u, 0u, 0u, 0u);
    for (int i = t; i < Gt * 16 * 16; i += kGemvThreads) part[i] = make_float2(0.f, 0.f);
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
        if ((t & 63) == 0) wave_ss[t >> 6] = ss;
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
                const int kb = g >> 5, s = (g >> 2) & 7, p = g & 3;
                xa[kb * kXaChunks + kSubChunks * s + p] = make_uint4(h0, h1, h2, h3);
                if (p == 0) {
                    zs[kb * 16 + s] = s0;
                    zs[kb * 16 + 8 + s] = t0;
                }
                if ((g & 31) == 0) xsh[kb] = sh;
            }
        }
    }
    const bool x_inexact = __syncthreads_or(inexact) != 0;
    if (mine > 0) {
#pragma unroll
        for (int u = kEarly; u < kGemvDepth; ++u) issue(ld[u]);
    }

    // The tiles.  The lane's running sums over the tiles of its group, all
    // of one class kb mod 4 (each (group, class) belongs to one wave):
    //   S lanes   v1 = sum r (the output), v2 = sum |r| (L)
    //   T lanes   v2 = sum |dm| T0, v3 = sum 15 |d sc| T0 (v2 + v3 = B)
    // each tile's sums scaled by 2^sh_kb.  They go to slot lane / 16 of
    // (row, class) in `part` when the wave moves to the next group, so a
    // row's sums do not depend on R or on which wave ran which tile.
    int cg = 0, ckb = wave;
    while (ckb >= nb) {
        ckb -= nb;
        ++cg;
    }
    const int slot = lane >> 4;
    float v1 = 0.f, v2 = 0.f, v3 = 0.f;
    auto flush = [&](int g, int kb) {
        part[((g * 16 + m) * 4 + (kb & 3)) * 4 + slot] = make_float2(v1, laneT ? v2 + v3 : v2);
        v1 = 0.f;
        v2 = 0.f;
        v3 = 0.f;
    };
    auto compute = [&](const TileLoad& l) {
        const uint4* alo = xa + alo_base + __umul24(ckb, alo_stride);
        const uint4* ahi = xa + ahi_base + __umul24(ckb, ahi_stride);
        const uint32_t qw[8] = {l.qa.x, l.qa.y, l.qa.z, l.qa.w, l.qb.x, l.qb.y, l.qb.z, l.qb.w};
        float4_t dlo = {0.f, 0.f, 0.f, 0.f}, dhi = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const uint32_t v0 = qw[2 * p], u1 = qw[2 * p + 1];
            const uint32_t s0 = v0 >> 8, s1 = u1 >> 8;
            const uint4 blo = make_uint4(v0 & 0x000F000Fu, s0 & 0x000F000Fu,
                                         u1 & 0x000F000Fu, s1 & 0x000F000Fu);
            const uint4 bhi = make_uint4(v0 & 0x00F000F0u, s0 & 0x00F000F0u,
                                         u1 & 0x00F000F0u, s1 & 0x00F000F0u);
            dlo = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, alo[p]),
                                                         __builtin_bit_cast(half8_t, blo), dlo,
                                                         0, 0, 0);
            dhi = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, ahi[p]),
                                                         __builtin_bit_cast(half8_t, bhi), dhi,
                                                         0, 0, 0);
        }
        // sub-blocks 4 half + i: even ones from the low-nibble instructions
        // (codes q 2^-24), odd ones from the high-nibble ones (q 2^-20)
        const float D[4] = {dlo[0], dhi[1], dlo[2], dhi[3]};
        const uint4 h = l.hdr;
        const float d = half_bits_to_float(h.x & 0xFFFFu);
        const float dmin = half_bits_to_float(h.x >> 16);
        const float dE = d * 0x1p24f, dO = d * 0x1p20f, d15 = fabsf(d) * 15.0f;
        const uint32_t sc_src = half ? h.w : h.y;
        const uint32_t m_src = half ? h.w >> 4 : h.z;
        const uint32_t scb = (sc_src & low_mask) | ((h.y >> 2) & top_mask);
        const uint32_t mb = (m_src & low_mask) | ((h.z >> 2) & top_mask);
        const float4_t Z = *reinterpret_cast<const float4_t*>(zs + ckb * 16 + zoff);
        const float sc[4] = {ubyte_to_float<0>(scb), ubyte_to_float<1>(scb),
                             ubyte_to_float<2>(scb), ubyte_to_float<3>(scb)};
        const float mm[4] = {ubyte_to_float<0>(mb), ubyte_to_float<1>(mb),
                             ubyte_to_float<2>(mb), ubyte_to_float<3>(mb)};
        float r[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float ds = ((i & 1) ? dO : dE) * sc[i];
            const float a = (dmin * mm[i]) * Z[i];
            r[i] = __builtin_fmaf(ds, D[i], -a);
        }
        const float zsc = ((sc[0] * Z[0] + sc[1] * Z[1]) + (sc[2] * Z[2] + sc[3] * Z[3]));
        const int sh = xsh[ckb];
        v1 += __builtin_amdgcn_ldexpf((r[0] + r[1]) + (r[2] + r[3]), sh);
        v2 += __builtin_amdgcn_ldexpf((fabsf(r[0]) + fabsf(r[1])) + (fabsf(r[2]) + fabsf(r[3])),
                                      sh);
        v3 += __builtin_amdgcn_ldexpf(d15 * zsc, sh);
        // next tile of this wave
        const int kb0 = ckb;
        ckb += 4;
        const int g0 = cg;
        while (ckb >= nb) {
            ckb -= nb;
            ++cg;
        }
        if (cg != g0) flush(g0, kb0);
    };
    if (mine > 0) {
        int i = 0;
        for (; i + kGemvDepth <= mine; i += kGemvDepth) {
#pragma unroll
            for (int u = 0; u < kGemvDepth; ++u) {
                compute(ld[u]);
                issue(ld[u]);
            }
        }
#pragma unroll
        for (int u = 0; u + 1 < kGemvDepth; ++u)
            if (i + u < mine) compute(ld[u]);
        // the last group, unless its last tile ended it (then cg >= Gt and
        // the group was flushed in compute)
        if (cg < Gt) flush(cg, ckb);
    }
    __syncthreads();

    // Rows: the classes' sums in a fixed order, the certificate, and the list
    // of rows to recompute (the list's order does not matter: a row's
    // recomputation is the same whichever wave runs it).
    const float kE = (192.0f + static_cast<float>(nb)) * 0x1p-24f;
    for (int q = t; q < kMats * rows; q += kGemvThreads) {
        const int mat = (kPair && q >= rows) ? 1 : 0;
        const int qq = q - mat * rows;
        const float2* pr = part + (mat * G * 16 + qq) * 16;
        float y = 0.f, L = 0.f, B = 0.f;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            y += pr[4 * k].x + pr[4 * k + 1].x;
            L += pr[4 * k].y + pr[4 * k + 1].y;
            B += pr[4 * k + 2].y + pr[4 * k + 3].y;
        }
        const float E = kE * B;
        const float lb = fmaxf(L - 2.0f * E, fabsf(y) - E);
        yrow[q] = y;
        if (x_inexact || !(E <= 1.9e-3f * lb + 0.99e-5f)) flist[1 + atomicAdd(flist, 1)] = q;
    }
    __syncthreads();
    const int nredo = flist[0];
    for (int e = wave; e < nredo; e += 4) {
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
