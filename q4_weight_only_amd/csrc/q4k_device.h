// q4k_device.h -- device-side Q4_K unpacking shared by every kernel of
// libjq4k (the M = 1 GEMV, the MFMA GEMM and the test exports), so that the
// exports' bit-exact checks exercise the hot path's own code.
//
// Format: GGUF's Q4_K super-block (genie-ai-runtime README, "At a glance":
// GGUF models, Qwen3-4B-Q4_K_M; kernels "INT4 dequant-fused GEMV" and
// "tensor-core MMQ Q4_K prefill").  A 144-byte block is nine 16-byte chunks:
//   chunk 0      header: d | dmin << 16, then scales[0..3], [4..7], [8..11]
//   chunks 1..8  qs[128]; the 32 bytes of "quarter" c (bytes 32c..32c+31)
//                hold weights 64c + l in their low nibbles and 64c + 32 + l in
//                their high nibbles (l = 0..31), i.e. sub-blocks 2c and 2c+1.
//   w = d * sc_s * q - dmin * m_s.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace jq4k {

constexpr int kQK = 256;          // weights per block
constexpr int kBlockBytes = 144;  // bytes per block
constexpr uint32_t kNibbleMask = 0x0F0F0F0Fu;  // value of the run-time `mask` arguments

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(2))) float float2_t;
typedef __attribute__((ext_vector_type(16))) float float16_t;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4_t;

// 16-byte global load (global_load_dwordx4).  A plain load: the
// non-temporal hint measured about 25% slower for streaming weights.
__device__ __forceinline__ uint4 load16(const void* p) {
    const u32x4_t v = *static_cast<const u32x4_t*>(p);
    return make_uint4(v.x, v.y, v.z, v.w);
}

// binary16 bit pattern (low 16 bits) -> fp32, exact.
__device__ __forceinline__ float half_bits_to_float(uint32_t bits) {
    return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(bits)));
}

// Scales and mins of sub-blocks 2c and 2c+1 (c = quarter, 0..3) from the
// scale dwords s0 = scales[0..3], s1 = scales[4..7], s2 = scales[8..11].
// Returns sc_(2c) | sc_(2c+1) << 8 in *sc and the same for the mins in *m.
// Sub-blocks j < 4 (c < 2): the low six bits of scales[j] and scales[j+4].
// Sub-blocks j >= 4 (c >= 2): low four bits from scales[j+4] (scale in the
// low nibble, min in the high one), top two bits from bits 6..7 of
// scales[j-4] (scale) and scales[j] (min).  Both cases read the byte pair at
// shift 16 * (c & 1); the choice between them is a select, so the routine is
// branch-free whether c is uniform or differs across lanes.
__device__ __forceinline__ void scale_min_pair(uint32_t c, uint32_t s0, uint32_t s1,
                                               uint32_t s2, uint32_t* sc, uint32_t* m) {
    const uint32_t sh = (c & 1u) << 4;
    const uint32_t a = s0 >> sh, b = s1 >> sh, e = s2 >> sh;
    const uint32_t sc_lo = a & 0x3F3Fu;
    const uint32_t m_lo = b & 0x3F3Fu;
    const uint32_t sc_hi = (e & 0x0F0Fu) | ((a >> 2) & 0x3030u);
    const uint32_t m_hi = ((e >> 4) & 0x0F0Fu) | ((b >> 2) & 0x3030u);
    const bool high = c >= 2u;
    *sc = high ? sc_hi : sc_lo;
    *m = high ? m_hi : m_lo;
}

// The quant nibbles of one qs dword (4 bytes), one quant per byte:
// low nibbles -> the 4 weights of the even sub-block, high -> the odd one.
__device__ __forceinline__ uint32_t low_quants(uint32_t v) { return v & 0x0F0F0F0Fu; }
__device__ __forceinline__ uint32_t high_quants(uint32_t v) { return (v >> 4) & 0x0F0F0F0Fu; }

// The same with the nibble mask supplied at run time (a kernel argument equal
// to 0x0F0F0F0F).  With a compile-time mask the compiler turns "mask, then
// convert byte k" into a bit-field extract plus a byte-0 convert, one extra
// instruction per weight; an opaque mask keeps one v_cvt_f32_ubyte{k} per
// weight.
__device__ __forceinline__ uint32_t low_quants_rt(uint32_t v, uint32_t mask) { return v & mask; }
__device__ __forceinline__ uint32_t high_quants_rt(uint32_t v, uint32_t mask) {
    return (v >> 4) & mask;
}

// Byte k of a 32-bit word as fp32 (one v_cvt_f32_ubyte{k} when the compiler
// cannot see which bits of the word are zero; see low_quants_rt).
template <int k>
__device__ __forceinline__ float ubyte_to_float(uint32_t v) {
    return static_cast<float>((v >> (8 * k)) & 0xFFu);
}

// Per-sub-block affine constants of a quarter: w = ds * q - dm.
struct QuarterScales {
    float ds0, dm0;  // even sub-block 2c
    float ds1, dm1;  // odd sub-block 2c+1
};

// From the 16-byte header chunk and the quarter index.  d*sc and dmin*m are
// exact in fp32 (at most 11 + 6 significant bits), so fma(ds, q, -dm) is the
// exact value rounded once.
__device__ __forceinline__ QuarterScales quarter_scales(uint4 hdr, uint32_t c) {
    const float d = half_bits_to_float(hdr.x & 0xFFFFu);
    const float dmin = half_bits_to_float(hdr.x >> 16);
    uint32_t scp, mp;
    scale_min_pair(c, hdr.y, hdr.z, hdr.w, &scp, &mp);
    QuarterScales s;
    s.ds0 = d * ubyte_to_float<0>(scp);
    s.ds1 = d * ubyte_to_float<1>(scp);
    s.dm0 = dmin * ubyte_to_float<0>(mp);
    s.dm1 = dmin * ubyte_to_float<1>(mp);
    return s;
}

// fp32 weights of one qs dword: lo[0..3] are weights 64c + p + 0..3 and
// hi[0..3] are weights 64c + 32 + p + 0..3, p = byte offset within the quarter.
// `mask` is 0x0F0F0F0F, passed in at run time (see low_quants_rt).
__device__ __forceinline__ void dequant_dword_f32(uint32_t v, const QuarterScales& s,
                                                  float lo[4], float hi[4], uint32_t mask) {
    const uint32_t ql = low_quants_rt(v, mask), qh = high_quants_rt(v, mask);
    lo[0] = __builtin_fmaf(s.ds0, ubyte_to_float<0>(ql), -s.dm0);
    lo[1] = __builtin_fmaf(s.ds0, ubyte_to_float<1>(ql), -s.dm0);
    lo[2] = __builtin_fmaf(s.ds0, ubyte_to_float<2>(ql), -s.dm0);
    lo[3] = __builtin_fmaf(s.ds0, ubyte_to_float<3>(ql), -s.dm0);
    hi[0] = __builtin_fmaf(s.ds1, ubyte_to_float<0>(qh), -s.dm1);
    hi[1] = __builtin_fmaf(s.ds1, ubyte_to_float<1>(qh), -s.dm1);
    hi[2] = __builtin_fmaf(s.ds1, ubyte_to_float<2>(qh), -s.dm1);
    hi[3] = __builtin_fmaf(s.ds1, ubyte_to_float<3>(qh), -s.dm1);
}

// Two fp32 -> packed bf16 pair, round-to-nearest-even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    const float2_t f = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_t));
}

typedef __attribute__((ext_vector_type(2))) _Float16 half2_t;

// The bf16 dequantisation below reads quants as binary16 subnormals: a build
// that flushes denormals would turn them into zeros.
#if defined(__FAST_MATH__)
#error "q4k kernels need denormals preserved; build without -ffast-math"
#endif

// fma(scale, (float)h, c) for a binary16 half h of a 32-bit word: one
// v_fma_mix_f32, which widens h exactly (binary16 subnormals included: the
// kernels run with denormals preserved) and rounds once.
__device__ __forceinline__ float fma_half_lo(float scale, uint32_t h2, float c) {
    return __builtin_fmaf(scale, static_cast<float>(__builtin_bit_cast(half2_t, h2)[0]), c);
}
__device__ __forceinline__ float fma_half_hi(float scale, uint32_t h2, float c) {
    return __builtin_fmaf(scale, static_cast<float>(__builtin_bit_cast(half2_t, h2)[1]), c);
}

// bf16 weights of one qs dword, as two packed pairs per half:
// lo2[0] = (w0, w1), lo2[1] = (w2, w3) of the even sub-block; hi2 likewise.
// The same values as dequant_dword_f32 rounded to bf16, with no integer to
// float conversion: a low nibble masked in place in a 16-bit half is the
// binary16 subnormal q * 2^-24, a high nibble q * 2^-20, so with ds scaled by
// 2^24 (2^20; exact, a power of two) fma(ds', h, -dm) is ds * q - dm rounded
// once.  Per 8 weights: 1 shift, 4 masks, 8 v_fma_mix_f32, 4 bf16 packs.
// `mask` is 0x0F0F0F0F at run time (see low_quants_rt).
__device__ __forceinline__ void dequant_dword_bf16(uint32_t v, const QuarterScales& s,
                                                   uint32_t lo2[2], uint32_t hi2[2],
                                                   uint32_t mask) {
    const uint32_t m_lo = mask & 0x000F000Fu;   // bits 0-3 of each half
    const uint32_t m_hi = m_lo << 4;            // bits 4-7 of each half
    const uint32_t v8 = v >> 8;
    const uint32_t a02 = v & m_lo, a13 = v8 & m_lo;    // even sub-block, weights 0,2 / 1,3
    const uint32_t b02 = v & m_hi, b13 = v8 & m_hi;    // odd sub-block
    const float s0 = s.ds0 * 0x1p24f, s1 = s.ds1 * 0x1p20f;
    lo2[0] = pack_bf16x2(fma_half_lo(s0, a02, -s.dm0), fma_half_lo(s0, a13, -s.dm0));
    lo2[1] = pack_bf16x2(fma_half_hi(s0, a02, -s.dm0), fma_half_hi(s0, a13, -s.dm0));
    hi2[0] = pack_bf16x2(fma_half_lo(s1, b02, -s.dm1), fma_half_lo(s1, b13, -s.dm1));
    hi2[1] = pack_bf16x2(fma_half_hi(s1, b02, -s.dm1), fma_half_hi(s1, b13, -s.dm1));
}

// ---- binary16 activations (the M = 1 GEMV) ----------------------------

// Two fp32 -> packed binary16 pair, round-to-nearest-even
// (v_cvt_pk_f16_f32).  Written as the instruction so that the compiler
// cannot fold it into the fma producing its inputs (v_fma_mix{lo,hi}_f16 round
// once from the exact value and issue at about half the rate).
__device__ __forceinline__ uint32_t pack_f16x2(float a, float b) {
    uint32_t r;
    asm("v_cvt_pk_f16_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
    return r;
}

// silu(z) = z * sigmoid(z) = z / (1 + exp(-z)), fp32 (the SwiGLU epilogues),
// on the hardware's base-2 exponential and reciprocal (v_exp_f32, v_rcp_f32;
// about 1 ulp each): exp(-z) = 2^(-z log2 e).  For very negative z the
// exponential overflows to inf and the reciprocal to 0, giving the limit -0;
// for large z it gives z.
__device__ __forceinline__ float silu(float z) {
    constexpr float kLog2e = 1.4426950408889634f;
    return z * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-z * kLog2e));
}

}  // namespace jq4k
