// kv_convert.hip -- FP16 <-> INT8 KV-cache convert (the genie-ai-runtime
// README, "Project layout": FP16<->INT8 KV convert; "At a glance": an INT8 KV
// cache by default, with FP16-ULP-bounded drift).
//
// One KV vector (a token's head, dim binary16 values) has one fp32 scale
// s = max|v| / 127 and int8 codes q = rint(v / s) (q = 0 when s = 0); the
// dequantised values are fp16(fp32(q * s)), round to nearest even.  Every
// step is one IEEE operation (correctly rounded division and product), so the
// codes, scales and fp16 values are fixed bit for bit.
//
// The codes without a division per value.  With y = 1/s correctly rounded
// (one division per lane), q0 = v*y rounded, the residual r = v - q0*s (one
// fma) and q1 = q0 + r*y (one fma), rint(q1) equals rint(v / s) for every
// binary16 v and every binary16 max|v| >= |v| (an exhaustive check over all
// such pairs, run by the tests on the CPU).  A vector whose scale is zero or
// infinite takes the division.
//
// Both directions stream: 3 + 4/dim bytes per value.  A vector is handled by
// G lanes (G = the power of two >= dim / 8, at most 64): lane j of the group
// owns values 8j .. 8j + 7 (one 16-byte fp16 load, one 8-byte code store),
// the group's max comes from a butterfly over its G lanes, and 64 / G vectors
// share a wave.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace jq4k {

constexpr int kKvThreads = 256;

template <int G>
__global__ __launch_bounds__(kKvThreads) void kv_quant_kernel(const uint16_t* __restrict__ v,
                                                              int8_t* __restrict__ q,
                                                              float* __restrict__ scale,
                                                              long nvec, int dim) {
    const long gid = static_cast<long>(blockIdx.x) * kKvThreads + threadIdx.x;
    const long vec = gid / G;
    const int j = static_cast<int>(gid % G);
    const bool live = vec < nvec && 8 * j < dim;
    float x[8];
    float amax = 0.f;
    if (live) {
        const uint4 raw = *reinterpret_cast<const uint4*>(v + vec * dim + 8 * j);
        const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            x[2 * i] = static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(w[i])));
            x[2 * i + 1] =
                static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(w[i] >> 16)));
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(x[i]));
    }
    // max over the vector's G lanes (a butterfly inside the aligned group)
#pragma unroll
    for (int o = G / 2; o > 0; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o, G));
    if (!live) return;
    const float s = amax / 127.0f;
    const float y = 1.0f / s;
    const bool finite = s != 0.0f && s < __builtin_inff();
    uint32_t packed[2] = {0u, 0u};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        float c;
        if (finite) {
            const float q0 = __fmul_rn(x[i], y);
            const float r = __builtin_fmaf(-q0, s, x[i]);
            c = rintf(__builtin_fmaf(r, y, q0));
        } else {
            c = s != 0.0f ? rintf(x[i] / s) : 0.0f;
        }
        c = fminf(fmaxf(c, -127.0f), 127.0f);
        const uint32_t b = static_cast<uint32_t>(static_cast<int>(c)) & 0xFFu;
        packed[i >> 2] |= b << (8 * (i & 3));
    }
    *reinterpret_cast<uint2*>(q + vec * dim + 8 * j) = make_uint2(packed[0], packed[1]);
    if (j == 0) scale[vec] = s;
}

template <int G>
__global__ __launch_bounds__(kKvThreads) void kv_dequant_kernel(const int8_t* __restrict__ q,
                                                                const float* __restrict__ scale,
                                                                uint16_t* __restrict__ v,
                                                                long nvec, int dim) {
    const long gid = static_cast<long>(blockIdx.x) * kKvThreads + threadIdx.x;
    const long vec = gid / G;
    const int j = static_cast<int>(gid % G);
    if (vec >= nvec || 8 * j >= dim) return;
    const float s = scale[vec];
    const uint2 raw = *reinterpret_cast<const uint2*>(q + vec * dim + 8 * j);
    const uint32_t w[2] = {raw.x, raw.y};
    uint32_t out[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int8_t c0 = static_cast<int8_t>(w[i >> 1] >> (16 * (i & 1)));
        const int8_t c1 = static_cast<int8_t>(w[i >> 1] >> (16 * (i & 1) + 8));
        // the fp32 product is kept as a register value before its fp16
        // conversion: otherwise the compiler fuses both into one
        // mixed-precision instruction that rounds once, which differs from
        // rounding to fp32 and then to fp16 on rare ties
        float p0 = static_cast<float>(c0) * s, p1 = static_cast<float>(c1) * s;
        asm volatile("" : "+v"(p0), "+v"(p1));
        const _Float16 h0 = static_cast<_Float16>(p0);
        const _Float16 h1 = static_cast<_Float16>(p1);
        out[i] = static_cast<uint32_t>(__builtin_bit_cast(uint16_t, h0)) |
                 (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, h1)) << 16);
    }
    *reinterpret_cast<uint4*>(v + vec * dim + 8 * j) = make_uint4(out[0], out[1], out[2], out[3]);
}

// Lanes per vector: the power of two >= dim / 8 (dim a multiple of 8, <= 512).
int kv_group(int dim) {
    int g = 1;
    while (8 * g < dim) g *= 2;
    return g;
}

long kv_grid(long nvec, int dim) {
    const long threads = nvec * kv_group(dim);
    return (threads + kKvThreads - 1) / kKvThreads;
}

#define JQ4K_KV_DISPATCH(KERNEL, ...)                                                        \
    switch (kv_group(dim)) {                                                                 \
        case 1: hipLaunchKernelGGL(KERNEL<1>, grid, dim3(kKvThreads), 0, stream, __VA_ARGS__); break;   \
        case 2: hipLaunchKernelGGL(KERNEL<2>, grid, dim3(kKvThreads), 0, stream, __VA_ARGS__); break;   \
        case 4: hipLaunchKernelGGL(KERNEL<4>, grid, dim3(kKvThreads), 0, stream, __VA_ARGS__); break;   \
        case 8: hipLaunchKernelGGL(KERNEL<8>, grid, dim3(kKvThreads), 0, stream, __VA_ARGS__); break;   \
        case 16: hipLaunchKernelGGL(KERNEL<16>, grid, dim3(kKvThreads), 0, stream, __VA_ARGS__); break; \
        case 32: hipLaunchKernelGGL(KERNEL<32>, grid, dim3(kKvThreads), 0, stream, __VA_ARGS__); break; \
        default: hipLaunchKernelGGL(KERNEL<64>, grid, dim3(kKvThreads), 0, stream, __VA_ARGS__); break; \
    }

hipError_t launch_kv_quant(const uint16_t* v, int8_t* q, float* scale, long nvec, int dim,
                           hipStream_t stream) {
    const dim3 grid(static_cast<unsigned>(kv_grid(nvec, dim)));
    JQ4K_KV_DISPATCH(kv_quant_kernel, v, q, scale, nvec, dim)
    return hipGetLastError();
}

hipError_t launch_kv_dequant(const int8_t* q, const float* scale, uint16_t* v, long nvec, int dim,
                             hipStream_t stream) {
    const dim3 grid(static_cast<unsigned>(kv_grid(nvec, dim)));
    JQ4K_KV_DISPATCH(kv_dequant_kernel, q, scale, v, nvec, dim)
    return hipGetLastError();
}

#undef JQ4K_KV_DISPATCH

}  // namespace jq4k
