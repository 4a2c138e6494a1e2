// probes.hip -- measurement kernels for the benchmark's ceilings: what this
// GPU reaches on streaming reads of HBM and on a loop of bf16 matrix
// instructions, beside the published peaks the roofline fractions use.  None
// is on the matmul path.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "jq4k_probe.h"

namespace jq4k {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_p;
typedef __attribute__((ext_vector_type(16))) float float16_p;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4_p;

constexpr int kProbeThreads = 256;
constexpr int kReadUnroll = 8;

// Every lane reads 16 bytes per load, kReadUnroll loads in flight, the grid
// striding over the buffer; the XOR of everything read goes to sink[thread]
// so that no load is dead.
__global__ __launch_bounds__(kProbeThreads) void probe_read_kernel(const u32x4_p* __restrict__ p,
                                                                   long n16,
                                                                   uint32_t* __restrict__ sink) {
    const long tid = blockIdx.x * static_cast<long>(kProbeThreads) + threadIdx.x;
    const long stride = static_cast<long>(gridDim.x) * kProbeThreads;
    u32x4_p acc = {0u, 0u, 0u, 0u};
    long i = tid;
    for (; i + (kReadUnroll - 1) * stride < n16; i += kReadUnroll * stride) {
        u32x4_p v[kReadUnroll];
#pragma unroll
        for (int u = 0; u < kReadUnroll; ++u) v[u] = p[i + u * stride];
#pragma unroll
        for (int u = 0; u < kReadUnroll; ++u) acc ^= v[u];
    }
    for (; i < n16; i += stride) acc ^= p[i];
    sink[tid] = acc.x ^ acc.y ^ acc.z ^ acc.w;
}

// A second streaming read, in the pattern that reads HBM fastest here: a
// workgroup per 36 KB, each thread nine 16-byte non-temporal loads in flight,
// each wave instruction 1 KB of consecutive bytes, then the workgroup ends
// (short-lived workgroups keep every CU's queue full without a loop).
constexpr int kStreamLoads = 9;
constexpr long kStreamChunks = static_cast<long>(kProbeThreads) * kStreamLoads;

__global__ __launch_bounds__(kProbeThreads) void probe_stream_kernel(const u32x4_p* __restrict__ p,
                                                                     long n16,
                                                                     uint32_t* __restrict__ sink) {
    const long base = blockIdx.x * kStreamChunks + threadIdx.x;
    u32x4_p v[kStreamLoads];
#pragma unroll
    for (int k = 0; k < kStreamLoads; ++k) {
        const long i = min(base + static_cast<long>(k) * kProbeThreads, n16 - 1);
        v[k] = __builtin_nontemporal_load(p + i);
    }
    u32x4_p acc = v[0];
#pragma unroll
    for (int k = 1; k < kStreamLoads; ++k) acc ^= v[k];
    const uint32_t x = acc.x ^ acc.y ^ acc.z ^ acc.w;
    if (x == 0x9E3779B9u) sink[threadIdx.x] = x;   // keeps the loads live; writes almost never
}

// Eight independent chains of v_mfma_f32_32x32x16_bf16 per wave on register
// operands, `iters` rounds; the accumulators' sum goes to sink[thread].
__global__ __launch_bounds__(kProbeThreads) void probe_mfma_kernel(long iters,
                                                                   float* __restrict__ sink) {
    const uint32_t t = threadIdx.x;
    const bf16x8_p a = __builtin_bit_cast(bf16x8_p, u32x4_p{0x3F803F80u ^ (t & 1u), 0x3F803F80u,
                                                            0x3F803F80u, 0x3F803F80u});
    const bf16x8_p b = __builtin_bit_cast(bf16x8_p, u32x4_p{0x3C003C00u, 0x3C003C00u ^ (t & 2u),
                                                            0x3C003C00u, 0x3C003C00u});
    float16_p acc[8];
#pragma unroll
    for (int c = 0; c < 8; ++c)
        for (int e = 0; e < 16; ++e) acc[c][e] = 0.f;
    for (long it = 0; it < iters; ++it) {
#pragma unroll
        for (int c = 0; c < 8; ++c)
            acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[c], 0, 0, 0);
    }
    float s = 0.f;
#pragma unroll
    for (int c = 0; c < 8; ++c)
        for (int e = 0; e < 16; ++e) s += acc[c][e];
    sink[blockIdx.x * kProbeThreads + t] = s;
}

typedef __attribute__((ext_vector_type(4))) int int4_p;
typedef __attribute__((ext_vector_type(4))) float float4_p;

// The inner loop of an int8-activation Q4_K matmul (activations quantised to
// int8 per 32 values with one fp32 scale each, weights as their 4-bit codes):
// a wave owns a 64 x 64 output tile in fp32; for every sub-block of 32 k it
// issues the 16 v_mfma_i32_16x16x32_i8 of the tile (exact int32 sums over
// the sub-block) and rescales each int32 sum into the fp32 tile,
//   y += (d sc)_n (dx_m S) - (dmin m)_n (dx sx)_m,
// as the sub-block's scales differ per row of W and per activation block.
// Operands come from registers (no loads, no code unpacking, no activation
// quantisation): an upper bound on such a kernel's rate on this chip.
__global__ __launch_bounds__(kProbeThreads) void probe_mmq_kernel(long iters,
                                                                  float* __restrict__ sink) {
    const uint32_t t = threadIdx.x;
    const long a = 0x0102030405060708L ^ t, b = 0x0807060504030201L + t;
    float4_p y[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) y[i] = float4_p{0.f, 0.f, 0.f, 0.f};
    float ds[4], dm[4], dx[4][4], dxs[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        ds[i] = 1e-3f * (i + 1 + (t & 3));
        dm[i] = 2e-3f * (i + 1);
        for (int r = 0; r < 4; ++r) {
            dx[i][r] = 1e-2f * (r + 1 + i);
            dxs[i][r] = 3e-2f * (r + i);
        }
    }
    for (long it = 0; it < iters; ++it) {
#pragma unroll
        for (int mi = 0; mi < 4; ++mi)
#pragma unroll
            for (int ni = 0; ni < 4; ++ni) {
                const int4_p s = __builtin_amdgcn_mfma_i32_16x16x32_i8(
                    a + mi, b + ni, int4_p{0, 0, 0, 0}, 0, 0, 0);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float f = static_cast<float>(s[r]);
                    y[mi * 4 + ni][r] = __builtin_fmaf(ds[ni], dx[mi][r] * f,
                                                       __builtin_fmaf(-dm[ni], dxs[mi][r],
                                                                      y[mi * 4 + ni][r]));
                }
            }
        // next sub-block: other scales
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            ds[i] += 1e-7f;
            dx[i][0] += 1e-7f;
        }
    }
    float acc = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) acc += y[i][0] + y[i][1] + y[i][2] + y[i][3];
    sink[blockIdx.x * kProbeThreads + t] = acc;
}

}  // namespace jq4k

extern "C" {

int jq4k_probe_read(const void* p, size_t bytes, uint32_t* sink, int workgroups,
                    hipStream_t stream) {
    if (p == nullptr || sink == nullptr || workgroups <= 0 || bytes % 16 != 0 ||
        reinterpret_cast<uintptr_t>(p) % 16 != 0)
        return -1;
    if (bytes == 0) return 0;
    hipLaunchKernelGGL(jq4k::probe_read_kernel, dim3(workgroups), dim3(jq4k::kProbeThreads), 0,
                       stream, static_cast<const jq4k::u32x4_p*>(p),
                       static_cast<long>(bytes / 16), sink);
    return static_cast<int>(hipGetLastError());
}

int jq4k_probe_stream(const void* p, size_t bytes, uint32_t* sink, hipStream_t stream) {
    if (p == nullptr || sink == nullptr || bytes % 16 != 0 ||
        reinterpret_cast<uintptr_t>(p) % 16 != 0)
        return -1;
    if (bytes == 0) return 0;
    const long n16 = static_cast<long>(bytes / 16);
    const long grid = (n16 + jq4k::kStreamChunks - 1) / jq4k::kStreamChunks;
    if (grid > 0x7FFFFFFFL) return -1;
    hipLaunchKernelGGL(jq4k::probe_stream_kernel, dim3(static_cast<unsigned>(grid)),
                       dim3(jq4k::kProbeThreads), 0, stream,
                       static_cast<const jq4k::u32x4_p*>(p), n16, sink);
    return static_cast<int>(hipGetLastError());
}

int jq4k_probe_mfma(long iters, float* sink, int workgroups, hipStream_t stream) {
    if (sink == nullptr || workgroups <= 0 || iters < 0) return -1;
    hipLaunchKernelGGL(jq4k::probe_mfma_kernel, dim3(workgroups), dim3(jq4k::kProbeThreads), 0,
                       stream, iters, sink);
    return static_cast<int>(hipGetLastError());
}

int jq4k_probe_mmq(long iters, float* sink, int workgroups, hipStream_t stream) {
    if (sink == nullptr || workgroups <= 0 || iters < 0) return -1;
    hipLaunchKernelGGL(jq4k::probe_mmq_kernel, dim3(workgroups), dim3(jq4k::kProbeThreads), 0,
                       stream, iters, sink);
    return static_cast<int>(hipGetLastError());
}

}  // extern "C"
