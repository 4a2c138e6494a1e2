// probes.hip -- two measurement kernels for the benchmark's ceilings: what
// this GPU reaches on a plain streaming read of HBM and on a loop of bf16
// matrix instructions, beside the published peaks the roofline fractions
// use.  Neither is on the matmul path.
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

int jq4k_probe_mfma(long iters, float* sink, int workgroups, hipStream_t stream) {
    if (sink == nullptr || workgroups <= 0 || iters < 0) return -1;
    hipLaunchKernelGGL(jq4k::probe_mfma_kernel, dim3(workgroups), dim3(jq4k::kProbeThreads), 0,
                       stream, iters, sink);
    return static_cast<int>(hipGetLastError());
}

}  // extern "C"
