// exports.hip -- field unpack and dequantisation of whole blocks, for tests.
//
// These run the same device routines the matmul kernels run (scale_min_pair,
// low_quants / high_quants, quarter_scales, dequant_dword_f32/_bf16), one
// workgroup of 64 threads per block: threads 0..31 take one quant dword each
// (quarter c = t / 8, byte offset p = 4 (t % 8)), threads 32..35 the scale
// and min pair of quarter t - 32.
#include "q4k_device.h"

namespace jq4k {

constexpr int kExportThreads = 64;
constexpr unsigned kExportMaxGrid = 65536;

enum class ExportKind { kFields, kF32, kBf16 };

template <ExportKind kind>
__global__ __launch_bounds__(kExportThreads) void q4k_export_kernel(
    const uint8_t* __restrict__ W, long nblocks, uint8_t* __restrict__ q,
    uint8_t* __restrict__ sc, uint8_t* __restrict__ m, float* __restrict__ wf,
    uint32_t* __restrict__ wh, uint32_t qmask) {
    const int t = threadIdx.x;
    for (long b = blockIdx.x; b < nblocks; b += gridDim.x) {
        const uint8_t* blk = W + b * kBlockBytes;
        const uint4 hdr = *reinterpret_cast<const uint4*>(blk);
        if (t < 32) {
            const int c = t >> 3, p = 4 * (t & 7);
            const uint32_t v = *reinterpret_cast<const uint32_t*>(blk + 16 + 32 * c + p);
            const long lo0 = b * kQK + 64 * c + p;  // first even-sub-block weight
            const long hi0 = lo0 + 32;              // first odd-sub-block weight
            if constexpr (kind == ExportKind::kFields) {
                const uint32_t ql = low_quants_rt(v, qmask), qh = high_quants_rt(v, qmask);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    q[lo0 + i] = static_cast<uint8_t>(ql >> (8 * i));
                    q[hi0 + i] = static_cast<uint8_t>(qh >> (8 * i));
                }
            } else if constexpr (kind == ExportKind::kF32) {
                const QuarterScales s = quarter_scales(hdr, static_cast<uint32_t>(c));
                float lo[4], hi[4];
                dequant_dword_f32(v, s, lo, hi, qmask);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    wf[lo0 + i] = lo[i];
                    wf[hi0 + i] = hi[i];
                }
            } else {
                const QuarterScales s = quarter_scales(hdr, static_cast<uint32_t>(c));
                uint32_t lo2[2], hi2[2];
                dequant_dword_bf16(v, s, lo2, hi2, qmask);
                wh[lo0 / 2] = lo2[0];
                wh[lo0 / 2 + 1] = lo2[1];
                wh[hi0 / 2] = hi2[0];
                wh[hi0 / 2 + 1] = hi2[1];
            }
        } else if constexpr (kind == ExportKind::kFields) {
            if (t < 36) {
                const int c = t - 32;
                uint32_t scp, mp;
                scale_min_pair(static_cast<uint32_t>(c), hdr.y, hdr.z, hdr.w, &scp, &mp);
                sc[b * 8 + 2 * c] = static_cast<uint8_t>(scp);
                sc[b * 8 + 2 * c + 1] = static_cast<uint8_t>(scp >> 8);
                m[b * 8 + 2 * c] = static_cast<uint8_t>(mp);
                m[b * 8 + 2 * c + 1] = static_cast<uint8_t>(mp >> 8);
            }
        }
    }
}

static unsigned export_grid(long nblocks) {
    return static_cast<unsigned>(nblocks < static_cast<long>(kExportMaxGrid) ? nblocks
                                                                             : kExportMaxGrid);
}

hipError_t launch_unpack_fields(const uint8_t* W, long nblocks, uint8_t* q, uint8_t* sc,
                                uint8_t* m, hipStream_t stream) {
    hipLaunchKernelGGL(q4k_export_kernel<ExportKind::kFields>, dim3(export_grid(nblocks)),
                       dim3(kExportThreads), 0, stream, W, nblocks, q, sc, m, nullptr, nullptr, kNibbleMask);
    return hipGetLastError();
}

hipError_t launch_dequant_f32(const uint8_t* W, long nblocks, float* w, hipStream_t stream) {
    hipLaunchKernelGGL(q4k_export_kernel<ExportKind::kF32>, dim3(export_grid(nblocks)),
                       dim3(kExportThreads), 0, stream, W, nblocks, nullptr, nullptr, nullptr, w,
                       nullptr, kNibbleMask);
    return hipGetLastError();
}

hipError_t launch_dequant_bf16(const uint8_t* W, long nblocks, uint16_t* w, hipStream_t stream) {
    hipLaunchKernelGGL(q4k_export_kernel<ExportKind::kBf16>, dim3(export_grid(nblocks)),
                       dim3(kExportThreads), 0, stream, W, nblocks, nullptr, nullptr, nullptr,
                       nullptr, reinterpret_cast<uint32_t*>(w), kNibbleMask);
    return hipGetLastError();
}

}  // namespace jq4k
