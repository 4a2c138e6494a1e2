// gemm_skinny.hip -- Q4_K matmul for small M (2 .. 64 tokens, a short
// prompt's prefill), on the gfx950 matrix cores.
//
// Y (M x N) = X (M x K) . W^T with W in Q4_K (genie-ai-runtime README, "At a
// glance": "tensor-core MMQ Q4_K prefill").  At these M the matmul streams W
// from HBM about as a GEMV does (each weight meets at most 64 tokens), so the
// design keeps the per-weight work low and the weights out of LDS:
//   * a workgroup (4 waves) computes 64 rows of W (output features) x all M,
//     one 16-row tile of W per wave, over a range of K (split K below);
//   * each wave loads its W straight into registers and dequantises it there
//     (fma(d*sc, q, -dmin*m), the exact value rounded once, then RNE to
//     bf16) into the B operand of v_mfma_f32_16x16x32_bf16;
//   * X (bf16) goes through LDS, one half block (128 of K) per stage, double
//     buffered and shared by the four waves; its rows past M read as zeros
//     (buffer loads with a range check), so M is padded to 16 MT rows;
//   * one barrier per stage; W has kSkDepth stages in flight per wave.
//
// Operand layout.  The matrix instruction sums over its 32 k positions in
// any order, so the kernel assigns k to (lane, item) to fit Q4_K: lane l of a
// wave (n = l % 16, part p = l / 16) loads the 16 quant bytes
// qs[64 h + 16 p .. +15] of its row's block, half h of the block, i.e. quarter
// c = 2h + p/2, byte offset 16 (p & 1).  Their low nibbles are weights
// 64c + 16(p & 1) + 0..15 (sub-block 2c), the high nibbles the same + 32
// (sub-block 2c+1).  K-step t = 0..3 of the stage takes the low nibbles of
// dwords {0,1}, {2,3}, then the high nibbles of {0,1}, {2,3} as the lane's
// 8 B-operand values; the A operand (X) of lane (m = l % 16, p) supplies the
// 8 matching x values, chunk 8(p/2) + 4(t/2) + 2(p&1) + (t&1) of the stage's
// 16 chunks of row m.  The accumulators of lane l hold D[m][n] for
// n = l % 16 and m = 4 (l / 16) + r, r = 0..3 (D = X . W^T, 16 x 16).
//
// Split K works as in gemm.hip (the 64 x 64 tile schedule and workspace are
// the same): each K range writes its partial tile, the last to arrive adds
// them in range order, writes Y and resets the tile's counter.
#include <type_traits>

#include "q4k_device.h"
#include "tile_sched.h"

namespace jq4k {

typedef __attribute__((ext_vector_type(4))) float float4_t;

constexpr int kSkThreads = 256;   // four waves
constexpr int kSkBN = 64;         // rows of W per workgroup: 16 per wave
constexpr int kSkDepth = 4;       // stages of W in flight per wave
constexpr int kSkChunks = 16;     // 16-byte chunks of X per row per stage
// word 3 of a raw buffer resource (see gemm.hip)
constexpr int kSkBufferConfig = 0x00020000;

// LDS slot of chunk j of X row r in a stage buffer: rows of 16 chunks, the
// chunk index XOR-ed with the row so that 16 rows read at one chunk hit 16
// different 16-byte slots of the 256-byte bank window.
__device__ __forceinline__ int sk_slot(int row, int j) { return row * kSkChunks + (j ^ (row & 15)); }

template <int MT>
__global__ __launch_bounds__(kSkThreads) void q4k_gemm_skinny_kernel(const GemmBatch batch,
                                                                     uint32_t qmask) {
    constexpr int kRows = 16 * MT;   // rows of X staged (M padded)
    __shared__ uint4 xs[2][kRows * kSkChunks];
    int q, tm, tn, split;
    if (!tile_sched_next(batch.s, blockIdx.x, &q, &tm, &tn, &split)) return;
    const GemmProblem& pr = batch.p[q];
    const int M = pr.M, N = pr.N, K = pr.K;
    const int nb = K / kQK;
    const int S = batch.s.splits[q];
    const int kb0 = split * nb / S, kb1 = (split + 1) * nb / S;
    const int nstage = 2 * (kb1 - kb0);   // half blocks
    const int hb0 = 2 * kb0;

    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int li = lane & 15, p = lane >> 4;
    const int n0 = tn * kSkBN;

    // ---- W: row n0 + 16 wave + li (clamped: rows past N feed outputs that
    // are never stored)
    const int wn = min(n0 + 16 * wave + li, N - 1);
    const uint8_t* wrow = pr.W + static_cast<long>(wn) * nb * kBlockBytes;
    // Stage st is half hb = hb0 + st of block hb / 2; hb0 is even and the
    // pipeline below is unrolled by kSkDepth (even), so the half of ring
    // entry u is u & 1.  The block header travels with the even (first-half)
    // entries; the even stage decodes the scales of both halves and keeps
    // the second half's in `hold` for the odd stage after it.
    struct WRegs {
        uint4 hdr;   // even entries only
        uint4 qs;
    };
    static_assert(kSkDepth % 2 == 0, "the ring alternates block halves");
    WRegs ring[kSkDepth];
    QuarterScales hold;
    auto load_w = [&](int st, WRegs& r, bool first_half) {
        // past the end: a harmless repeat of the last block
        const int hb = min(hb0 + st, hb0 + nstage - 2 + (first_half ? 0 : 1));
        const uint8_t* blk = wrow + static_cast<long>(hb >> 1) * kBlockBytes;
        if (first_half) r.hdr = load16(blk);
        r.qs = load16(blk + 16 + 64 * (hb & 1) + 16 * p);
    };

    // ---- X: rows 0 .. kRows-1 of the M rows, chunk g = t + 256 j -> row
    // g / 16, chunk g % 16; rows past M read as zeros
    const __amdgpu_buffer_rsrc_t xres = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(pr.X), 0, static_cast<int>(static_cast<long>(M) * K * 2),
        kSkBufferConfig);
    // X of the next kSkDepth stages waits in registers, as far ahead as W:
    // the hardware counts loads back in issue order, so a wait for an X load
    // issued after some W load also waits for that W load.
    uint4 xring[kSkDepth][MT];
    auto load_x = [&](int st, uint4 (&xr)[MT]) {
        const int hb = hb0 + min(st, nstage - 1);
#pragma unroll
        for (int j = 0; j < MT; ++j) {
            const int g = t + j * kSkThreads;
            const int row = g >> 4, ch = g & 15;
            const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(
                xres, (row * K + hb * 128 + ch * 8) * 2, 0, 0);
            xr[j] = make_uint4(v.x, v.y, v.z, v.w);
        }
    };
    auto store_x = [&](const uint4 (&xr)[MT], uint4* buf) {
#pragma unroll
        for (int j = 0; j < MT; ++j) {
            const int g = t + j * kSkThreads;
            buf[sk_slot(g >> 4, g & 15)] = xr[j];
        }
    };

    float4_t acc[MT];
#pragma unroll
    for (int i = 0; i < MT; ++i) acc[i] = float4_t{0.f, 0.f, 0.f, 0.f};

    // One stage of the wave: dequantise the 32 weights of the lane into four
    // B operands and multiply them with the A operands of every M tile.
    auto compute = [&](const QuarterScales& sc, const uint4& qs, const uint4* buf) {
        const WRegs r{uint4{}, qs};
        uint32_t lo[4][2], hi[4][2];
        dequant_dword_bf16(r.qs.x, sc, lo[0], hi[0], qmask);
        dequant_dword_bf16(r.qs.y, sc, lo[1], hi[1], qmask);
        dequant_dword_bf16(r.qs.z, sc, lo[2], hi[2], qmask);
        dequant_dword_bf16(r.qs.w, sc, lo[3], hi[3], qmask);
        const uint4 bq[4] = {make_uint4(lo[0][0], lo[0][1], lo[1][0], lo[1][1]),
                             make_uint4(lo[2][0], lo[2][1], lo[3][0], lo[3][1]),
                             make_uint4(hi[0][0], hi[0][1], hi[1][0], hi[1][1]),
                             make_uint4(hi[2][0], hi[2][1], hi[3][0], hi[3][1])};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const int ch = 8 * (p >> 1) + 4 * (ks >> 1) + 2 * (p & 1) + (ks & 1);
            const bf16x8_t b = __builtin_bit_cast(bf16x8_t, bq[ks]);
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                const bf16x8_t a =
                    __builtin_bit_cast(bf16x8_t, buf[sk_slot(16 * mt + li, ch)]);
                acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[mt], 0, 0, 0);
            }
        }
    };

    // ---- pipeline.  Stage st's X and W are requested kSkDepth iterations
    // ahead (X first), X of stage st is stored to LDS buffer st & 1 in the
    // iteration before it is used, and each iteration ends with one barrier:
    //   iteration st: compute stage st (W from ring st % D, X from LDS);
    //                 store X of stage st + 1 to the other buffer;
    //                 request X of stage st + 1 + D, then W of stage st + D.
    // Indices past the end are clamped (harmless repeats).
#pragma unroll
    for (int u = 0; u < kSkDepth; ++u) {
        load_x(u, xring[u]);
        load_w(u, ring[u], (u & 1) == 0);
    }
    store_x(xring[0], xs[0]);
    load_x(kSkDepth, xring[0]);
    __syncthreads();

    // One pipeline step; `u` (compile-time) is st % kSkDepth, with the parity
    // of st.
    auto step = [&](int st, auto u_c) {
        constexpr int u = decltype(u_c)::value;
        constexpr int un = (u + 1) % kSkDepth;
        if constexpr ((u & 1) == 0) {
            // quarter 2h + p/2 of the lane, h = 0 now and h = 1 next stage
            const QuarterScales sc = quarter_scales(ring[u].hdr, static_cast<uint32_t>(p >> 1));
            hold = quarter_scales(ring[u].hdr, static_cast<uint32_t>(2 + (p >> 1)));
            compute(sc, ring[u].qs, xs[0]);
        } else {
            compute(hold, ring[u].qs, xs[1]);
        }
        store_x(xring[un], xs[(u + 1) & 1]);
        load_x(st + 1 + kSkDepth, xring[un]);
        load_w(st + kSkDepth, ring[u], (u & 1) == 0);
        __syncthreads();
    };
    // Whole groups of kSkDepth stages run without branches (so that the
    // waits for each stage's loads stay exact), then the last few stages.
    const int nfull = nstage - nstage % kSkDepth;
    for (int s = 0; s < nfull; s += kSkDepth) {
        step(s + 0, std::integral_constant<int, 0>{});
        step(s + 1, std::integral_constant<int, 1>{});
        step(s + 2, std::integral_constant<int, 2>{});
        step(s + 3, std::integral_constant<int, 3>{});
    }
    if (nfull + 0 < nstage) step(nfull + 0, std::integral_constant<int, 0>{});
    if (nfull + 1 < nstage) step(nfull + 1, std::integral_constant<int, 1>{});
    if (nfull + 2 < nstage) step(nfull + 2, std::integral_constant<int, 2>{});
    static_assert(kSkDepth == 4, "the unrolled steps above");

    // ---- split K: publish the partial; the last K range adds them all
    if (S > 1) {
        float4_t* mine = reinterpret_cast<float4_t*>(pr.part) +
                         (static_cast<long>(tm * batch.s.tn[q] + tn) * S + split) * 64 * 16;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) mine[mt * kSkThreads + t] = acc[mt];
        // the partials of the workgroup, then the counter (agent scope)
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
        __syncthreads();
        int* last = reinterpret_cast<int*>(&xs[0][0]);
        int* cnt = pr.cnt + tm * batch.s.tn[q] + tn;
        if (t == 0) {
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
            const int prev = __hip_atomic_fetch_add(cnt, 1, __ATOMIC_RELAXED,
                                                    __HIP_MEMORY_SCOPE_AGENT);
            const bool is_last = prev == S - 1;
            if (is_last) {
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
                *cnt = 0;   // ready for the next call
            }
            *last = is_last;
        }
        __syncthreads();
        if (!*last) return;
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
        // every partial from the workspace, this range's own included (the
        // thread reads back what it wrote): the sum does not depend on which
        // range arrived last
        const float4_t* base = mine - static_cast<long>(split) * 64 * 16;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            float4_t total = base[mt * kSkThreads + t];
            for (int u = 1; u < S; ++u)
                total += base[static_cast<long>(u) * 64 * 16 + mt * kSkThreads + t];
            acc[mt] = total;
        }
    }

    // ---- Y: lane holds D[m][n], n = n0 + 16 wave + li, m = 16 mt + 4 p + r
    const int n = n0 + 16 * wave + li;
    if (n < N) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int m = 16 * mt + 4 * p + r;
                if (m < M) pr.Y[static_cast<long>(m) * N + n] = acc[mt][r];
            }
    }
}

// Problems with M <= 64 in 64 x 64 tiles (the same schedule, split plan and
// workspace as the 64-row MFMA tile), 16 MT rows of X per workgroup with MT
// from the largest M.  splits null: whole K.
hipError_t launch_gemm_skinny(const uint8_t* const* W, const uint16_t* const* X,
                              float* const* Y, const int* M, const int* N, const int* K,
                              int count, const int* splits, void* ws, hipStream_t stream) {
    GemmBatch b;
    const long grid = gemm_batch_init(b, W, X, Y, M, N, K, count, 64, kSkBN, splits, ws);
    int max_m = 1;
    for (int i = 0; i < count; ++i) max_m = M[i] > max_m ? M[i] : max_m;
    const dim3 g(static_cast<unsigned>(grid)), blk(kSkThreads);
    switch ((max_m + 15) / 16) {
        case 1: hipLaunchKernelGGL(q4k_gemm_skinny_kernel<1>, g, blk, 0, stream, b, kNibbleMask); break;
        case 2: hipLaunchKernelGGL(q4k_gemm_skinny_kernel<2>, g, blk, 0, stream, b, kNibbleMask); break;
        case 3: hipLaunchKernelGGL(q4k_gemm_skinny_kernel<3>, g, blk, 0, stream, b, kNibbleMask); break;
        default: hipLaunchKernelGGL(q4k_gemm_skinny_kernel<4>, g, blk, 0, stream, b, kNibbleMask); break;
    }
    return hipGetLastError();
}

}  // namespace jq4k
