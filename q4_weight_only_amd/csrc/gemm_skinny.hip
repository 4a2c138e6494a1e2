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
//   * X (bf16, its M rows) goes through LDS two blocks (512 of K) at a time,
//     shared by the four waves; the next two blocks wait in registers while
//     the current ones are used, so there are two barriers per two blocks;
//   * W has kSkDepth half blocks in flight per wave.
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
// 8 matching x values, chunk 8(p/2) + 4(t/2) + 2(p&1) + (t&1) of the half
// block's 16 chunks of row m.  The accumulators of lane l hold D[m][n] for
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
constexpr int kSkDepth = 8;       // stages (half blocks) of W in flight per wave
constexpr int kSkSuper = 4;       // stages per X staging step (two blocks)
constexpr int kSkRowChunks = 16 * kSkSuper;   // 16-byte chunks of X per row per step
// LDS row stride in chunks: one chunk of padding, so that 16 rows read at
// one chunk (row stride 1040 bytes = 260 banks, 4 mod 64) hit 16 different
// 16-byte slots of the 64 banks, and a lane's reads differ only by
// compile-time offsets
constexpr int kSkRowStride = kSkRowChunks + 1;
// word 3 of a raw buffer resource (see gemm.hip)
constexpr int kSkBufferConfig = 0x00020000;

// LDS bytes of the X buffer for batches whose largest M is max_m.
size_t gemm_skinny_lds_bytes(int max_m) {
    return static_cast<size_t>(max_m) * kSkRowStride * 16;
}

template <int MT>
__global__ __launch_bounds__(kSkThreads) void q4k_gemm_skinny_kernel(const GemmBatch batch,
                                                                     uint32_t qmask) {
    extern __shared__ uint4 xs[];   // M rows x kSkRowStride chunks
    int q, tm, tn, split;
    if (!tile_sched_next(batch.s, blockIdx.x, &q, &tm, &tn, &split)) return;
    const GemmProblem& pr = batch.p[q];
    const int M = pr.M, N = pr.N, K = pr.K;
    const int nb = K / kQK;
    const int S = batch.s.splits[q];
    const int kb0 = split * nb / S, kb1 = (split + 1) * nb / S;
    const int nstage = 2 * (kb1 - kb0);   // half blocks (even)
    const int hb0 = 2 * kb0;

    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int li = lane & 15, p = lane >> 4;
    const int n0 = tn * kSkBN;

    // ---- W: row n0 + 16 wave + li (clamped: rows past N feed outputs that
    // are never stored).  Stage st is half hb = hb0 + st of block hb / 2;
    // hb0 is even and the steps below are unrolled by kSkDepth (even), so the
    // half of ring entry u is u & 1, and ring entry u holds the stages st
    // with st % kSkDepth == u.  The block header travels with the even
    // (first-half) entries; the even stage decodes the scales of both halves
    // and keeps the second half's in `hold` for the odd stage after it.
    const int wn = min(n0 + 16 * wave + li, N - 1);
    const uint8_t* wrow = pr.W + static_cast<long>(wn) * nb * kBlockBytes;
    struct WRegs {
        uint4 hdr;   // even entries only
        uint4 qs;
    };
    static_assert(kSkDepth % 2 == 0 && kSkDepth == 2 * kSkSuper, "two X steps per ring");
    WRegs ring[kSkDepth];
    QuarterScales hold;
    auto load_w = [&](int st, WRegs& r, bool first_half) {
        // past the end: a harmless repeat of the last block
        const int hb = min(hb0 + st, hb0 + nstage - 2 + (first_half ? 0 : 1));
        const uint8_t* blk = wrow + static_cast<long>(hb >> 1) * kBlockBytes;
        if (first_half) r.hdr = load16(blk);
        r.qs = load16(blk + 16 + 64 * (hb & 1) + 16 * p);
    };

    // ---- X: the M rows, kSkSuper stages at a time.  Chunk g = t + 256 j of
    // a step is row g / 64 = 4 j + wave, chunk g % 64 = lane.  The loads of
    // step j + 1 are requested at the start of step j and stored to LDS at
    // its end, so their latency is covered by the step's four stages.
    const __amdgpu_buffer_rsrc_t xres = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(pr.X), 0, static_cast<int>(static_cast<long>(M) * K * 2),
        kSkBufferConfig);
    constexpr int kXLoads = 4 * MT;   // covers rows < 16 MT
    const int nsuper = (nstage + kSkSuper - 1) / kSkSuper;
    uint4 xr[kXLoads];
    const int wave_s = __builtin_amdgcn_readfirstlane(wave);   // wave-uniform
    auto load_x = [&](int j) {
        const int hbs = hb0 + kSkSuper * min(j, nsuper - 1);
        const int hb = min(hbs + (lane >> 4), hb0 + nstage - 1);
#pragma unroll
        for (int i = 0; i < kXLoads; ++i) {
            const int row = min(4 * i + wave_s, M - 1);
            const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(
                xres, (row * K + hb * 128 + (lane & 15) * 8) * 2, 0, 0);
            xr[i] = make_uint4(v.x, v.y, v.z, v.w);
        }
    };
    // rows 4 i + wave past M are row M - 1 again: the same values to the
    // same place (no branch, so the waits for W loads stay exact)
    auto store_x = [&]() {
#pragma unroll
        for (int i = 0; i < kXLoads; ++i)
            xs[min(4 * i + wave_s, M - 1) * kSkRowStride + lane] = xr[i];
    };

    float4_t acc[MT];
#pragma unroll
    for (int i = 0; i < MT; ++i) acc[i] = float4_t{0.f, 0.f, 0.f, 0.f};
    // A operand rows of the lane, one per M tile (rows past M read row M - 1:
    // their outputs are never stored), from chunk 8 (p / 2) + 2 (p & 1)
    const uint4* xa[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
        xa[mt] = xs + min(16 * mt + li, M - 1) * kSkRowStride + 8 * (p >> 1) + 2 * (p & 1);

    // One stage of the wave: dequantise the 32 weights of the lane into four
    // B operands and multiply them with the A operands of every M tile.
    auto compute = [&](const QuarterScales& sc, const uint4& qs, int hb_in_step) {
        uint32_t lo[4][2], hi[4][2];
        dequant_dword_bf16(qs.x, sc, lo[0], hi[0], qmask);
        dequant_dword_bf16(qs.y, sc, lo[1], hi[1], qmask);
        dequant_dword_bf16(qs.z, sc, lo[2], hi[2], qmask);
        dequant_dword_bf16(qs.w, sc, lo[3], hi[3], qmask);
        const uint4 bq[4] = {make_uint4(lo[0][0], lo[0][1], lo[1][0], lo[1][1]),
                             make_uint4(lo[2][0], lo[2][1], lo[3][0], lo[3][1]),
                             make_uint4(hi[0][0], hi[0][1], hi[1][0], hi[1][1]),
                             make_uint4(hi[2][0], hi[2][1], hi[3][0], hi[3][1])};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const int c = 16 * hb_in_step + 4 * (ks >> 1) + (ks & 1);   // + the lane's part
            const bf16x8_t b = __builtin_bit_cast(bf16x8_t, bq[ks]);
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                const bf16x8_t a = __builtin_bit_cast(bf16x8_t, xa[mt][c]);
                acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[mt], 0, 0, 0);
            }
        }
    };

    // One stage: `u` (compile-time) is the stage's W ring entry (with the
    // parity of the stage); u % kSkSuper is its place in its X step.
    auto step = [&](int st, auto u_c) {
        constexpr int u = decltype(u_c)::value;
        if constexpr ((u & 1) == 0) {
            // quarter 2h + p/2 of the lane, h = 0 now and h = 1 next stage
            const QuarterScales sc = quarter_scales(ring[u].hdr, static_cast<uint32_t>(p >> 1));
            hold = quarter_scales(ring[u].hdr, static_cast<uint32_t>(2 + (p >> 1)));
            compute(sc, ring[u].qs, u % kSkSuper);
        } else {
            compute(hold, ring[u].qs, u % kSkSuper);
        }
        __builtin_amdgcn_sched_barrier(0);
        load_w(st + kSkDepth, ring[u], (u & 1) == 0);
        __builtin_amdgcn_sched_barrier(0);
    };
    // the four stages of one X step, ring entries u0 .. u0 + 3
    auto xstep = [&](int s0, auto u0_c) {
        constexpr int u0 = decltype(u0_c)::value;
        step(s0 + 0, std::integral_constant<int, u0 + 0>{});
        step(s0 + 1, std::integral_constant<int, u0 + 1>{});
        step(s0 + 2, std::integral_constant<int, u0 + 2>{});
        step(s0 + 3, std::integral_constant<int, u0 + 3>{});
    };
    using U0 = std::integral_constant<int, 0>;
    using U1 = std::integral_constant<int, 1>;
    using U4 = std::integral_constant<int, 4>;
    using U5 = std::integral_constant<int, 5>;

    // ---- pipeline: X of step 0 in LDS, W of stages 0 .. kSkDepth-1 in
    // flight.  Scheduling barriers keep every load where it is written: the
    // compiler otherwise moves the loads (whose registers are read stages
    // later) to the end of the loop body, next to their first use, and
    // waits for them there.  Step j: request X of step j + 1 (past the end: a harmless
    // repeat), run its kSkSuper stages (each requesting W kSkDepth stages
    // ahead), then barrier, X of step j + 1 to LDS, barrier.  nstage is even,
    // so a last partial step has exactly two stages.
    load_x(0);
#pragma unroll
    for (int u = 0; u < kSkDepth; ++u) load_w(u, ring[u], (u & 1) == 0);
    store_x();
    __syncthreads();
    const int nfull = nstage / kSkSuper;
    // two X steps per iteration: the ring's kSkDepth stages
    auto full_step = [&](int j, auto u0_c) {
        load_x(j + 1);
        __builtin_amdgcn_sched_barrier(0);
        xstep(kSkSuper * j, u0_c);
        __syncthreads();
        store_x();
        __syncthreads();
    };
    int j = 0;
    for (; j + 1 < nfull; j += 2) {
        full_step(j, U0{});
        full_step(j + 1, U4{});
    }
    if (j < nfull) full_step(j++, U0{});
    if (nstage % kSkSuper != 0) {
        // stages 4 nfull and 4 nfull + 1: ring entries 0, 1 or 4, 5
        if ((nfull & 1) == 0) {
            step(nstage - 2, U0{});
            step(nstage - 1, U1{});
        } else {
            step(nstage - 2, U4{});
            step(nstage - 1, U5{});
        }
    }
    static_assert(kSkSuper == 4 && kSkDepth == 8, "the unrolled steps above");

    // ---- split K: publish the partial; the last K range adds them all
    if (S > 1) {
        float4_t* mine = reinterpret_cast<float4_t*>(pr.part) +
                         (static_cast<long>(tm * batch.s.tn[q] + tn) * S + split) * 64 * 16;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) mine[mt * kSkThreads + t] = acc[mt];
        // the partials of the workgroup, then the counter (agent scope)
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
        __syncthreads();
        int* last = reinterpret_cast<int*>(&xs[0]);
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

    // ---- Y: lane holds D[m][n], n = n0 + 16 wave + li, m = 16 mt + 4 p + r.
    // Streaming (nontemporal) stores: Y is not read again here, and the
    // agent-scope release of a split tile writes back the XCD's dirty L2
    // lines (1% faster on the Qwen3-4B layer at M = 33; the partial tiles,
    // which the last range reads back, measured slower that way).
    const int n = n0 + 16 * wave + li;
    if (n < N) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int m = 16 * mt + 4 * p + r;
                if (m < M)
                    __builtin_nontemporal_store(acc[mt][r], &pr.Y[static_cast<long>(m) * N + n]);
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
    const size_t lds = gemm_skinny_lds_bytes(max_m);
    switch ((max_m + 15) / 16) {
        case 1: hipLaunchKernelGGL(q4k_gemm_skinny_kernel<1>, g, blk, lds, stream, b, kNibbleMask); break;
        case 2: hipLaunchKernelGGL(q4k_gemm_skinny_kernel<2>, g, blk, lds, stream, b, kNibbleMask); break;
        case 3: hipLaunchKernelGGL(q4k_gemm_skinny_kernel<3>, g, blk, lds, stream, b, kNibbleMask); break;
        default: hipLaunchKernelGGL(q4k_gemm_skinny_kernel<4>, g, blk, lds, stream, b, kNibbleMask); break;
    }
    return hipGetLastError();
}

}  // namespace jq4k
