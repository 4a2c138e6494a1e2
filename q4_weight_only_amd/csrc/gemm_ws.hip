// gemm_ws.hip -- wave-specialised Q4_K matmul on the gfx950 matrix cores.
//
// Y (M x N) = X (M x K) . W^T with W in Q4_K (genie-ai-runtime README, "At a
// glance": "tensor-core MMQ Q4_K prefill"), for large M.  A workgroup of
// eight waves computes a 256 x 128 tile of Y.  The dequantisation of W is
// vector-ALU work of about two instructions per weight, done once per tile;
// instead of interleaving it with the matrix instructions in one stream, the
// workgroup splits the roles by wave:
//   * waves 0..3 (consumers) read operand fragments from LDS and issue
//     v_mfma_f32_32x32x16_bf16 into fp32 accumulators (each owns 128 x 64);
//   * waves 4..7 (producers) fetch W (header + quant bytes), dequantise it to
//     bf16 (fma(d*sc, q, -dmin*m) rounded once, then rounded to bf16) and
//     write the W slab to LDS;
//   * both roles copy the next stage of X (bf16, no conversion) from global
//     memory to LDS, rows 0..127 the consumers, rows 128..255 the producers.
// The hardware places one consumer and one producer wave on each SIMD, so the
// vector ALU and the matrix core run side by side.  The K loop advances one
// quarter block (64 weights) per stage; LDS holds two stages and one barrier
// per stage hands filled buffers on.  X is fetched one stage ahead (mostly L2
// hits: every column tile re-reads it), W four stages ahead (from HBM).
// Spreading the LDS writes over all eight waves matters: measured on the
// chip, four waves write LDS at about 40 bytes per clock per CU, eight at
// about 70, and a stage writes 48 KB.
#include "q4k_device.h"
#include "tile_sched.h"

namespace jq4k {

namespace {

constexpr int kWsThreads = 512;
constexpr int kWsBM = 256, kWsBN = 128, kWsBK = 64;
constexpr int kWsRowChunks = kWsBK / 8;
constexpr int kWsLdsChunks = (kWsBM + kWsBN) * kWsRowChunks;   // per buffer
constexpr int kWsXChunks = kWsBM * kWsRowChunks / 256;          // X chunks of a stage per 256 threads
constexpr int kWsTM = 4, kWsTN = 2;                             // 32x32 tiles per consumer
constexpr int kWsBufferConfig = 0x00020000;   // raw buffer resource word 3 (gfx9 family)

// Same swizzle as the single-role kernel: chunk c of row r at c ^ f(r).
__device__ __forceinline__ int ws_chunk(int row, int chunk) {
    return row * kWsRowChunks + (chunk ^ (((row >> 1) ^ ((row & 1) << 2)) & 7));
}

// A producer thread's global data for one stage, X and W in separate
// register rings: X (mostly L2 hits) is fetched two stages ahead, W (a
// stream from HBM, with the longer latency) kWsWDepth stages ahead.
constexpr int kWsWDepth = 4;

// X chunks a thread copies per stage: each role copies half of the slab.
constexpr int kWsXHalf = kWsXChunks / 2;

struct WsXRegs {
    uint4 x[kWsXHalf];
};

struct WsWRegs {
    uint4 hdr;
    uint4 q;  // 16 quant bytes: half of the row's quarter
};

}  // namespace

// kPair: SwiGLU of a gate/up pair, with the tile layout of gemm_tile's
// kPair (gemm.hip): tile row wr is row n0 + 32 (wr / 64) + wr % 32 of the
// gate (W) or the up matrix (W2) as (wr / 32) is even or odd; each consumer
// wave's two 32-column k-tiles are then the gate and up columns of the same
// 32 outputs, and the tile writes 64 columns of H = silu(gate) * up.
template <bool kPair>
__global__ __launch_bounds__(kWsThreads) void q4k_gemm_ws_kernel(const GemmBatch batch,
                                                                 uint32_t qmask) {
    __shared__ uint4 lds[2][kWsLdsChunks];

    const int t = threadIdx.x;
    const int wave = t >> 6, lane = t & 63;

    int q, tm, tn;
    int split;   // always 0: this kernel takes whole K
    if (!tile_sched_next(batch.s, blockIdx.x, &q, &tm, &tn, &split)) return;
    const GemmProblem& pr = batch.p[q];
    const uint8_t* __restrict__ W = pr.W;
    const uint16_t* __restrict__ X = pr.X;
    float* __restrict__ Y = pr.Y;
    const int M = pr.M, N = pr.N, K = pr.K;
    const int n0 = tn * (kPair ? kWsBN / 2 : kWsBN), m0 = tm * kWsBM;
    const int nb = K / kQK;
    const int nstage = K / kWsBK;  // a multiple of 4
    auto last = [&](int s) { return min(s, nstage - 1); };

    // X through a buffer resource over rows m0 .. m0 + BM - 1 below M
    // (zeros past the end; the loads stay in registers until stored).  The
    // consumer waves fetch and store X: chunk g = t + 256 j of a stage is
    // row g / 8, chunk g % 8.
    const long xrows = min(static_cast<long>(kWsBM), static_cast<long>(M - m0));
    const __amdgpu_buffer_rsrc_t xres = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(X + static_cast<long>(m0) * K), 0,
        static_cast<int>(xrows * K * 2), kWsBufferConfig);
    // chunk j of the thread's half: consumers take rows 0..127, producers
    // rows 128..255 of the slab
    const int xj0 = wave >= 4 ? kWsXHalf : 0;
    auto x_off = [&](int j) {
        const int g = (t & 255) + (xj0 + j) * 256;
        return ((g >> 3) * K + (g & 7) * 8) * 2;
    };
    auto x_lds = [&](int j) {
        const int g = (t & 255) + (xj0 + j) * 256;
        return ws_chunk(g >> 3, g & 7);
    };
    auto load_x = [&](int s, WsXRegs& r) {
#pragma unroll
        for (int j = 0; j < kWsXHalf; ++j) {
            const u32x4_t v =
                __builtin_amdgcn_raw_buffer_load_b128(xres, x_off(j) + s * kWsBK * 2, 0, 0);
            r.x[j] = make_uint4(v.x, v.y, v.z, v.w);
        }
    };
    auto store_x = [&](const WsXRegs& r, uint4* buf) {
#pragma unroll
        for (int j = 0; j < kWsXHalf; ++j) buf[x_lds(j)] = r.x[j];
    };

    // The two roles run separate loops (their registers never need to be
    // live together); both loops pass the same 1 + nstage barriers.
    if (wave >= 4) {
        // ---------------- producers: fetch, dequantise, fill LDS
        const int pt = t - 256;                        // 0..255
        const int wr = pt >> 1, qoff = (pt & 1) * 16;  // W row of the tile, quant byte offset
        // Rows past N (or M) are clamped to the last row: they only feed
        // outputs that are never stored.
        const int wn_row = kPair ? n0 + 32 * (wr >> 6) + (wr & 31) : n0 + wr;
        const uint8_t* wsrc = kPair && ((wr >> 5) & 1) ? pr.W2 : W;
        const uint8_t* wrow = wsrc + static_cast<long>(min(wn_row, N - 1)) * nb * kBlockBytes;
        const int wlds_lo0 = kWsBM * kWsRowChunks + ws_chunk(wr, (qoff >> 3));
        const int wlds_lo1 = kWsBM * kWsRowChunks + ws_chunk(wr, (qoff >> 3) + 1);
        const int wlds_hi0 = kWsBM * kWsRowChunks + ws_chunk(wr, 4 + (qoff >> 3));
        const int wlds_hi1 = kWsBM * kWsRowChunks + ws_chunk(wr, 5 + (qoff >> 3));
        WsWRegs wq[kWsWDepth];
        auto load_w = [&](int s, WsWRegs& r) {
            const uint8_t* blk = wrow + (s >> 2) * kBlockBytes;
            r.hdr = *reinterpret_cast<const uint4*>(blk);
            r.q = *reinterpret_cast<const uint4*>(blk + 16 + 32 * (s & 3) + qoff);
        };
        auto store_w = [&](int s, const WsWRegs& r, uint4* buf) {
            const QuarterScales sc = quarter_scales(r.hdr, static_cast<uint32_t>(s & 3));
            uint32_t lo_a[2], hi_a[2], lo_b[2], hi_b[2];
            dequant_dword_bf16(r.q.x, sc, lo_a, hi_a, qmask);
            dequant_dword_bf16(r.q.y, sc, lo_b, hi_b, qmask);
            buf[wlds_lo0] = make_uint4(lo_a[0], lo_a[1], lo_b[0], lo_b[1]);
            buf[wlds_hi0] = make_uint4(hi_a[0], hi_a[1], hi_b[0], hi_b[1]);
            dequant_dword_bf16(r.q.z, sc, lo_a, hi_a, qmask);
            dequant_dword_bf16(r.q.w, sc, lo_b, hi_b, qmask);
            buf[wlds_lo1] = make_uint4(lo_a[0], lo_a[1], lo_b[0], lo_b[1]);
            buf[wlds_hi1] = make_uint4(hi_a[0], hi_a[1], hi_b[0], hi_b[1]);
        };
        // Stage j's W is stored (buffer j & 1) one turn before the consumers
        // use it, four turns after it was fetched; W slot j % 4 holds stage j.
        // nstage is a multiple of 4, so the loop body is four turns with
        // constant slot indices.
        static_assert(kWsWDepth == 4, "the loop below is unrolled for a ring of four");
        // Scheduling barriers close every turn: without them the compiler
        // moves a turn's global loads (whose registers are read turns
        // later) down to the end of the loop body, and the next iteration
        // then waits for them at once.
        auto turn_end = [] {
            __builtin_amdgcn_sched_barrier(0);
            __syncthreads();
            __builtin_amdgcn_sched_barrier(0);
        };
        // The producers' half of X goes one stage ahead, like the consumers'.
        WsXRegs xp;
        load_x(0, xp);
#pragma unroll
        for (int u = 0; u < kWsWDepth; ++u) load_w(last(u), wq[u]);
        store_w(0, wq[0], lds[0]);
        store_x(xp, lds[0]);
        load_x(last(1), xp);
        load_w(last(4), wq[0]);
        turn_end();
        for (int s = 0; s < nstage; s += 4) {
            store_w(last(s + 1), wq[1], lds[1]);
            store_x(xp, lds[1]);
            load_x(last(s + 2), xp);
            load_w(last(s + 5), wq[1]);
            turn_end();
            store_w(last(s + 2), wq[2], lds[0]);
            store_x(xp, lds[0]);
            load_x(last(s + 3), xp);
            load_w(last(s + 6), wq[2]);
            turn_end();
            store_w(last(s + 3), wq[3], lds[1]);
            store_x(xp, lds[1]);
            load_x(last(s + 4), xp);
            load_w(last(s + 7), wq[3]);
            turn_end();
            store_w(last(s + 4), wq[0], lds[0]);
            store_x(xp, lds[0]);
            load_x(last(s + 5), xp);
            load_w(last(s + 8), wq[0]);
            turn_end();
        }
        return;
    }

    // ---------------- consumers: LDS fragments -> MFMA -> fp32 Y
    const int wm = wave >> 1, wn = wave & 1;
    const int arow = wm * 128 + (lane & 31);
    const int bcol = wn * 64 + (lane & 31);
    const int khalf = lane >> 5;
    float16_t acc[kWsTM][kWsTN];
#pragma unroll
    for (int i = 0; i < kWsTM; ++i)
#pragma unroll
        for (int j = 0; j < kWsTN; ++j) acc[i][j] = float16_t{};
    auto read_frags = [&](const uint4* buf, int ks, bf16x8_t* a, bf16x8_t* b) {
        const uint4* wb = buf + kWsBM * kWsRowChunks;
        const int ch = 2 * ks + khalf;
#pragma unroll
        for (int i = 0; i < kWsTM; ++i)
            a[i] = __builtin_bit_cast(bf16x8_t, buf[ws_chunk(arow + 32 * i, ch)]);
#pragma unroll
        for (int j = 0; j < kWsTN; ++j)
            b[j] = __builtin_bit_cast(bf16x8_t, wb[ws_chunk(bcol + 32 * j, ch)]);
    };
    auto mma = [&](const bf16x8_t* a, const bf16x8_t* b) {
#pragma unroll
        for (int i = 0; i < kWsTM; ++i)
#pragma unroll
            for (int j = 0; j < kWsTN; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0,
                                                                     0);
    };
    // Four k-steps of 16 per stage; the fragments of step ks + 1 are read
    // while step ks multiplies (two named fragment sets).  The last step of
    // a stage is issued after the barrier, behind the reads of the next
    // stage's first fragments, so the matrix cores stay busy while the LDS
    // latency of the new stage passes.
    // The scheduling barriers keep that order: without them the compiler
    // sinks each fragment read to just before its first use and waits for
    // it there, which exposes the LDS latency every two matrix instructions.
    bf16x8_t a0[kWsTM], b0[kWsTN], a1[kWsTM], b1[kWsTN];
    auto fence = [] { __builtin_amdgcn_sched_barrier(0); };
    // The consumers also move their half of X: during stage s they store X
    // of stage s + 1 (fetched one stage earlier) into the next buffer and
    // fetch X of stage s + 2 into the same registers.
    WsXRegs xr;
    auto half = [&](int s, const uint4* cur, uint4* nxt, WsXRegs& xq) {
        mma(a0, b0);
        fence();
        read_frags(cur, 2, a0, b0);
        fence();
        store_x(xq, nxt);
        fence();
        load_x(last(s + 2), xq);
        fence();
        mma(a1, b1);
        fence();
        read_frags(cur, 3, a1, b1);
        fence();
        mma(a0, b0);
        fence();
        __syncthreads();
        read_frags(nxt, 0, a0, b0);
        fence();
        mma(a1, b1);
        fence();
        read_frags(nxt, 1, a1, b1);
        fence();
    };
    load_x(0, xr);
    store_x(xr, lds[0]);
    load_x(last(1), xr);
    __syncthreads();
    read_frags(lds[0], 0, a0, b0);
    read_frags(lds[0], 1, a1, b1);
    for (int s = 0; s < nstage; s += 2) {
        half(s, lds[0], lds[1], xr);
        half(s + 1, lds[1], lds[0], xr);
    }
    if constexpr (kPair) {
        static_assert(kWsTN == 2, "one gate/up pair of k-tiles per consumer wave");
        const int n = n0 + wn * 32 + (lane & 31);
        if (n >= N) return;
#pragma unroll
        for (int i = 0; i < kWsTM; ++i) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int m = m0 + wm * 128 + 32 * i + 8 * (r >> 2) + 4 * khalf + (r & 3);
                if (m < M) Y[static_cast<long>(m) * N + n] = silu(acc[i][0][r]) * acc[i][1][r];
            }
        }
        return;
    }
#pragma unroll
    for (int i = 0; i < kWsTM; ++i) {
#pragma unroll
        for (int j = 0; j < kWsTN; ++j) {
            const int n = n0 + wn * 64 + 32 * j + (lane & 31);
            if (n >= N) continue;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int m = m0 + wm * 128 + 32 * i + 8 * (r >> 2) + 4 * khalf + (r & 3);
                if (m < M) Y[static_cast<long>(m) * N + n] = acc[i][j][r];
            }
        }
    }
}

hipError_t launch_gemm_ws(const uint8_t* const* W, const uint16_t* const* X, float* const* Y,
                          const int* M, const int* N, const int* K, int count,
                          hipStream_t stream) {
    GemmBatch b;
    const long grid = gemm_batch_init(b, W, X, Y, M, N, K, count, kWsBM, kWsBN);
    hipLaunchKernelGGL(q4k_gemm_ws_kernel<false>, dim3(static_cast<unsigned>(grid)),
                       dim3(kWsThreads), 0, stream, b, kNibbleMask);
    return hipGetLastError();
}

hipError_t launch_gemm_ws_pair(const uint8_t* Wg, const uint8_t* Wu, const uint16_t* X, float* H,
                               int M, int N, int K, hipStream_t stream) {
    GemmBatch b;
    const long grid = gemm_batch_init(b, &Wg, &X, &H, &M, &N, &K, 1, kWsBM, kWsBN / 2);
    b.p[0].W2 = Wu;
    hipLaunchKernelGGL(q4k_gemm_ws_kernel<true>, dim3(static_cast<unsigned>(grid)),
                       dim3(kWsThreads), 0, stream, b, kNibbleMask);
    return hipGetLastError();
}

}  // namespace jq4k
