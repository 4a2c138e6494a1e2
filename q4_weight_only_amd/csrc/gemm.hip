// gemm.hip -- Q4_K matmul on the gfx950 matrix cores, for M > 1 (prefill).
//
// Y (M x N) = X (M x K) . W^T with W in Q4_K (genie-ai-runtime README, "At a
// glance": "tensor-core MMQ Q4_K prefill").  Each workgroup computes a BM x BN
// tile of Y.  The K loop advances one quarter block (64 weights = sub-blocks
// 2c, 2c+1 of block kb) per stage:
//   * the BN x 64 slab of W is fetched as header + 32 quant bytes per row,
//     dequantised in registers to fp32 (fma(d*sc, q, -dmin*m), the exact
//     value rounded once), rounded to bf16 (RNE) and written to LDS;
//   * the BM x 64 slab of X (bf16) is copied to LDS;
//   * four waves multiply the slabs with v_mfma_f32_32x32x16_bf16 into fp32
//     accumulators.
// LDS is double-buffered and the loop is software-pipelined: while stage s
// is on the matrix cores, stage s+1 is dequantised into the other buffer and
// the global loads of stages s+2 and s+3 are in flight; one barrier per stage.
// LDS rows are 128 bytes (8 chunks of 16 bytes), XOR-swizzled by row (see
// lds_chunk) so the operand reads hit distinct banks.
//
// Operand layouts (v_mfma_f32_32x32x16_bf16): lane l supplies row l % 32 of
// A and column l % 32 of B, k = 8 (l / 32) .. +7 of the 16-wide k step; the
// 16 accumulators of lane l hold column l % 32, rows 8 (r / 4) + 4 (l / 32)
// + r % 4 for r = 0..15.
#include "q4k_device.h"
#include "tile_sched.h"

namespace jq4k {

constexpr int kGemmThreads = 256;
constexpr int kBK = 64;               // K per stage: one quarter block
constexpr int kRowChunks = kBK / 8;   // 16-byte chunks per LDS row
// Word 3 of a raw buffer resource on gfx9-family GPUs (32-bit data format,
// no swizzle): byte-addressed loads with a range check against num_records.
constexpr int kBufferConfig = 0x00020000;

// Chunk c of tile row r sits at chunk c ^ f(r), f(r) = (r >> 1) ^ 4 (r & 1).
// An MFMA operand read has 16 lanes on 16 consecutive rows and one chunk;
// f gives them 16 different 16-byte slots in every 256-byte window (and 8
// different slots in every 128-byte window for each run of 8 lanes), so
// reads and the row-wise tile writes are free of bank conflicts.
__device__ __forceinline__ int lds_chunk(int row, int chunk) {
    return row * kRowChunks + (chunk ^ (((row >> 1) ^ ((row & 1) << 2)) & 7));
}

template <int BM, int BN, int WM, int WN>
struct GemmCfg {
    static_assert(WM * WN == 4, "four waves");
    static constexpr int kWaveM = BM / WM, kWaveN = BN / WN;
    static_assert(kWaveM % 32 == 0 && kWaveN % 32 == 0, "32x32 MFMA tiles");
    static constexpr int kTM = kWaveM / 32, kTN = kWaveN / 32;
    static constexpr int kXChunks = BM * kRowChunks / kGemmThreads;  // per thread
    static_assert(kXChunks >= 1 && BM * kRowChunks % kGemmThreads == 0, "X slab split");
    static constexpr int kThreadsPerRow = kGemmThreads / BN;          // W slab split
    static_assert(kThreadsPerRow == 1 || kThreadsPerRow == 2 || kThreadsPerRow == 4, "BN");
    static constexpr int kQBytes = 32 / kThreadsPerRow;               // quant bytes / thread
    static constexpr int kLdsChunks = (BM + BN) * kRowChunks;         // per buffer
    // register sets of global data in flight: deeper for the 64-row tile,
    // whose loop is load-latency-bound at small M
    static constexpr int kSets = BM == 64 ? 4 : 2;
};

// One BM x BN tile of Y = X . W^T, rows m0.. and columns n0.. (the whole
// K loop and the epilogue), computed by the 256 threads of a workgroup.
//
// kPair (SwiGLU of a gate/up pair, H = silu(X.Wg^T) * (X.Wu^T)): the tile's
// BN rows of W are BN/2 rows of W (gate) and the same BN/2 rows of W2 (up),
// interleaved in runs of 32 so that k-tile 2j of every wave holds gate
// columns and k-tile 2j+1 the matching up columns: tile row wr is row
// n0 + 32 (wr / 64) + wr % 32 of W if (wr / 32) is even, of W2 if odd, and
// the tile writes BN/2 columns of H from column n0 (each wave 64 wide).
template <int BM, int BN, int WM, int WN, bool kPair>
__device__ __forceinline__ void gemm_tile(const uint8_t* __restrict__ W,
                                          const uint8_t* __restrict__ W2,
                                          const uint16_t* __restrict__ X, float* __restrict__ Y,
                                          int M, int N, int K, int n0, int m0, uint32_t qmask,
                                          uint4 (*lds)[GemmCfg<BM, BN, WM, WN>::kLdsChunks]) {
    using C = GemmCfg<BM, BN, WM, WN>;
    static_assert(!kPair || C::kWaveN == 64, "pairs need 64-wide wave tiles");
    const int t = threadIdx.x;
    const int lane = t & 63, wave = t >> 6;
    const int wm = wave / WN, wn = wave % WN;
    const int nb = K / kQK;
    const int nstage = K / kBK;

    // ---- W slab assignment: row wr of the tile, quant bytes [qoff, qoff + kQBytes)
    const int wr = t / C::kThreadsPerRow;
    const int qoff = (t % C::kThreadsPerRow) * C::kQBytes;
    // rows past N are clamped to row N-1: they only feed output columns that
    // are never stored
    const int wn_row = kPair ? n0 + 32 * (wr >> 6) + (wr & 31) : n0 + wr;
    const uint8_t* wsrc = kPair && ((wr >> 5) & 1) ? W2 : W;
    const uint8_t* wrow = wsrc + static_cast<long>(min(wn_row, N - 1)) * nb * kBlockBytes;

    // ---- X slab assignment: chunk g = t + 256 j -> row g / 8, chunk g % 8.
    // X is read through a buffer resource over rows m0 .. m0 + BM - 1 (only
    // those below M): the hardware returns zeros past the end, and buffer
    // loads are kept in registers until their LDS store instead of being
    // re-issued there by the compiler.
    const long xrows = min(static_cast<long>(BM), static_cast<long>(M - m0));
    const __amdgpu_buffer_rsrc_t xres = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(X + static_cast<long>(m0) * K), 0,
        static_cast<int>(xrows * K * 2), kBufferConfig);

    // Global data of one stage, held in registers until it is stored to LDS.
    struct StageRegs {
        uint4 x[C::kXChunks];
        uint4 hdr;
        uint32_t q[C::kQBytes / 4];
    };
    StageRegs rs[C::kSets];

    auto load_stage = [&](int s, StageRegs& r) {
        const int kb = s >> 2, c = s & 3;
#pragma unroll
        for (int j = 0; j < C::kXChunks; ++j) {
            const int g = t + j * kGemmThreads;
            const int row = g >> 3, ch = g & 7;
            const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(
                xres, (row * K + s * kBK + ch * 8) * 2, 0, 0);
            r.x[j] = make_uint4(v.x, v.y, v.z, v.w);
        }
        const uint8_t* blk = wrow + kb * kBlockBytes;
        r.hdr = *reinterpret_cast<const uint4*>(blk);
        const uint8_t* q = blk + 16 + 32 * c + qoff;
        if constexpr (C::kQBytes == 32) {
            const uint4 a = *reinterpret_cast<const uint4*>(q);
            const uint4 b = *reinterpret_cast<const uint4*>(q + 16);
            r.q[0] = a.x; r.q[1] = a.y; r.q[2] = a.z; r.q[3] = a.w;
            r.q[4] = b.x; r.q[5] = b.y; r.q[6] = b.z; r.q[7] = b.w;
        } else if constexpr (C::kQBytes == 16) {
            const uint4 a = *reinterpret_cast<const uint4*>(q);
            r.q[0] = a.x; r.q[1] = a.y; r.q[2] = a.z; r.q[3] = a.w;
        } else {
            const uint2 a = *reinterpret_cast<const uint2*>(q);
            r.q[0] = a.x; r.q[1] = a.y;
        }
    };

    auto store_stage = [&](int s, const StageRegs& r, uint4* buf) {
        const int c = s & 3;
#pragma unroll
        for (int j = 0; j < C::kXChunks; ++j) {
            const int g = t + j * kGemmThreads;
            buf[lds_chunk(g >> 3, g & 7)] = r.x[j];
        }
        uint4* wbuf = buf + BM * kRowChunks;
        const QuarterScales sc = quarter_scales(r.hdr, static_cast<uint32_t>(c));
        // 8 quant bytes -> one 16-byte chunk of the even sub-block (k offset
        // qoff + 0..7) and one of the odd sub-block (k offset 32 + qoff + 0..7)
#pragma unroll
        for (int j = 0; j < C::kQBytes / 8; ++j) {
            uint32_t lo_a[2], hi_a[2], lo_b[2], hi_b[2];
            dequant_dword_bf16(r.q[2 * j], sc, lo_a, hi_a, qmask);
            dequant_dword_bf16(r.q[2 * j + 1], sc, lo_b, hi_b, qmask);
            const int ch = (qoff >> 3) + j;
            wbuf[lds_chunk(wr, ch)] = make_uint4(lo_a[0], lo_a[1], lo_b[0], lo_b[1]);
            wbuf[lds_chunk(wr, 4 + ch)] = make_uint4(hi_a[0], hi_a[1], hi_b[0], hi_b[1]);
        }
    };

    float16_t acc[C::kTM][C::kTN];
#pragma unroll
    for (int i = 0; i < C::kTM; ++i)
#pragma unroll
        for (int j = 0; j < C::kTN; ++j) acc[i][j] = float16_t{};

    const int arow = wm * C::kWaveM + (lane & 31);  // A row within the tile (+32 i)
    const int bcol = wn * C::kWaveN + (lane & 31);  // B column within the tile (+32 j)
    const int khalf = lane >> 5;

    // Software pipeline, one barrier per stage.  While the matrix cores work
    // on stage s from LDS buffer s & 1, the same instruction stream
    // dequantises stage s + 1 (from register set (s + 1) % S) into the other
    // buffer and requests stage s + 1 + S into the register set it just
    // freed, so global data has S stages of work to arrive (S = kSets).
    // Stage indices past the end are clamped (harmless repeats), keeping the
    // body one basic block.  Within a stage the operand fragments of k-step
    // ks + 1 are read from LDS while the MFMAs of k-step ks run.
    auto read_frags = [&](const uint4* buf, int ks, bf16x8_t* a, bf16x8_t* b) {
        const uint4* xb = buf;
        const uint4* wb = buf + BM * kRowChunks;
        const int ch = 2 * ks + khalf;
#pragma unroll
        for (int i = 0; i < C::kTM; ++i)
            a[i] = __builtin_bit_cast(bf16x8_t, xb[lds_chunk(arow + 32 * i, ch)]);
#pragma unroll
        for (int j = 0; j < C::kTN; ++j)
            b[j] = __builtin_bit_cast(bf16x8_t, wb[lds_chunk(bcol + 32 * j, ch)]);
    };
    auto mfma_stage = [&](const uint4* buf) {
        bf16x8_t a[2][C::kTM], b[2][C::kTN];
        read_frags(buf, 0, a[0], b[0]);
#pragma unroll
        for (int ks = 0; ks < kBK / 16; ++ks) {
            if (ks + 1 < kBK / 16) read_frags(buf, ks + 1, a[(ks + 1) & 1], b[(ks + 1) & 1]);
#pragma unroll
            for (int i = 0; i < C::kTM; ++i)
#pragma unroll
                for (int j = 0; j < C::kTN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                        a[ks & 1][i], b[ks & 1][j], acc[i][j], 0, 0, 0);
        }
    };
    auto last = [&](int s) { return min(s, nstage - 1); };

#pragma unroll
    for (int j = 0; j < C::kSets; ++j) load_stage(last(j), rs[j]);
    store_stage(0, rs[0], lds[0]);
    load_stage(last(C::kSets), rs[0]);
    __syncthreads();
    // nstage = K / 64 is a multiple of 4, hence of kSets
    for (int s = 0; s < nstage; s += C::kSets) {
#pragma unroll
        for (int u = 0; u < C::kSets; ++u) {
            mfma_stage(lds[u & 1]);
            store_stage(last(s + u + 1), rs[(u + 1) % C::kSets], lds[(u + 1) & 1]);
            load_stage(last(s + u + 1 + C::kSets), rs[(u + 1) % C::kSets]);
            __syncthreads();
        }
    }

    // ---- epilogue: fp32 Y, row-major
    if constexpr (kPair) {
        // k-tiles (2j, 2j + 1) are the gate and up columns of the same rows
#pragma unroll
        for (int i = 0; i < C::kTM; ++i) {
#pragma unroll
            for (int j = 0; j < C::kTN; j += 2) {   // kTN == 2: one pair
                const int n = n0 + wn * 32 + (lane & 31);
                if (n >= N) continue;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int m =
                        m0 + wm * C::kWaveM + 32 * i + 8 * (r >> 2) + 4 * khalf + (r & 3);
                    if (m < M) Y[static_cast<long>(m) * N + n] = silu(acc[i][j][r]) * acc[i][j + 1][r];
                }
            }
        }
        return;
    }
#pragma unroll
    for (int i = 0; i < C::kTM; ++i) {
#pragma unroll
        for (int j = 0; j < C::kTN; ++j) {
            const int n = n0 + wn * C::kWaveN + 32 * j + (lane & 31);
            if (n >= N) continue;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int m = m0 + wm * C::kWaveM + 32 * i + 8 * (r >> 2) + 4 * khalf + (r & 3);
                if (m < M) Y[static_cast<long>(m) * N + n] = acc[i][j][r];
            }
        }
    }
}

template <int BM, int BN, int WM, int WN, bool kPair>
__global__ __launch_bounds__(kGemmThreads) void q4k_gemm_mfma_kernel(const GemmBatch batch,
                                                                     uint32_t qmask) {
    using C = GemmCfg<BM, BN, WM, WN>;
    __shared__ uint4 lds[2][C::kLdsChunks];
    constexpr int kOutN = kPair ? BN / 2 : BN;   // output columns per tile
    int q, tm, tn, split;   // split: always 0 (these launches take whole K)
    if (!tile_sched_next(batch.s, blockIdx.x, &q, &tm, &tn, &split)) return;
    const GemmProblem& pr = batch.p[q];
    gemm_tile<BM, BN, WM, WN, kPair>(pr.W, pr.W2, pr.X, pr.Y, pr.M, pr.N, pr.K, tn * kOutN,
                                     tm * BM, qmask, lds);
}

template <int BM, int BN, int WM, int WN>
static hipError_t launch_cfg(const uint8_t* const* W, const uint16_t* const* X, float* const* Y,
                             const int* M, const int* N, const int* K, int count,
                             hipStream_t stream) {
    GemmBatch b;
    const long grid = gemm_batch_init(b, W, X, Y, M, N, K, count, BM, BN);
    hipLaunchKernelGGL((q4k_gemm_mfma_kernel<BM, BN, WM, WN, false>),
                       dim3(static_cast<unsigned>(grid)), dim3(kGemmThreads), 0, stream, b,
                       kNibbleMask);
    return hipGetLastError();
}

template <int BM, int BN, int WM, int WN>
static hipError_t launch_pair_cfg(const uint8_t* Wg, const uint8_t* Wu, const uint16_t* X,
                                  float* H, int M, int N, int K, hipStream_t stream) {
    GemmBatch b;
    const long grid = gemm_batch_init(b, &Wg, &X, &H, &M, &N, &K, 1, BM, BN / 2);
    b.p[0].W2 = Wu;
    hipLaunchKernelGGL((q4k_gemm_mfma_kernel<BM, BN, WM, WN, true>),
                       dim3(static_cast<unsigned>(grid)), dim3(kGemmThreads), 0, stream, b,
                       kNibbleMask);
    return hipGetLastError();
}

hipError_t launch_gemm_ws(const uint8_t* const* W, const uint16_t* const* X, float* const* Y,
                          const int* M, const int* N, const int* K, int count,
                          hipStream_t stream);
hipError_t launch_gemm_big(const uint8_t* const* W, const uint16_t* const* X, float* const* Y,
                           const int* M, const int* N, const int* K, int count,
                           hipStream_t stream);
constexpr int kTileBig = 512;   // tile code of the 256 x 256 kernel (gemm_big.hip)
hipError_t launch_gemm_rw(const uint8_t* const* W, const uint16_t* const* X, float* const* Y,
                          const int* M, const int* N, const int* K, int count,
                          hipStream_t stream);
constexpr int kTileRw = 1024;   // tile code of the register-W 256 x 256 kernel (gemm_rw.hip)

hipError_t launch_gemm_ws_pair(const uint8_t* Wg, const uint8_t* Wu, const uint16_t* X, float* H,
                               int M, int N, int K, hipStream_t stream);

// SwiGLU of a gate/up pair, H = silu(X.Wg^T) * (X.Wu^T): 64 x 128 tiles (64
// outputs) at M <= 64, 128 x 128 below M = 2048, else the 256-row kernel.
hipError_t launch_gemm_swiglu(const uint8_t* Wg, const uint8_t* Wu, const uint16_t* X, float* H,
                              int M, int N, int K, hipStream_t stream) {
    if (M <= 64) return launch_pair_cfg<64, 128, 2, 2>(Wg, Wu, X, H, M, N, K, stream);
    if (M < 2048) return launch_pair_cfg<128, 128, 2, 2>(Wg, Wu, X, H, M, N, K, stream);
    return launch_gemm_ws_pair(Wg, Wu, X, H, M, N, K, stream);
}

// Workgroups a SwiGLU launch takes (the largest of its tile choices).
long gemm_swiglu_launch_size(int M, int N) {
    TileSched s;
    return tile_sched_init(s, &M, &N, nullptr, 1, 64, 64, 1);
}

// Workgroups a launch of these problems takes (tiles, times the K ranges
// when splits is given, plus idle workgroups at the ends of XCD shares).
long gemm_launch_size(const int* M, const int* N, int count, int tile,
                      const int* splits) {
    const int bm = tile == kTileBig || tile == kTileRw ? 256 : tile;
    const int bn = tile == 64 ? 64 : tile == kTileBig || tile == kTileRw ? 256 : 128;
    TileSched s;
    return tile_sched_init(s, M, N, splits, count, bm, bn, 1);
}

// Split K for the 64 x 64 tiles (M <= 64, the small-M kernel): the K ranges
// of every problem and the workspace they take (see splitk_plan).
long gemm_splitk_plan(const int* M, const int* N, const int* K, int count, long min_items,
                      int* splits) {
    splitk_plan(M, N, K, count, 64, 64, min_items, splits);
    return splitk_workspace_bytes(M, N, splits, count, 64, 64);
}

// tile: 64, 128 or 256 rows of M per workgroup, or one of the 256 x 256
// codes, for the whole batch.  The 64-row tile is 64 columns wide: at
// M <= 64 the matmul streams W like a GEMV, and narrow tiles give it four
// times the workgroups of 256-wide ones (1.9x faster on a Qwen3-4B layer at
// M = 33).  256 is the wave-specialised 256 x 128 kernel of gemm_ws.hip;
// kTileRw the register-W kernel of gemm_rw.hip; kTileBig the single-role
// kernel of gemm_big.hip (by explicit path only).
hipError_t launch_gemm_mfma(const uint8_t* const* W, const uint16_t* const* X, float* const* Y,
                            const int* M, const int* N, const int* K, int count, int tile,
                            hipStream_t stream) {
    if (tile == 64) return launch_cfg<64, 64, 2, 2>(W, X, Y, M, N, K, count, stream);
    if (tile == 256) return launch_gemm_ws(W, X, Y, M, N, K, count, stream);
    if (tile == kTileBig) return launch_gemm_big(W, X, Y, M, N, K, count, stream);
    if (tile == kTileRw) return launch_gemm_rw(W, X, Y, M, N, K, count, stream);
    return launch_cfg<128, 128, 2, 2>(W, X, Y, M, N, K, count, stream);
}

}  // namespace jq4k
