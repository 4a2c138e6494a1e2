// gemm_big.hip -- Q4_K matmul for large M on the gfx950 matrix cores, with
// 256 x 256 output tiles.
//
// Y (M x N) = X (M x K) . W^T with W in Q4_K (genie-ai-runtime README, "At a
// glance": "tensor-core MMQ Q4_K prefill").  A workgroup of four waves (one
// per SIMD, up to 512 registers each) computes a 256 x 256 tile of Y; wave
// (wm, wn) owns rows 128 wm.. of X and rows 128 wn.. of W, i.e. 128 x 128
// outputs in 4 x 4 v_mfma_f32_32x32x16_bf16 accumulators (256 fp32 per lane,
// in the accumulation registers).
//
// Why this shape.  Per 64 weights of K a 256 x 128 tile moves 40 KB from L2
// into the CU (32 KB of it X) and writes 48 KB of LDS; measured on the chip,
// a CU takes about 50 bytes per clock from L2 and writes about 70 bytes per
// clock into LDS, so those two streams -- not the matrix cores -- set the
// pace of a 256 x 128 tile.  The 256 x 256 tile moves 44 KB and writes 64 KB
// of LDS for twice the multiply-adds, and its 128 x 128 wave tiles read
// 32 KB of LDS per 64 of K instead of 48 KB for two 128 x 64 ones.
//
// Every wave does every job: it fetches its share of the next-but-one stage
// of X (bf16) and W (header + quant bytes) into registers, writes the next
// stage to LDS (W dequantised to bf16: fma(d*sc, q, -dmin*m), the exact value
// rounded once, then RNE to bf16), and multiplies the current one.  LDS holds
// two stages; one barrier per stage (64 of K).
//
// Measured: on one Qwen3-4B layer at M = 2048 in one grouped launch it runs
// as fast as the 256-row wave-specialised kernel (gemm_ws.hip), and slower
// on a single projection, whose 256-wide tiles leave CUs idle.  Its loop
// without loads and dequantisation keeps the matrix cores about 70% busy;
// the vector work a wave places between its own matrix instructions does
// not overlap with them well enough yet.  Reached through JQ4K_PATH_MFMA_BIG.
#include "q4k_device.h"
#include "tile_sched.h"

namespace jq4k {

namespace {

constexpr int kBgThreads = 256;
constexpr int kBgBM = 256, kBgBN = 256, kBgBK = 64;
constexpr int kBgRowChunks = kBgBK / 8;                    // 16-byte chunks per row per stage
constexpr int kBgXChunks = kBgBM * kBgRowChunks / kBgThreads;   // X chunks per thread per stage
constexpr int kBgTM = 4, kBgTN = 4;                        // 32 x 32 tiles per wave
constexpr int kBgBufferConfig = 0x00020000;                // raw buffer resource word 3

// Chunk c of row r of a slab at r * 8 + (c ^ f(r)): the 32 rows a fragment
// read touches at one chunk land on distinct 16-byte bank groups.
__device__ __forceinline__ int bg_chunk(int row, int chunk) {
    return row * kBgRowChunks + (chunk ^ (((row >> 1) ^ ((row & 1) << 2)) & 7));
}

struct BgRegs {
    uint4 x[kBgXChunks];
    uint4 hdr, qa, qb;   // W row: header, quant bytes 0..15 and 16..31 of the quarter
};

}  // namespace

__global__ __launch_bounds__(kBgThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void q4k_gemm_big_kernel(const GemmBatch batch, uint32_t qmask) {
    // stage buffers: X slab (256 rows) then W slab (256 rows), 64 KB each
    __shared__ uint4 lds[2][(kBgBM + kBgBN) * kBgRowChunks];

    const int t = threadIdx.x;
    const int wave = t >> 6, lane = t & 63;

    int q, tm, tn, split;
    if (!tile_sched_next(batch.s, blockIdx.x, &q, &tm, &tn, &split)) return;
    const GemmProblem& pr = batch.p[q];
    const uint16_t* __restrict__ X = pr.X;
    float* __restrict__ Y = pr.Y;
    const int M = pr.M, N = pr.N, K = pr.K;
    const int n0 = tn * kBgBN, m0 = tm * kBgBM;
    const int nb = K / kQK;
    const int nstage = K / kBgBK;   // a multiple of 4
    auto last = [&](int s) { return min(s, nstage - 1); };

    // ---- the thread's share of the loads: X chunks g = t + 256 j (row g / 8,
    // chunk g % 8), and W row t of the tile (rows past N repeat row N - 1:
    // they feed outputs that are never stored)
    const long xrows = min(static_cast<long>(kBgBM), static_cast<long>(M - m0));
    const __amdgpu_buffer_rsrc_t xres = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(X + static_cast<long>(m0) * K), 0,
        static_cast<int>(xrows * K * 2), kBgBufferConfig);
    int xoff[kBgXChunks];
    int xlds[kBgXChunks];
#pragma unroll
    for (int j = 0; j < kBgXChunks; ++j) {
        const int g = t + j * kBgThreads;
        xoff[j] = ((g >> 3) * K + (g & 7) * 8) * 2;
        xlds[j] = bg_chunk(g >> 3, g & 7);
    }
    const uint8_t* wrow = pr.W + static_cast<long>(min(n0 + t, N - 1)) * nb * kBlockBytes;
    const int wbase = kBgBM * kBgRowChunks;

    // W first, then X, in this order (a scheduling barrier between): each
    // stage's waits then cover exactly its own loads.
    auto load_stage = [&](int s, BgRegs& r) {
        const uint8_t* blk = wrow + (s >> 2) * kBlockBytes;
        r.hdr = load16(blk);
        r.qa = load16(blk + 16 + 32 * (s & 3));
        r.qb = load16(blk + 32 + 32 * (s & 3));
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int j = 0; j < kBgXChunks; ++j) {
            const u32x4_t v =
                __builtin_amdgcn_raw_buffer_load_b128(xres, xoff[j] + s * kBgBK * 2, 0, 0);
            r.x[j] = make_uint4(v.x, v.y, v.z, v.w);
        }
    };
    // Stage s of the slab: X as loaded; W row t as 64 bf16 weights, chunk j
    // = weights 8 j .. 8 j + 7 of the quarter (low nibbles of quant bytes
    // 0..31 are weights 0..31, high nibbles weights 32..63).
    auto store_x = [&](const BgRegs& r, uint4* buf) {
#pragma unroll
        for (int j = 0; j < kBgXChunks; ++j) buf[xlds[j]] = r.x[j];
    };
    auto store_w = [&](int s, const BgRegs& r, uint4* buf) {
        const QuarterScales sc = quarter_scales(r.hdr, static_cast<uint32_t>(s & 3));
        const uint32_t qw[8] = {r.qa.x, r.qa.y, r.qa.z, r.qa.w, r.qb.x, r.qb.y, r.qb.z, r.qb.w};
#pragma unroll
        for (int h = 0; h < 4; ++h) {
            uint32_t lo_a[2], hi_a[2], lo_b[2], hi_b[2];
            dequant_dword_bf16(qw[2 * h], sc, lo_a, hi_a, qmask);
            dequant_dword_bf16(qw[2 * h + 1], sc, lo_b, hi_b, qmask);
            buf[wbase + bg_chunk(t, h)] = make_uint4(lo_a[0], lo_a[1], lo_b[0], lo_b[1]);
            buf[wbase + bg_chunk(t, 4 + h)] = make_uint4(hi_a[0], hi_a[1], hi_b[0], hi_b[1]);
        }
    };

    // ---- the wave's 128 x 128 outputs
    const int wm = wave >> 1, wn = wave & 1;
    const int arow = wm * 128 + (lane & 31);
    const int bcol = wn * 128 + (lane & 31);
    const int khalf = lane >> 5;
    float16_t acc[kBgTM][kBgTN];
#pragma unroll
    for (int i = 0; i < kBgTM; ++i)
#pragma unroll
        for (int j = 0; j < kBgTN; ++j) acc[i][j] = float16_t{};
    auto read_frags = [&](const uint4* buf, int ks, bf16x8_t* a, bf16x8_t* b) {
        const int ch = 2 * ks + khalf;
#pragma unroll
        for (int i = 0; i < kBgTM; ++i)
            a[i] = __builtin_bit_cast(bf16x8_t, buf[bg_chunk(arow + 32 * i, ch)]);
#pragma unroll
        for (int j = 0; j < kBgTN; ++j)
            b[j] = __builtin_bit_cast(bf16x8_t, buf[wbase + bg_chunk(bcol + 32 * j, ch)]);
    };
    auto mma = [&](const bf16x8_t* a, const bf16x8_t* b) {
#pragma unroll
        for (int i = 0; i < kBgTM; ++i)
#pragma unroll
            for (int j = 0; j < kBgTN; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0,
                                                                     0);
    };
    auto fence = [] { __builtin_amdgcn_sched_barrier(0); };

    // One stage: multiply stage s (buffer cur, fragments of its k-step 0 in
    // f0) while stage s + 1 goes from registers r to buffer nxt and r is
    // refilled with stage s + 3.  The last k-step's matrix instructions are
    // issued after the barrier, behind the reads of the next stage's first
    // fragments.  The scheduling barriers keep this order.
    bf16x8_t a0[kBgTM], b0[kBgTN], a1[kBgTM], b1[kBgTN];
    // The stage's work is written out in issue order, one matrix instruction
    // at a time with the other work of the stage placed between them, and
    // scheduling barriers keep that order: a matrix instruction runs for 32
    // cycles after it issues, and the vector and memory instructions that
    // follow it in the same wave issue meanwhile.
    auto m1 = [&](int idx, const bf16x8_t* a, const bf16x8_t* b) {
        const int i = idx >> 2, j = idx & 3;
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
    };
    auto stage = [&](int s, const uint4* cur, uint4* nxt, BgRegs& r) {
        read_frags(cur, 1, a1, b1);
        fence();
        // k-step 0, with X of stage s + 1 to LDS
#pragma unroll
        for (int idx = 0; idx < 16; ++idx) {
            m1(idx, a0, b0);
            fence();
            if (idx < kBgXChunks) nxt[xlds[idx]] = r.x[idx];
            fence();
        }
        read_frags(cur, 2, a0, b0);
        fence();
        // k-step 1, with W of stage s + 1 dequantised to LDS: per dword pair
        // h, four matrix instructions
        const QuarterScales sc = quarter_scales(r.hdr, static_cast<uint32_t>((s + 1) & 3));
        const uint32_t qw[8] = {r.qa.x, r.qa.y, r.qa.z, r.qa.w, r.qb.x, r.qb.y, r.qb.z, r.qb.w};
#pragma unroll
        for (int h = 0; h < 4; ++h) {
            uint32_t lo_a[2], hi_a[2], lo_b[2], hi_b[2];
            m1(4 * h, a1, b1);
            fence();
            dequant_dword_bf16(qw[2 * h], sc, lo_a, hi_a, qmask);
            fence();
            m1(4 * h + 1, a1, b1);
            fence();
            dequant_dword_bf16(qw[2 * h + 1], sc, lo_b, hi_b, qmask);
            fence();
            m1(4 * h + 2, a1, b1);
            fence();
            nxt[wbase + bg_chunk(t, h)] = make_uint4(lo_a[0], lo_a[1], lo_b[0], lo_b[1]);
            fence();
            m1(4 * h + 3, a1, b1);
            fence();
            nxt[wbase + bg_chunk(t, 4 + h)] = make_uint4(hi_a[0], hi_a[1], hi_b[0], hi_b[1]);
            fence();
        }
        // k-step 2, with the loads of stage s + 3 and the k-step 3 reads
        const int s3 = last(s + 3);
        const uint8_t* blk = wrow + (s3 >> 2) * kBlockBytes;
        m1(0, a0, b0);
        fence();
        r.hdr = load16(blk);
        fence();
        m1(1, a0, b0);
        fence();
        r.qa = load16(blk + 16 + 32 * (s3 & 3));
        fence();
        m1(2, a0, b0);
        fence();
        r.qb = load16(blk + 32 + 32 * (s3 & 3));
        fence();
#pragma unroll
        for (int idx = 3; idx < 16; ++idx) {
            m1(idx, a0, b0);
            fence();
            if (idx - 3 < kBgXChunks) {
                const int jx = idx - 3;
                const u32x4_t v =
                    __builtin_amdgcn_raw_buffer_load_b128(xres, xoff[jx] + s3 * kBgBK * 2, 0, 0);
                r.x[jx] = make_uint4(v.x, v.y, v.z, v.w);
            } else if (idx == 11) {
                read_frags(cur, 3, a1, b1);
            }
            fence();
        }
        __syncthreads();
        read_frags(nxt, 0, a0, b0);
        fence();
        mma(a1, b1);
        fence();
    };

    BgRegs rs[2];
    load_stage(0, rs[0]);
    load_stage(last(1), rs[1]);
    store_x(rs[0], lds[0]);
    store_w(0, rs[0], lds[0]);
    load_stage(last(2), rs[0]);
    __syncthreads();
    read_frags(lds[0], 0, a0, b0);
    for (int s = 0; s < nstage; s += 2) {
        stage(s, lds[0], lds[1], rs[1]);
        stage(s + 1, lds[1], lds[0], rs[0]);
    }

#pragma unroll
    for (int i = 0; i < kBgTM; ++i) {
#pragma unroll
        for (int j = 0; j < kBgTN; ++j) {
            const int n = n0 + wn * 128 + 32 * j + (lane & 31);
            if (n >= N) continue;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int m = m0 + wm * 128 + 32 * i + 8 * (r >> 2) + 4 * khalf + (r & 3);
                if (m < M) Y[static_cast<long>(m) * N + n] = acc[i][j][r];
            }
        }
    }
}

hipError_t launch_gemm_big(const uint8_t* const* W, const uint16_t* const* X, float* const* Y,
                           const int* M, const int* N, const int* K, int count,
                           hipStream_t stream) {
    GemmBatch b;
    const long grid = gemm_batch_init(b, W, X, Y, M, N, K, count, kBgBM, kBgBN);
    hipLaunchKernelGGL(q4k_gemm_big_kernel, dim3(static_cast<unsigned>(grid)), dim3(kBgThreads),
                       0, stream, b, kNibbleMask);
    return hipGetLastError();
}

}  // namespace jq4k
