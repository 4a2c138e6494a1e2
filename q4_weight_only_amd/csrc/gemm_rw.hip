// gemm_rw.hip -- Q4_K matmul for large M on the gfx950 matrix cores, with W
// dequantised straight into the matrix instructions' operand registers.
//
// Y (M x N) = X (M x K) . W^T with W in Q4_K (genie-ai-runtime README, "At a
// glance": "tensor-core MMQ Q4_K prefill").  A workgroup of four waves (one
// per SIMD, up to 512 registers each) computes a 256 x 256 tile of Y: every
// wave the same 256 rows of X against its own 64 rows of W, i.e. 256 x 64
// outputs in 8 x 2 v_mfma_f32_32x32x16_bf16 accumulators (256 fp32 per
// lane, in the accumulation registers).
//
// Why this shape.  The kernels that stage dequantised W in LDS spend their
// time on LDS (a 256 x 128 tile writes 48 KB and reads 96 KB of LDS per 64 of
// K against 1024 matrix-core cycles; the chip writes LDS at ~70 and reads at
// ~139 bytes per clock per CU).  Here W never enters LDS: each lane loads the
// Q4_K bytes of its own columns and dequantises them (fma(d*sc, q, -dmin*m),
// the exact value rounded once, then RNE to bf16 -- dequant_dword_bf16) into
// B operands.  Only X goes through LDS: 32 KB written and 128 KB read per 64
// of K, against 2048 matrix-core cycles per wave (~1400 cycles of LDS at
// those rates).  The dequantisation costs about 2.1 vector instructions per
// weight, 64 weights per lane per 64 of K (each dequantised weight feeds 256
// rows of X: a wave of 128 x 128 outputs would need twice the vector work
// per matrix instruction, which one wave per SIMD cannot hide), and is
// placed between the matrix instructions of the previous half stage.
//
// Operand order.  The instruction sums its 16 k in any order, so a stage
// (64 of K, one quarter of a block: sub-blocks 2c and 2c+1) maps k to
// (k-step kk, lane half kh, item e) to fit the code bytes: lane (n, kh)
// loads quant bytes 16 kh .. 16 kh + 15 of its column's quarter, whose low
// nibbles are weights 16 kh + 0..15 and high nibbles 32 + 16 kh + 0..15 of
// the quarter.  k-step kk takes the low nibbles of dwords {0,1} (kk = 0) or
// {2,3} (kk = 1), the high nibbles of {0,1} (kk = 2) or {2,3} (kk = 3), i.e.
// quarter positions 32 (kk / 2) + 16 kh + 8 (kk % 2) + e.  X is stored in LDS
// in that order: chunk 2 kk + kh of a row (16 bytes) holds source chunk
// 4 (kk / 2) + 2 kh + kk % 2 of the row's 64 values, so an A operand is one
// 16-byte read.
//
// Pipeline (per stage s, k-steps in the order 0, 2, 1, 3; X of stage s in
// LDS buffer s % 4):
//   k-steps 0, 2   B of k-steps 1 and 3 of stage s dequantised; A of
//                  k-steps 2 and 1 read
//   barrier        X of stage s + 1 has landed, and every wave is done
//                  with the buffer of stage s - 1
//   k-steps 1, 3   B of k-steps 0 and 2 of stage s + 1 dequantised; A of
//                  k-step 3 and of k-step 0 of stage s + 1 read; X of stage
//                  s + 3 copied into the buffer of stage s - 1 (global to
//                  LDS, no registers); on a block's first stage, the whole
//                  next block of W requested first
// so no operand read waits on the barrier: they are all issued half a stage
// or more before their matrix instructions.
// Vector work sits between the matrix instructions (scheduling groups):
// the wave issues in order and a matrix instruction occupies the matrix
// core for 32 cycles, so only interleaved vector work runs under it.
#include <type_traits>

#include "q4k_device.h"
#include "tile_sched.h"

namespace jq4k {

namespace {

constexpr int kRwThreads = 256;
constexpr int kRwBM = 256, kRwBN = 256, kRwBK = 64;
constexpr int kRwRowChunks = kRwBK / 8;                          // 16-byte chunks per row per stage
constexpr int kRwXChunks = kRwBM * kRwRowChunks / kRwThreads;    // X chunks per thread per stage
constexpr int kRwTM = 8, kRwTN = 2;                              // 32 x 32 tiles per wave
constexpr int kRwBufferConfig = 0x00020000;                      // raw buffer resource word 3

// Chunk c of row r of a slab at r * 8 + (c ^ f(r)): the 32 rows an operand
// read touches at one chunk land on distinct 16-byte bank groups.
__device__ __forceinline__ int rw_chunk(int row, int chunk) {
    return row * kRwRowChunks + (chunk ^ (((row >> 1) ^ ((row & 1) << 2)) & 7));
}

// The source chunk (of 8 values) of a row's stage that operand chunk
// ci = 2 kk + kh holds: 4 (kk / 2) + 2 kh + kk % 2.
__device__ __forceinline__ int rw_source_chunk(int ci) {
    return (ci & 4) | ((ci & 1) << 1) | ((ci >> 1) & 1);
}

// One Q4_K block of the lane's two columns: the whole block is loaded at
// once (four stages' worth), so each cache line of W crosses from L2 once
// instead of once per stage.
struct RwBlock {
    uint4 hdr[kRwTN];     // block headers
    uint4 q[kRwTN][4];    // quant bytes 16 kh .. 16 kh + 15 of quarters 0..3
};

}  // namespace

__global__ __launch_bounds__(kRwThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void q4k_gemm_rw_kernel(const GemmBatch batch, uint32_t qmask) {
    __shared__ uint4 xs[4][kRwBM * kRwRowChunks];

    const int t = threadIdx.x;
    const int wave = t >> 6, lane = t & 63;

    int q, tm, tn, split;
    if (!tile_sched_next(batch.s, blockIdx.x, &q, &tm, &tn, &split)) return;
    const GemmProblem& pr = batch.p[q];
    const uint16_t* __restrict__ X = pr.X;
    float* __restrict__ Y = pr.Y;
    const int M = pr.M, N = pr.N, K = pr.K;
    const int n0 = tn * kRwBN, m0 = tm * kRwBM;
    const int nb = K / kQK;
    const int nstage = K / kRwBK;   // a multiple of 4
    auto last = [&](int s) { return min(s, nstage - 1); };

    // ---- X: copied from global memory straight into LDS (buffer loads with
    // the LDS bit: the 64 lanes of one instruction fill 1 KB of LDS in lane
    // order, no registers), four buffers deep.  Wave w fills chunks
    // 512 w + 64 j + lane (j < 8) of a stage's slab: row c / 8, slot c % 8,
    // which holds operand chunk slot ^ f(row) (rw_chunk's swizzle).  Rows
    // past M read zeros (the buffer ends at row M - 1).
    const long xrows = min(static_cast<long>(kRwBM), static_cast<long>(M - m0));
    const __amdgpu_buffer_rsrc_t xres = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(X + static_cast<long>(m0) * K), 0,
        static_cast<int>(xrows * K * 2), kRwBufferConfig);
    const int wave_s = __builtin_amdgcn_readfirstlane(wave);
    int xoff[kRwXChunks];
#pragma unroll
    for (int j = 0; j < kRwXChunks; ++j) {
        const int c = 512 * wave + 64 * j + lane;
        const int row = c >> 3;
        const int ci = (c & 7) ^ (((row >> 1) ^ ((row & 1) << 2)) & 7);
        xoff[j] = (row * K + 8 * rw_source_chunk(ci)) * 2;
    }
    auto dma_x = [&](int s, uint4* buf) {
#pragma unroll
        for (int j = 0; j < kRwXChunks; ++j)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                xres, buf + 512 * wave_s + 64 * j, 16, xoff[j] + last(s) * kRwBK * 2, 0, 0, 0);
    };

    // ---- W: the lane's columns n0 + 64 wave + 32 jb + (lane % 32), jb < 2
    // (columns past N repeat column N - 1: their outputs are never stored)
    const int kh = lane >> 5;
    const uint8_t* wcol[kRwTN];
#pragma unroll
    for (int jb = 0; jb < kRwTN; ++jb)
        wcol[jb] = pr.W +
                   static_cast<long>(min(n0 + 64 * wave + 32 * jb + (lane & 31), N - 1)) * nb *
                       kBlockBytes;
    auto load_block = [&](int b, RwBlock& r) {
        const int off = min(b, nb - 1) * kBlockBytes;
#pragma unroll
        for (int jb = 0; jb < kRwTN; ++jb) {
            r.hdr[jb] = load16(wcol[jb] + off);
#pragma unroll
            for (int c = 0; c < 4; ++c) r.q[jb][c] = load16(wcol[jb] + off + 16 + 32 * c + 16 * kh);
        }
    };

    // B operands of the stage: bq[jb][kk].  dequant_half(h) fills k-steps h
    // (low nibbles of dwords 2h, 2h+1) and 2 + h (their high nibbles) from
    // quarter c of the block.
    uint4 bq[kRwTN][4];
    QuarterScales qs[kRwTN];
    auto scales = [&](const RwBlock& r, int c) {
#pragma unroll
        for (int jb = 0; jb < kRwTN; ++jb)
            qs[jb] = quarter_scales(r.hdr[jb], static_cast<uint32_t>(c));
    };
    auto dequant_half = [&](const RwBlock& r, int c, int h) {
#pragma unroll
        for (int jb = 0; jb < kRwTN; ++jb) {
            const uint4 qv = r.q[jb][c];
            const uint32_t w0 = h ? qv.z : qv.x;
            const uint32_t w1 = h ? qv.w : qv.y;
            uint32_t lo_a[2], hi_a[2], lo_b[2], hi_b[2];
            dequant_dword_bf16(w0, qs[jb], lo_a, hi_a, qmask);
            dequant_dword_bf16(w1, qs[jb], lo_b, hi_b, qmask);
            bq[jb][h] = make_uint4(lo_a[0], lo_a[1], lo_b[0], lo_b[1]);
            bq[jb][2 + h] = make_uint4(hi_a[0], hi_a[1], hi_b[0], hi_b[1]);
        }
    };

    // ---- A operands and the matrix instructions
    float16_t acc[kRwTM][kRwTN];
#pragma unroll
    for (int i = 0; i < kRwTM; ++i)
#pragma unroll
        for (int jb = 0; jb < kRwTN; ++jb) acc[i][jb] = float16_t{};
    const int arow = lane & 31;
    auto read_a = [&](const uint4* buf, int kk, bf16x8_t* a) {
#pragma unroll
        for (int i = 0; i < kRwTM; ++i)
            a[i] = __builtin_bit_cast(bf16x8_t, buf[rw_chunk(32 * i + arow, 2 * kk + kh)]);
    };
    auto mma = [&](int kk, const bf16x8_t* a) {
#pragma unroll
        for (int i = 0; i < kRwTM; ++i)
#pragma unroll
            for (int jb = 0; jb < kRwTN; ++jb)
                acc[i][jb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                    a[i], __builtin_bit_cast(bf16x8_t, bq[jb][kk]), acc[i][jb], 0, 0, 0);
    };
    auto fence = [] { __builtin_amdgcn_sched_barrier(0); };

    bf16x8_t a0[kRwTM], a1[kRwTM];
    // Order of the region just written (the wave issues in order and a
    // matrix instruction occupies the matrix core for 32 cycles, so the
    // vector work has to sit between the matrix instructions to run under
    // them): first the region's `reads` LDS reads of operands (needed 16
    // matrix instructions later), then 32 times one matrix instruction and
    // `v` vector instructions, the second 16 of them each followed by one of
    // the `mem` remaining LDS / global memory instructions while they last.
    auto interleave = [](auto reads_c, auto v_c, auto mem_c) {
        constexpr int reads = decltype(reads_c)::value, v = decltype(v_c)::value,
                      mem = decltype(mem_c)::value;
        __builtin_amdgcn_sched_group_barrier(0x100, reads, 0);      // DS read
#pragma unroll
        for (int i = 0; i < 32; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);      // MFMA
            __builtin_amdgcn_sched_group_barrier(0x002, v, 0);      // VALU
            if (i >= 16 && (i - 16) * 2 < mem)
                __builtin_amdgcn_sched_group_barrier(0x090, 2, 0);  // DS / VMEM
        }
    };
    // One stage, quarter c (compile-time) of block b = s / 4, X in buffer c:
    // multiply stage s (its k-step 0 operands already in a0, B of k-steps 0
    // and 2 already in bq), dequantise half 1 of stage s and half 0 of stage
    // s + 1, read the k-step 0 operands of stage s + 1 and copy X of stage
    // s + 3.  At c = 0 the block ring turns (W of block b moves to cur_b) and
    // block b + 1 is requested into nxt_b.  Two scheduling regions of 32
    // matrix instructions each, with the barrier between them.
    RwBlock cur_b, nxt_b;
    auto stage = [&](int s, auto c_c) {
        constexpr int c = decltype(c_c)::value;
        const uint4* cur = xs[c];
        const uint4* nxt = xs[(c + 1) & 3];
        uint4* xdma = xs[(c + 3) & 3];
        if constexpr (c == 0) cur_b = nxt_b;
        // region 1: k-steps 0 and 2, half 1 of this stage dequantised, the
        // k-step 1 operands read
        read_a(cur, 2, a1);
        mma(0, a0);
        dequant_half(cur_b, c, 1);
        read_a(cur, 1, a0);
        mma(2, a1);
        interleave(std::integral_constant<int, 8>{}, std::integral_constant<int, 3>{},
                   std::integral_constant<int, 8>{});
        fence();
        // X of stage s + 1 (copied in the second region of stage s - 2) has
        // landed.  Issued after it: at c = 1 the block loads of stage s - 1
        // (10) and the X copy of stage s - 1 (8); else that X copy alone.  A
        // bare barrier: __syncthreads would also wait for the loads still in
        // flight.  Past it every wave is done with the buffer of stage s - 1.
        if constexpr (c == 1)
            asm volatile("s_waitcnt vmcnt(18) lgkmcnt(0)" ::: "memory");
        else
            asm volatile("s_waitcnt vmcnt(8) lgkmcnt(0)" ::: "memory");
        __builtin_amdgcn_s_barrier();
        fence();
        if constexpr (c == 0) {
            load_block((s >> 2) + 1, nxt_b);
            fence();
        }
        // region 2: k-steps 1 and 3, half 0 of the next stage dequantised,
        // the operands of k-step 3 and of the next stage's k-step 0 read, X
        // of stage s + 3 copied into the buffer stage s - 1 used
        read_a(cur, 3, a1);
        mma(1, a0);
        if constexpr (c < 3) {
            scales(cur_b, c + 1);
            dequant_half(cur_b, c + 1, 0);
        } else {
            scales(nxt_b, 0);
            dequant_half(nxt_b, 0, 0);
        }
        read_a(nxt, 0, a0);
        mma(3, a1);
        dma_x(s + 3, xdma);
        interleave(std::integral_constant<int, 8>{}, std::integral_constant<int, 4>{},
                   std::integral_constant<int, 16>{});
        fence();
    };
    using C0 = std::integral_constant<int, 0>;
    using C1 = std::integral_constant<int, 1>;
    using C2 = std::integral_constant<int, 2>;
    using C3 = std::integral_constant<int, 3>;

    load_block(0, nxt_b);
    dma_x(0, xs[0]);
    dma_x(1, xs[1]);
    dma_x(2, xs[2]);
    // W block 0 and this wave's part of X stage 0 have landed (the copies of
    // stages 1 and 2, 16 instructions, may still be in flight)
    asm volatile("s_waitcnt vmcnt(16)" ::: "memory");
    scales(nxt_b, 0);
    dequant_half(nxt_b, 0, 0);
    __builtin_amdgcn_s_barrier();
    read_a(xs[0], 0, a0);
    for (int s = 0; s < nstage; s += 4) {
        stage(s, C0{});
        stage(s + 1, C1{});
        stage(s + 2, C2{});
        stage(s + 3, C3{});
    }

    // ---- Y: lane holds D[m][n] for n = 32 jb + lane % 32 and
    // m = 32 i + 8 (r / 4) + 4 kh + r % 4 of the wave's 256 x 64.  Streaming
    // (nontemporal) stores: Y is not read again here, and keeping it out of
    // L2 leaves the X and W lines that other workgroups still read (12 and
    // 6% faster on the Qwen3-4B layer at M = 2048 and the LM head at M = 512).
#pragma unroll
    for (int i = 0; i < kRwTM; ++i) {
#pragma unroll
        for (int jb = 0; jb < kRwTN; ++jb) {
            const int n = n0 + 64 * wave + 32 * jb + (lane & 31);
            if (n >= N) continue;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int m = m0 + 32 * i + 8 * (r >> 2) + 4 * kh + (r & 3);
                if (m < M) __builtin_nontemporal_store(acc[i][jb][r], Y + static_cast<long>(m) * N + n);
            }
        }
    }
}

hipError_t launch_gemm_rw(const uint8_t* const* W, const uint16_t* const* X, float* const* Y,
                          const int* M, const int* N, const int* K, int count,
                          hipStream_t stream) {
    GemmBatch b;
    const long grid = gemm_batch_init(b, W, X, Y, M, N, K, count, kRwBM, kRwBN);
    hipLaunchKernelGGL(q4k_gemm_rw_kernel, dim3(static_cast<unsigned>(grid)), dim3(kRwThreads), 0,
                       stream, b, kNibbleMask);
    return hipGetLastError();
}

}  // namespace jq4k
