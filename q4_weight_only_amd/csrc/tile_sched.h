// tile_sched.h -- which output tile each workgroup of a matmul launch
// computes, and the list of problems a launch carries.
//
// A launch covers one or more independent problems, each a TM x TN grid of
// output tiles.  An MI355X has eight accelerator complex dies (XCDs), each
// with its own L2; the hardware hands workgroup i to XCD i % 8, in order.
// The schedule gives every XCD the same share of every problem (problem q
// contributes per_xcd[q] = ceil(TM TN / 8) consecutive entries to each XCD's
// queue), so the XCDs finish together whatever the problems' sizes, and the
// problems appear in each queue in the order the host lists them (longest K
// first, so the long tiles do not form the tail).
//
// Inside a problem the tiles run in grouped order: bands of group_m tile rows;
// within a band, column by column, the band's rows fastest.  The workgroups
// resident on one XCD then share a few row blocks of X and a few column blocks
// of W, both small enough to stay in its L2, instead of every row of tiles
// streaming all of W again.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace jq4k {

constexpr int kXcds = 8;
constexpr int kSchedMax = 16;   // problems per launch

struct TileSched {
    int count;
    int group_m;                    // tile rows per band
    int tm[kSchedMax], tn[kSchedMax];
    int per_xcd[kSchedMax];         // queue entries of problem q on every XCD
    int xfirst[kSchedMax + 1];      // prefix sums of per_xcd
};

// Host side: problems 0..count-1 (in queue order) with M[q] x N[q] outputs in
// BM x BN tiles.  Returns the number of workgroups to launch (8 xfirst[count]).
inline long tile_sched_init(TileSched& s, const int* M, const int* N, int count, int BM, int BN,
                            int group_m) {
    s = TileSched{};
    s.count = count;
    s.group_m = group_m;
    long queue = 0;
    for (int q = 0; q < count; ++q) {
        s.tm[q] = (M[q] + BM - 1) / BM;
        s.tn[q] = (N[q] + BN - 1) / BN;
        const long tiles = static_cast<long>(s.tm[q]) * s.tn[q];
        s.per_xcd[q] = static_cast<int>((tiles + kXcds - 1) / kXcds);
        s.xfirst[q] = static_cast<int>(queue);
        queue += s.per_xcd[q];
    }
    s.xfirst[count] = static_cast<int>(queue);
    return queue * kXcds;
}

// The tile of workgroup `block`.  Returns false for the few workgroups past
// the end of a problem's share (they have nothing to do); otherwise sets the
// problem index and the tile's row and column.
__host__ __device__ __forceinline__ bool tile_sched_next(const TileSched& s, unsigned block,
                                                         int* q_out, int* tile_m, int* tile_n) {
    const int x = static_cast<int>(block % kXcds), j = static_cast<int>(block / kXcds);
    int q = 0;
    while (q + 1 < s.count && j >= s.xfirst[q + 1]) ++q;
    const int TM = s.tm[q], TN = s.tn[q];
    const int t = x * s.per_xcd[q] + (j - s.xfirst[q]);
    if (t >= TM * TN) return false;
    const int band = t / (s.group_m * TN);
    const int first = band * s.group_m;
    const int rows = TM - first < s.group_m ? TM - first : s.group_m;
    const int r = t - band * s.group_m * TN;
    *q_out = q;
    *tile_m = first + r % rows;
    *tile_n = r / rows;
    return true;
}

// One launch computes the tiles of up to kSchedMax independent problems (a
// single matmul is a batch of one); the descriptors and the tile schedule
// travel in the kernel arguments.
struct GemmProblem {
    const uint8_t* W;
    const uint16_t* X;
    float* Y;
    int M, N, K;
    const uint8_t* W2;   // up matrix of a SwiGLU pair (W is the gate), else null
};

struct GemmBatch {
    GemmProblem p[kSchedMax];
    TileSched s;
};

// Band height of the grouped tile order, in tile rows: 256 rows of X for
// the 64- and 128-row tiles, 512 for the 256-row tile (measured best on the
// seven projections of a layer at M = 512 .. 4096).
constexpr int group_rows(int BM) { return BM >= 256 ? 2 : 256 / BM; }

// Host side: the batch for BM x BN tiles, problems queued longest K first
// (stable).  Returns the number of workgroups to launch.
inline long gemm_batch_init(GemmBatch& b, const uint8_t* const* W, const uint16_t* const* X,
                            float* const* Y, const int* M, const int* N, const int* K, int count,
                            int BM, int BN) {
    int order[kSchedMax];
    for (int i = 0; i < count; ++i) order[i] = i;
    for (int i = 1; i < count; ++i)
        for (int j = i; j > 0 && K[order[j]] > K[order[j - 1]]; --j) {
            const int t = order[j];
            order[j] = order[j - 1];
            order[j - 1] = t;
        }
    b = GemmBatch{};
    int Ms[kSchedMax], Ns[kSchedMax];
    for (int i = 0; i < count; ++i) {
        const int o = order[i];
        b.p[i] = {W[o], X[o], Y[o], M[o], N[o], K[o], nullptr};
        Ms[i] = M[o];
        Ns[i] = N[o];
    }
    return tile_sched_init(b.s, Ms, Ns, count, BM, BN, group_rows(BM));
}

}  // namespace jq4k
