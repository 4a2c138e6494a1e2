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
//
// A problem may split K: each of its tiles is then splits[q] queue entries,
// one per range of K blocks, adjacent in one XCD's queue (per_xcd[q] is a
// multiple of splits[q]), so the partial sums of a tile meet in one L2.
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
    int splits[kSchedMax];          // K ranges per tile of problem q (1: whole K)
    int per_xcd[kSchedMax];         // queue entries of problem q on every XCD
    int xfirst[kSchedMax + 1];      // prefix sums of per_xcd
};

// Host side: problems 0..count-1 (in queue order) with M[q] x N[q] outputs in
// BM x BN tiles, splits[q] K ranges per tile (null: 1 for all).  Returns the
// number of workgroups to launch (8 xfirst[count]).
inline long tile_sched_init(TileSched& s, const int* M, const int* N, const int* splits,
                            int count, int BM, int BN, int group_m) {
    s = TileSched{};
    s.count = count;
    s.group_m = group_m;
    long queue = 0;
    for (int q = 0; q < count; ++q) {
        s.tm[q] = (M[q] + BM - 1) / BM;
        s.tn[q] = (N[q] + BN - 1) / BN;
        s.splits[q] = splits ? splits[q] : 1;
        const long tiles = static_cast<long>(s.tm[q]) * s.tn[q];
        s.per_xcd[q] = static_cast<int>((tiles + kXcds - 1) / kXcds * s.splits[q]);
        s.xfirst[q] = static_cast<int>(queue);
        queue += s.per_xcd[q];
    }
    s.xfirst[count] = static_cast<int>(queue);
    return queue * kXcds;
}

// The tile of workgroup `block`.  Returns false for the few workgroups past
// the end of a problem's share (they have nothing to do); otherwise sets the
// problem index, the tile's row and column and the K range (0 .. splits - 1).
__host__ __device__ __forceinline__ bool tile_sched_next(const TileSched& s, unsigned block,
                                                         int* q_out, int* tile_m, int* tile_n,
                                                         int* split) {
    const int x = static_cast<int>(block % kXcds), j = static_cast<int>(block / kXcds);
    int q = 0;
    while (q + 1 < s.count && j >= s.xfirst[q + 1]) ++q;
    const int TM = s.tm[q], TN = s.tn[q], S = s.splits[q];
    const int e = x * s.per_xcd[q] + (j - s.xfirst[q]);
    const int t = e / S;
    if (t >= TM * TN) return false;
    *split = e - t * S;
    const int band = t / (s.group_m * TN);
    const int first = band * s.group_m;
    const int rows = TM - first < s.group_m ? TM - first : s.group_m;
    const int r = t - band * s.group_m * TN;
    *q_out = q;
    *tile_m = first + r % rows;
    *tile_n = r / rows;
    return true;
}

// ---- split K (host side).
//
// K splits per problem for a launch of BM x BN tiles: each K range is whole
// Q4_K blocks (splits <= K / 256).  With S0 the fewest 64-wide K stages per
// tile among the problems, a range is about T = 2 S0 stages (at least 16):
// every problem takes round(K / 64 / T) ranges, so no workgroup runs more
// than about twice the shortest whole-K one (each split adds a partial tile
// and its publication: on a Qwen3-4B layer at M = 33, ranges of S0 stages
// measured 12% slower, of S0 / 2 stages 85% slower); while the launch has
// fewer than min_items workgroups, T halves (not below 16 stages).
//
// The last round.  min_items is also what the launch holds at once (two
// workgroups per CU), min_items / 8 per XCD.  Entries of an XCD's queue past
// its last whole round run after the others, nearly alone; when they are
// whole tiles they set the length of the launch.  If one problem that keeps
// whole K has no more tiles per XCD than a quarter round but at least that
// overflow, and K short enough that its halves are the shortest ranges of
// the launch (queued last), it is split in 2: the overflow is then made of
// half ranges.  Among such problems the fewest tiles per XCD win (ties: the
// last given).  On a Qwen3-4B layer at M = 16 .. 64 that is v: 4-7% faster.
// Returns the number of workgroups' worth of tiles x ranges.
constexpr int kSplitMinStages = 16;

inline long splitk_plan(const int* M, const int* N, const int* K, int count, int BM, int BN,
                        long min_items, int* splits) {
    int T = 0x7FFFFFFF;
    for (int q = 0; q < count; ++q) T = K[q] / 64 < T ? K[q] / 64 : T;
    T *= 2;
    if (T < kSplitMinStages) T = kSplitMinStages;
    long items = 0;
    for (;;) {
        items = 0;
        for (int q = 0; q < count; ++q) {
            const int nst = K[q] / 64, nb = K[q] / 256;
            int S = (nst + T / 2) / T;
            S = S < 1 ? 1 : (S > nb ? nb : S);
            splits[q] = S;
            items += static_cast<long>((M[q] + BM - 1) / BM) * ((N[q] + BN - 1) / BN) * S;
        }
        if (items >= min_items || T <= kSplitMinStages) break;
        T = T / 2 < kSplitMinStages ? kSplitMinStages : T / 2;
    }
    // the last round (above)
    const long round = min_items / kXcds;
    long queue = 0;
    for (int q = 0; q < count; ++q)
        queue += (static_cast<long>((M[q] + BM - 1) / BM) * ((N[q] + BN - 1) / BN) + kXcds - 1) /
                 kXcds * splits[q];
    const long over = round > 0 ? queue % round : 0;
    if (queue <= round || over == 0) return items;
    int pick = -1;
    long pick_x = 0;
    for (int q = 0; q < count; ++q) {
        const long tiles = static_cast<long>((M[q] + BM - 1) / BM) * ((N[q] + BN - 1) / BN);
        const long per_x = (tiles + kXcds - 1) / kXcds;
        if (splits[q] != 1 || K[q] / 256 < 2 || per_x < over || 4 * per_x > round) continue;
        bool last = true;   // K[q] / 2 < K[p] / S[p] for every other problem
        for (int p = 0; p < count; ++p)
            if (p != q && static_cast<long>(K[q]) * splits[p] >= 2L * K[p]) last = false;
        if (last && (pick < 0 || per_x <= pick_x)) {
            pick = q;
            pick_x = per_x;
        }
    }
    if (pick >= 0) {
        splits[pick] = 2;
        items += static_cast<long>((M[pick] + BM - 1) / BM) * ((N[pick] + BN - 1) / BN);
    }
    return items;
}

// Workspace of a split-K launch: one int counter per split tile, padded to
// 256 bytes, then for each split tile `splits` partial BM x BN fp32 tiles.
inline long splitk_counter_bytes(long counters) { return (counters * 4 + 255) / 256 * 256; }

inline long splitk_workspace_bytes(const int* M, const int* N, const int* splits, int count,
                                   int BM, int BN) {
    long counters = 0, floats = 0;
    for (int q = 0; q < count; ++q) {
        if (splits[q] <= 1) continue;
        const long tiles = static_cast<long>((M[q] + BM - 1) / BM) * ((N[q] + BN - 1) / BN);
        counters += tiles;
        floats += tiles * splits[q] * BM * BN;
    }
    if (counters == 0) return 0;
    return splitk_counter_bytes(counters) + floats * 4;
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
    float* part;         // split K: partial tiles, splits x BM x BN floats per tile
    int* cnt;            // split K: one arrival counter per tile (zero between calls)
};

struct GemmBatch {
    GemmProblem p[kSchedMax];
    TileSched s;
};

// Band height of the grouped tile order, in tile rows: 256 rows of X for
// the 64- and 128-row tiles, 512 for the 256-row tile (measured best on the
// seven projections of a layer at M = 512 .. 4096).
constexpr int group_rows(int BM) { return BM >= 256 ? 2 : 256 / BM; }

// Host side: the batch for BM x BN tiles, problems queued longest K range
// first (K / splits; stable).  splits null: whole K everywhere.  With splits,
// `ws` is the workspace laid out as splitk_workspace_bytes describes.
// Returns the number of workgroups to launch.
inline long gemm_batch_init(GemmBatch& b, const uint8_t* const* W, const uint16_t* const* X,
                            float* const* Y, const int* M, const int* N, const int* K, int count,
                            int BM, int BN, const int* splits = nullptr, void* ws = nullptr) {
    int S[kSchedMax];
    for (int i = 0; i < count; ++i) S[i] = splits ? splits[i] : 1;
    int order[kSchedMax];
    for (int i = 0; i < count; ++i) order[i] = i;
    // a before b when K_a / S_a > K_b / S_b
    auto longer = [&](int a, int c) {
        return static_cast<long>(K[a]) * S[c] > static_cast<long>(K[c]) * S[a];
    };
    for (int i = 1; i < count; ++i)
        for (int j = i; j > 0 && longer(order[j], order[j - 1]); --j) {
            const int t = order[j];
            order[j] = order[j - 1];
            order[j - 1] = t;
        }
    b = GemmBatch{};
    int Ms[kSchedMax], Ns[kSchedMax], Ss[kSchedMax];
    int* cnt = static_cast<int*>(ws);
    float* part = nullptr;
    if (ws) {
        long counters = 0;
        for (int i = 0; i < count; ++i)
            if (S[i] > 1) counters += static_cast<long>((M[i] + BM - 1) / BM) * ((N[i] + BN - 1) / BN);
        part = reinterpret_cast<float*>(static_cast<char*>(ws) + splitk_counter_bytes(counters));
    }
    for (int i = 0; i < count; ++i) {
        const int o = order[i];
        b.p[i] = {W[o], X[o], Y[o], M[o], N[o], K[o], nullptr, nullptr, nullptr};
        Ms[i] = M[o];
        Ns[i] = N[o];
        Ss[i] = S[o];
        if (S[o] > 1 && ws) {
            const long tiles = static_cast<long>((M[o] + BM - 1) / BM) * ((N[o] + BN - 1) / BN);
            b.p[i].cnt = cnt;
            b.p[i].part = part;
            cnt += tiles;
            part += tiles * S[o] * BM * BN;
        }
    }
    return tile_sched_init(b.s, Ms, Ns, Ss, count, BM, BN, group_rows(BM));
}

}  // namespace jq4k
