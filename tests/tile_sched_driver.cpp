// Host driver for the matmul tile schedule: reads "count BM BN group_m" and
// count pairs "M N" from stdin, prints the launch size, then one line per
// workgroup: "q tile_m tile_n", or "-1" for an idle workgroup.
#include <cstdio>

#include "tile_sched.h"

int main() {
    int count, BM, BN, group_m;
    if (std::scanf("%d %d %d %d", &count, &BM, &BN, &group_m) != 4) return 2;
    if (count < 1 || count > jq4k::kSchedMax) return 2;
    int M[jq4k::kSchedMax], N[jq4k::kSchedMax];
    for (int i = 0; i < count; ++i)
        if (std::scanf("%d %d", &M[i], &N[i]) != 2) return 2;
    jq4k::TileSched s;
    const long grid = jq4k::tile_sched_init(s, M, N, count, BM, BN, group_m);
    std::printf("%ld\n", grid);
    for (long b = 0; b < grid; ++b) {
        int q, tm, tn;
        if (jq4k::tile_sched_next(s, static_cast<unsigned>(b), &q, &tm, &tn))
            std::printf("%d %d %d\n", q, tm, tn);
        else
            std::printf("-1\n");
    }
    return 0;
}
