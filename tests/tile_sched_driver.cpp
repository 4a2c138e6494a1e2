// Host driver for the matmul tile schedule: reads "count BM BN group_m" and
// count triples "M N splits" from stdin, prints the launch size, then one
// line per workgroup: "q tile_m tile_n split", or "-1" for an idle workgroup.
//
// With "plan" as the first word instead, reads "count BM BN min_items" and
// count triples "M N K", and prints the K splits of splitk_plan, its item
// count and the workspace bytes on one line.
#include <cstdio>
#include <cstdlib>

#include "tile_sched.h"

static int plan() {
    int count, BM, BN;
    long min_items;
    if (std::scanf("%d %d %d %ld", &count, &BM, &BN, &min_items) != 4) return 2;
    if (count < 1 || count > jq4k::kSchedMax) return 2;
    int M[jq4k::kSchedMax], N[jq4k::kSchedMax], K[jq4k::kSchedMax], S[jq4k::kSchedMax];
    for (int i = 0; i < count; ++i)
        if (std::scanf("%d %d %d", &M[i], &N[i], &K[i]) != 3) return 2;
    const long items = jq4k::splitk_plan(M, N, K, count, BM, BN, min_items, S);
    for (int i = 0; i < count; ++i) std::printf("%d ", S[i]);
    std::printf("%ld %ld\n", items, jq4k::splitk_workspace_bytes(M, N, S, count, BM, BN));
    return 0;
}

int main() {
    char word[16];
    if (std::scanf("%15s", word) != 1) return 2;
    if (word[0] == 'p') return plan();
    int count, BM, BN, group_m;
    count = std::atoi(word);
    if (std::scanf("%d %d %d", &BM, &BN, &group_m) != 3) return 2;
    if (count < 1 || count > jq4k::kSchedMax) return 2;
    int M[jq4k::kSchedMax], N[jq4k::kSchedMax], S[jq4k::kSchedMax];
    for (int i = 0; i < count; ++i)
        if (std::scanf("%d %d %d", &M[i], &N[i], &S[i]) != 3) return 2;
    jq4k::TileSched s;
    const long grid = jq4k::tile_sched_init(s, M, N, S, count, BM, BN, group_m);
    std::printf("%ld\n", grid);
    for (long b = 0; b < grid; ++b) {
        int q, tm, tn, split;
        if (jq4k::tile_sched_next(s, static_cast<unsigned>(b), &q, &tm, &tn, &split))
            std::printf("%d %d %d %d\n", q, tm, tn, split);
        else
            std::printf("-1\n");
    }
    return 0;
}
