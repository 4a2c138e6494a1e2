"""Host checks of the matmul tile schedule (csrc/tile_sched.h), compiled into
a small host program: every tile of every problem (and every K range of a
split tile) is computed by exactly one workgroup, each XCD (workgroup index
mod 8) gets an equal share of every problem, the K ranges of a tile sit next
to each other on one XCD, the grouped order keeps bands of tile rows
together, and the split-K plan gives every workgroup about the same number of
K stages."""
import collections
import os
import subprocess

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "q4_weight_only_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    exe = str(tmp_path_factory.mktemp("sched") / "tile_sched_driver")
    subprocess.run([HIPCC, "-std=c++17", "-x", "hip", "--offload-arch=gfx950", "-I", CSRC,
                    os.path.join(ROOT, "tests", "tile_sched_driver.cpp"), "-o", exe],
                   check=True, capture_output=True)
    return exe


def schedule(driver, BM, BN, group_m, shapes, splits=None):
    """Rows (q, tile_m, tile_n) per workgroup (split K: (q, tile_m, tile_n,
    range)); (-1,) for an idle one."""
    whole_k = splits is None
    splits = splits or [1] * len(shapes)
    inp = f"{len(shapes)} {BM} {BN} {group_m} " + " ".join(
        f"{m} {n} {s}" for (m, n), s in zip(shapes, splits))
    out = subprocess.run([driver], input=inp, capture_output=True, text=True, check=True)
    lines = out.stdout.split("\n")
    grid = int(lines[0])
    rows = [tuple(map(int, l.split())) for l in lines[1:1 + grid]]
    assert len(rows) == grid and grid % 8 == 0
    if whole_k:
        assert all(r == (-1,) or r[3] == 0 for r in rows)
        rows = [r if r == (-1,) else r[:3] for r in rows]
    return rows


def plan(driver, BM, BN, min_items, shapes):
    """splitk_plan: (splits per problem, items, workspace bytes)."""
    inp = f"plan {len(shapes)} {BM} {BN} {min_items} " + " ".join(
        f"{m} {n} {k}" for m, n, k in shapes)
    out = subprocess.run([driver], input=inp, capture_output=True, text=True, check=True)
    v = list(map(int, out.stdout.split()))
    return v[:len(shapes)], v[-2], v[-1]


def check(rows, BM, BN, shapes, splits=None):
    whole_k = splits is None
    splits = splits or [1] * len(shapes)
    seen = collections.Counter(r for r in rows if r != (-1,))
    for q, ((m, n), S) in enumerate(zip(shapes, splits)):
        tm, tn = -(-m // BM), -(-n // BN)
        if whole_k:
            want = {(q, i, j) for i in range(tm) for j in range(tn)}
        else:
            want = {(q, i, j, s) for i in range(tm) for j in range(tn) for s in range(S)}
        got = {k for k in seen if k[0] == q}
        assert got == want, f"problem {q}: tiles missing or extra"
    assert all(c == 1 for c in seen.values()), "a tile computed twice"
    # equal share per XCD: per problem, the XCD counts differ by at most one
    # whole per-XCD share boundary (the last XCDs may come up short)
    for q, ((m, n), S) in enumerate(zip(shapes, splits)):
        total = -(-m // BM) * -(-n // BN)
        per = -(-total // 8) * S
        counts = [sum(1 for b, r in enumerate(rows) if b % 8 == x and r[0] == q and r != (-1,))
                  for x in range(8)]
        assert sum(counts) == total * S
        assert max(counts) == per


@pytest.mark.parametrize("BM,BN,group_m", [(128, 128, 4), (64, 256, 8), (256, 128, 2),
                                           (128, 128, 1), (128, 128, 3)])
def test_every_tile_once(driver, BM, BN, group_m):
    rng = np.random.default_rng(BM * 7 + group_m)
    for count in (1, 2, 7, 16):
        shapes = [(int(rng.integers(1, 1500)), int(rng.integers(1, 3000)))
                  for _ in range(count)]
        rows = schedule(driver, BM, BN, group_m, shapes)
        check(rows, BM, BN, shapes)


def test_prefill_layer_shapes(driver):
    shapes = [(2048, 9728), (2048, 4096), (2048, 1024), (2048, 2560)]
    rows = schedule(driver, 128, 128, 4, shapes)
    check(rows, 128, 128, shapes)


def test_grouped_order(driver):
    """Within an XCD's share, tiles of one problem go band by band (group_m
    tile rows), column by column, the band's rows fastest."""
    M, N, BM, BN, g = 2048, 9728, 128, 128, 4
    rows = schedule(driver, BM, BN, g, [(M, N)])
    tn_count = -(-N // BN)
    order = [r for r in rows[0::8] if r != (-1,)]   # XCD 0's queue, in order
    expect = []
    for t in range(len(order)):
        band, r = divmod(t, g * tn_count)
        expect.append((0, band * g + r % g, r // g))
    assert order == expect


def test_single_tile_and_ragged_band(driver):
    rows = schedule(driver, 128, 128, 4, [(1, 1)])
    assert rows[0] == (0, 0, 0) and all(r == (-1,) for r in rows[1:])
    shapes = [(5 * 128 + 3, 3 * 128)]        # 6 tile rows: one full band, one of 2
    rows = schedule(driver, 128, 128, 4, shapes)
    check(rows, 128, 128, shapes)


def test_split_ranges_adjacent_on_one_xcd(driver):
    """The K ranges of a tile are consecutive entries of one XCD's queue."""
    rng = np.random.default_rng(5)
    for count in (1, 3, 7):
        shapes = [(int(rng.integers(1, 65)), int(rng.integers(1, 3000))) for _ in range(count)]
        splits = [int(rng.integers(1, 11)) for _ in range(count)]
        rows = schedule(driver, 64, 64, 4, shapes, splits)
        check(rows, 64, 64, shapes, splits)
        for x in range(8):
            queue = [r for r in rows[x::8] if r != (-1,)]
            i = 0
            while i < len(queue):
                q, tm, tn, s = queue[i]
                S = splits[q]
                assert s == 0
                assert queue[i:i + S] == [(q, tm, tn, u) for u in range(S)]
                i += S


LAYER_M33 = [(33, 4096, 2560), (33, 1024, 2560), (33, 1024, 2560), (33, 2560, 4096),
             (33, 9728, 2560), (33, 9728, 2560), (33, 2560, 9728)]


def test_splitk_plan(driver):
    """The seven projections of a Qwen3-4B layer at M = 33: ranges of about
    twice the shortest whole K (80 stages): down splits in 2 (76 stages
    each).  That queues 65 entries per XCD against 64 resident workgroups,
    so v (2 tiles per XCD, K = 2560) also splits in 2 and its half ranges
    fill the last round: 536 workgroups, and a workspace of one counter and
    S partial 64 x 64 tiles per split tile."""
    S, items, ws = plan(driver, 64, 64, 512, LAYER_M33)
    assert S == [1, 1, 2, 1, 1, 1, 2]
    assert items == 64 + 16 + 16 * 2 + 40 + 152 + 152 + 40 * 2
    counters = 16 + 40
    assert ws == (counters * 4 + 255) // 256 * 256 + (16 * 2 + 40 * 2) * 64 * 64 * 4
    # down alone: too few tiles, so the target halves down to 16 stages
    S, items, _ = plan(driver, 64, 64, 512, [(33, 2560, 9728)])
    assert S == [10] and items == 400
    # short K never splits below one block per range, nor below 16 stages
    S, items, ws = plan(driver, 64, 64, 512, [(8, 64, 256), (8, 64, 512)])
    assert S == [1, 1] and ws == 0
    # per-range stage counts stay within a factor of about three of each other
    rng = np.random.default_rng(9)
    for _ in range(20):
        shapes = [(int(rng.integers(1, 65)), int(rng.integers(1, 20000)),
                   256 * int(rng.integers(1, 80))) for _ in range(int(rng.integers(1, 8)))]
        S, items, _ = plan(driver, 64, 64, 512, shapes)
        assert all(1 <= s <= k // 256 for s, (_, _, k) in zip(S, shapes))
        assert items == sum(-(-m // 64) * -(-n // 64) * s for s, (m, n, _) in zip(S, shapes))
        lens = [k / 64 / s for s, (_, _, k) in zip(S, shapes)]
        if min(k for _, _, k in shapes) >= 16 * 64 * 2:
            assert max(lens) <= 3 * min(lens) + 16


def test_splitk_last_round(driver):
    """The last-round rule of splitk_plan.  On the M = 33 layer the entries of
    each XCD's queue past its 64 resident workgroups are all half ranges of
    the problem it split (queued last, longest range first).  It leaves the
    plan alone when no entry runs past a whole round, when no problem with
    whole K covers the overflow in at most a quarter round of tiles, when
    the halves would not be the shortest ranges, and for a single problem."""
    S, items, _ = plan(driver, 64, 64, 512, LAYER_M33)
    # the launch queues the problems longest K range first (stable)
    order = sorted(range(7), key=lambda q: -LAYER_M33[q][2] / S[q])
    shapes = [LAYER_M33[q][:2] for q in order]
    splits = [S[q] for q in order]
    rows = schedule(driver, 64, 64, 4, shapes, splits)
    check(rows, 64, 64, shapes, splits)
    for x in range(8):
        queue = [r for r in rows[x::8] if r != (-1,)]
        assert len(queue) == 67
        assert all(order[i] == 2 and splits[i] == 2 for i, *_ in queue[64:])
    # an exact round: 64 entries per XCD (512 tiles of one K), no change
    S, items, ws = plan(driver, 64, 64, 512, [(33, 64 * 256, 2560), (33, 64 * 256, 2560)])
    assert S == [1, 1] and items == 512 and ws == 0
    # overflow of 8 per XCD, every problem too large to cover it in a
    # quarter round (17 tiles per XCD): no change
    shapes = [(33, 64 * 136, 2560)] * 4
    S, items, ws = plan(driver, 64, 64, 512, shapes)
    assert S == [1, 1, 1, 1] and items == 544 and ws == 0
    # the problem with the fewest tiles (K = 5120) would halve to 2560, not
    # shorter than the K = 2560 problems' whole ranges: the next one is split
    shapes = [(33, 64 * 8 * 2, 5120), (33, 64 * 8 * 61, 2560), (33, 64 * 8 * 3, 2560)]
    S, items, _ = plan(driver, 64, 64, 512, shapes)
    assert S == [1, 1, 2] and items == 8 * (2 + 61 + 2 * 3)
    # ties: the last given of the problems with the fewest tiles per XCD
    shapes = [(33, 64 * 8 * 61, 2560), (33, 64 * 8 * 2, 2560), (33, 64 * 8 * 2, 2560)]
    S, _, _ = plan(driver, 64, 64, 512, shapes)
    assert S == [1, 1, 2]
    # one problem past a round: never split by this rule (its own plan only)
    S, _, _ = plan(driver, 64, 64, 512, [(33, 151936, 2560)])
    assert S == [1]
