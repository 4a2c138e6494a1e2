"""Host checks of the matmul tile schedule (csrc/tile_sched.h), compiled into
a small host program: every tile of every problem is computed by exactly one
workgroup, each XCD (workgroup index mod 8) gets an equal share of every
problem, and the grouped order keeps bands of tile rows together."""
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


def schedule(driver, BM, BN, group_m, shapes):
    inp = f"{len(shapes)} {BM} {BN} {group_m} " + " ".join(f"{m} {n}" for m, n in shapes)
    out = subprocess.run([driver], input=inp, capture_output=True, text=True, check=True)
    lines = out.stdout.split("\n")
    grid = int(lines[0])
    rows = [tuple(map(int, l.split())) for l in lines[1:1 + grid]]
    assert len(rows) == grid and grid % 8 == 0
    return rows


def check(rows, BM, BN, shapes):
    seen = collections.Counter(r for r in rows if r != (-1,))
    for q, (m, n) in enumerate(shapes):
        tm, tn = -(-m // BM), -(-n // BN)
        want = {(q, i, j) for i in range(tm) for j in range(tn)}
        got = {k for k in seen if k[0] == q}
        assert got == want, f"problem {q}: tiles missing or extra"
    assert all(c == 1 for c in seen.values()), "a tile computed twice"
    # equal share per XCD: per problem, the XCD counts differ by at most one
    # whole per-XCD share boundary (the last XCDs may come up short)
    for q, (m, n) in enumerate(shapes):
        total = -(-m // BM) * -(-n // BN)
        per = -(-total // 8)
        counts = [sum(1 for b, r in enumerate(rows) if b % 8 == x and r[0] == q and r != (-1,))
                  for x in range(8)]
        assert sum(counts) == total
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
