"""The cached step's launch shape (bca_decode_layout, host only): waves per workgroup and the
query tiles of 384, 256 and 128 rows per (batch, head, key range), as include/bca.h states them.

* The tiles cover every query row, and every tile holds at least one row.
* The width rules: unsplit shares that are whole per XCD take 12-wave workgroups once 384-row
  tiles fill one round of the CUs; other shapes once they give every CU two workgroups; 4-wave
  ones, in 128-row tiles, otherwise.
* The mix equals a replay written here from the header's description: for each candidate, a list
  schedule of one XCD's tiles (384-row tiles first, then 256, then 128) on its CUs, each tile
  priced at its busiest SIMD's step time (1, 0.88, 0.66 for 3, 2, 1 waves with rows) + 0.01.
  With a bf16 cache, the two-launch plan (384-row tiles, then 256-row tail tiles, each phase in
  whole rounds at 1.01 and 0.737 per tile + 0.02) replaces it when at least 3% shorter.
* Bad arguments are BCA_ERR_ARG.
"""
import heapq

import pytest

bca = pytest.importorskip("block_causal_attention_amd")
from block_causal_attention_amd import _lib  # noqa: E402


def cdiv(a, b):
    return -(-a // b)


def replay(n, nb, cx):
    quarters = cdiv(n, 128)

    def cost(row0, rows):
        busiest = cdiv(cdiv(min(rows, n - row0), 32), 4)
        return {3: 1.0, 2: 0.88, 1: 0.66}[min(busiest, 3)] + 0.01

    best = None  # (span, (n3, n2, n1))
    for n2 in range(17):
        for n1 in range(3):
            n3 = max(0, cdiv(quarters - 2 * n2 - n1, 3))
            covered = 384 * n3 + 256 * n2 + 128 * n1
            last = 128 if n1 else 256 if n2 else 384
            if n3 + n2 + n1 == 0 or covered < n or covered - last >= n:
                continue
            tiles = [(384 * t, 384) for _ in range(nb) for t in range(n3)]
            tiles += [(384 * n3 + 256 * t, 256) for _ in range(nb) for t in range(n2)]
            tiles += [(384 * n3 + 256 * n2 + 128 * t, 128) for _ in range(nb) for t in range(n1)]
            free = [0.0] * cx
            span = 0.0
            for row0, rows in tiles:          # a free CU takes the next tile
                done = heapq.heappop(free) + cost(row0, rows)
                heapq.heappush(free, done)
                span = max(span, done)
            if best is None or span < best[0] - 1e-9:
                best = (span, (n3, n2, n1))
    return best


def two_launch(n, nb, cx):
    """384-row tiles in the 12-wave kernel, then 256-row tail tiles, each phase in whole rounds:
    (span, n3, n_tail) of the best n3 (fewest on ties)."""
    best = None
    n3 = 0
    while 384 * n3 < n:
        n_tail = cdiv(n - 384 * n3, 256)
        span = cdiv(nb * n3, cx) * 1.01 + (0.02 if n3 else 0.0) + cdiv(nb * n_tail, cx) * 0.737
        if best is None or span < best[0] - 1e-9:
            best = (span, n3, n_tail)
        n3 += 1
    return best


def covers(n, tiles):
    heights = [384] * tiles[0] + [256] * tiles[1] + [128] * tiles[2]
    starts = [sum(heights[:i]) for i in range(len(heights))]
    return sum(heights) >= n and all(s < n for s in starts)


SHAPES = [(n, g, s, c) for n in (1, 100, 384, 385, 777, 1024, 2048, 3072, 3356, 3615, 4000, 4096,
                                 5120, 8192, 16384, 40000)
          for g in (1, 8, 24, 32, 64, 256) for s in (1, 3) for c in (256, 304, 80)]


@pytest.mark.parametrize("fmt", [0, 1])
@pytest.mark.parametrize("n,bh,n_split,cus", SHAPES)
def test_layout_covers_rows_and_follows_the_rules(n, bh, n_split, cus, fmt):
    waves, t3, t2, t1, tail = bca.decode_layout(n, bh, n_split, fmt, cus)
    t12, n256 = cdiv(n, 384), cdiv(n, 256)
    mixable = n_split == 1 and bh % 8 == 0 and cus % 8 == 0
    wide = t12 * bh >= cus if mixable else t12 * bh * n_split >= 2 * cus
    if mixable and not wide and fmt == 0:
        # under one round of 384-row tiles over a bf16 cache: one round of 12-wave workgroups
        # when 256-row tiles would need a second, all rows in the 8-wave launch when its tiles
        # fill more than half of the CUs, else 4-wave workgroups
        if n256 * bh > cus:
            assert (waves, t3, t2, t1, tail) == (12, t12, 0, 0, 0)
            return
        if 2 * n256 * bh > cus:
            assert (waves, t3, t2, t1, tail) == (12, 0, 0, 0, n256)
            return
    assert waves == (12 if wide else 4)
    if waves == 4:
        assert (t3, t2, t1, tail) == (0, 0, cdiv(n, 128), 0)
        return
    if not mixable:
        assert (t3, t2, t1, tail) == (t12, 0, 0, 0)
        return
    span, mix = replay(n, bh // 8, cus // 8)
    two = two_launch(n, bh // 8, cus // 8)
    if fmt == 0 and bh // 8 >= 4 and two is not None and two[0] < 0.97 * span:
        assert (t3, t2, t1, tail) == (two[1], 0, 0, two[2])
        assert 384 * t3 < n <= 384 * t3 + 256 * tail and 384 * t3 + 256 * (tail - 1) < n
    else:
        assert (t3, t2, t1, tail) == mix + (0,)
        assert covers(n, mix)


def test_headline_shapes():
    # the CFG cached step (B = 2, H = 32, N = 4,096) on 256 CUs, bf16 cache: two rounds of
    # 384-row tiles, then one round of 256-row tiles in the 8-wave tail launch; over an FP8
    # cache the same rows in one launch (384- and 256-row tiles)
    assert bca.decode_layout(4096, 64, 1, 0, 256) == (12, 8, 0, 0, 4)
    assert bca.decode_layout(4096, 64, 1, 1, 256) == (12, 8, 4, 0, 0)
    assert bca.decode_layout(16384, 64, 1, 0, 256) == (12, 40, 4, 0, 0)
    # under one round of 384-row tiles: the 512^2 target (unsplit and split) keeps 4-wave
    # workgroups; over a bf16 cache N = 2,048 at B = 1 runs all its rows in the 8-wave launch,
    # N = 2,304 one round of 12-wave workgroups; an FP8 cache keeps the 4-wave launch
    assert bca.decode_layout(1024, 32, 1, 0, 256) == (4, 0, 0, 8, 0)
    assert bca.decode_layout(1024, 32, 3, 0, 256) == (4, 0, 0, 8, 0)
    assert bca.decode_layout(2048, 32, 1, 0, 256) == (12, 0, 0, 0, 8)
    assert bca.decode_layout(2304, 32, 1, 0, 256) == (12, 6, 0, 0, 0)
    assert bca.decode_layout(2048, 32, 1, 1, 256) == (4, 0, 0, 16, 0)


@pytest.mark.parametrize("args", [(0, 64, 1, 0, 256), (4096, 0, 1, 0, 256), (4096, 64, 0, 0, 256),
                                  (4096, 64, 1, 0, -1), (2**31, 64, 1, 0, 256),
                                  (4096, 2**31, 1, 0, 256), (4096, 2**30, 2, 0, 256),
                                  (4096, 64, 1, 3, 256)])
def test_bad_arguments(args):
    with pytest.raises(bca.BcaError) as e:
        bca.decode_layout(*args)
    assert e.value.status == _lib.BCA_ERR_ARG
