"""The cached step's launch shape (bca_decode_layout, host only): waves per workgroup and the
query tiles of 384, 256 and 128 rows per (batch, head, key range) group, as include/bca.h
states them.

* The tiles cover every query row, and every tile holds at least one row.
* 12-wave workgroups exactly where 384-row tiles give every CU two workgroups; 4-wave ones,
  in 128-row tiles, otherwise.
* The mix equals a replay written here from the header's description: for each candidate, a list
  schedule of one XCD's tiles (384-row tiles first, then 256, then 128) on its CUs, each tile
  priced at its busiest SIMD's step time (1, 0.88, 0.66 for 3, 2, 1 waves with rows) + 0.01.
* Shares that are not whole per XCD keep 384-row tiles only; bad arguments are BCA_ERR_ARG.
"""
import heapq

import pytest

bca = pytest.importorskip("block_causal_attention_amd")
from block_causal_attention_amd import _lib  # noqa: E402


def replay(n, nb, cx):
    quarters = -(-n // 128)

    def cost(row0, rows):
        live = min(rows, n - row0)
        busiest = -(-(-(-live // 32)) // 4)
        return {3: 1.0, 2: 0.88, 1: 0.66}[min(busiest, 3)] + 0.01

    best = None
    for n2 in range(5):
        for n1 in range(2):
            n3 = max(0, -(-(quarters - 2 * n2 - n1) // 3))
            covered = 384 * n3 + 256 * n2 + 128 * n1
            last = 128 if n1 else 256 if n2 else 384
            if n3 + n2 + n1 == 0 or covered < n or covered - last >= n:
                continue
            free = [0.0] * cx
            span = 0.0
            base = 0
            for count, height in ((n3, 384), (n2, 256), (n1, 128)):
                for _ in range(nb):
                    for t in range(count):
                        done = heapq.heappop(free) + cost(base + height * t, height)
                        heapq.heappush(free, done)
                        span = max(span, done)
                base += height * count
            if best is None or span < best[0] - 1e-9:
                best = (span, (n3, n2, n1))
    return best[1]


def covers(n, tiles):
    heights = [384] * tiles[0] + [256] * tiles[1] + [128] * tiles[2]
    starts = [sum(heights[:i]) for i in range(len(heights))]
    return sum(heights) >= n and all(s < n for s in starts)


SHAPES = [(n, g, c) for n in (1, 100, 384, 385, 777, 1024, 3356, 3615, 4000, 4096, 8192, 12288,
                              16384, 40000)
          for g in (1, 8, 24, 32, 64, 256, 1000) for c in (256, 304, 80)]


@pytest.mark.parametrize("n,groups,cus", SHAPES)
def test_layout_covers_rows_and_follows_the_rules(n, groups, cus):
    waves, t3, t2, t1 = bca.decode_layout(n, groups, cus)
    wide = -(-n // 384) * groups >= 2 * cus
    assert waves == (12 if wide else 4)
    if waves == 4:
        assert (t3, t2, t1) == (0, 0, -(-n // 128))
        return
    assert covers(n, (t3, t2, t1))
    if groups % 8 == 0 and cus % 8 == 0:
        assert (t3, t2, t1) == replay(n, groups // 8, cus // 8)
    else:
        assert (t3, t2, t1) == (-(-n // 384), 0, 0)


def test_headline_shapes():
    # the CFG cached step (B = 2, H = 32, N = 4,096) on 256 CUs: two rounds of 384-row tiles and
    # one of 256-row tiles; at B = 1 the grid is small and takes 4-wave workgroups
    assert bca.decode_layout(4096, 64, 256) == (12, 8, 4, 0)
    assert bca.decode_layout(4096, 32, 256) == (4, 0, 0, 32)
    assert bca.decode_layout(16384, 64, 256) == (12, 40, 4, 0)
    assert bca.decode_layout(3356, 64, 256) == (12, 6, 4, 1)


@pytest.mark.parametrize("args", [(0, 64, 256), (4096, 0, 256), (4096, 64, -1), (2**31, 64, 256),
                                  (4096, 2**31, 256)])
def test_bad_arguments(args):
    with pytest.raises(bca.BcaError) as e:
        bca.decode_layout(*args)
    assert e.value.status == _lib.BCA_ERR_ARG
