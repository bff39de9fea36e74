"""Pins of the oracle's batch-of-sequences attention (CPU only).

* A dense construction over the whole row axis: one softmax per row over ALL rows, with the rule
  in words (same sequence, and key at or before the query or in the query's image block) as the
  mask.  Padding rows between sequences are never visible.  It must equal the per-sequence
  oracle, packed or with gaps.
* A batch of one is the single-sequence oracle.
* Sequences are independent: rewriting every row outside sequence b leaves b unchanged, bit for
  bit.
* Per-branch prefix caches laid end to end and the batched cached step: each branch's target
  rows equal its rows of the dense construction; one branch is the plain cached step.
Planted mistakes (the packed batch treated as one sequence; a cache read one row off) are caught.
"""
import numpy as np
import pytest

import bca_workloads as W
from oracle import bca_oracle as O


def dense_rule_over_rows(q, k, v, ids_list, row_start):
    R, H, D = q.shape
    seq = np.full(R, -1)
    idv = np.zeros(R, dtype=np.int64)
    loc = np.zeros(R, dtype=np.int64)
    for b, ids in enumerate(ids_list):
        a = row_start[b]
        seq[a:a + len(ids)] = b
        idv[a:a + len(ids)] = ids
        loc[a:a + len(ids)] = np.arange(len(ids))
    out = {}
    sc = 1 / np.sqrt(D)
    for b, ids in enumerate(ids_list):
        rows = np.arange(row_start[b], row_start[b] + len(ids))
        res = np.zeros((len(ids), H, D))
        for r_i, i in enumerate(rows):
            vis = np.array([seq[j] == b and (loc[i] >= loc[j] or (idv[i] >= 0 and idv[i] == idv[j]))
                            for j in range(R)])
            for h in range(H):
                s = q[i, h] @ k[:, h].T * sc
                s = np.where(vis, s, -np.inf)
                p = np.exp(s - s.max())
                res[r_i, h] = (p / p.sum()) @ v[:, h]
        out[b] = res
    return out


def batch(seed, lens, gaps=None):
    rng = np.random.default_rng(seed)
    ids_list = [W.random_layout(rng, n, max_seg=max(1, n // 3)) for n in lens]
    if gaps is None:
        starts = O.packed_row_starts(lens)
    else:
        starts = np.cumsum([0] + [n + g for n, g in zip(lens, gaps)])[:-1]
    R = int(starts[-1] + lens[-1] + 3)
    q, k, v = (rng.standard_normal((R, 2, 128)) for _ in range(3))
    return q, k, v, ids_list, starts


@pytest.mark.parametrize("gaps", [None, [3, 0, 5]])
def test_dense_rule_over_all_rows(gaps):
    q, k, v, ids_list, starts = batch(1, [9, 14, 6], gaps)
    want = dense_rule_over_rows(q, k, v, ids_list, starts)
    got = O.attention_varlen(q, k, v, ids_list, starts)
    for b in want:
        np.testing.assert_allclose(got[b], want[b], rtol=0, atol=1e-12)


def test_batch_of_one_is_the_single_sequence():
    q, k, v, ids_list, starts = batch(2, [40])
    got = O.attention_varlen(q, k, v, ids_list, starts)[0]
    want = O.attention(q[None, :40], k[None, :40], v[None, :40], ids_list[0])[0]
    assert np.array_equal(got, want)


def test_sequences_are_independent():
    q, k, v, ids_list, starts = batch(3, [20, 31, 12], [2, 4, 0])
    base = O.attention_varlen(q, k, v, ids_list, starts)
    for b in range(3):
        a, n = starts[b], len(ids_list[b])
        q2, k2, v2 = q.copy(), k.copy(), v.copy()
        outside = np.ones(q.shape[0], bool)
        outside[a:a + n] = False
        for t in (q2, k2, v2):
            t[outside] = 50.0
        assert np.array_equal(O.attention_varlen(q2, k2, v2, ids_list, starts)[b], base[b])


def test_planted_mistake_one_long_sequence_is_caught():
    q, k, v, ids_list, starts = batch(4, [7, 9, 5])
    # wrong: the packed batch as one sequence (later sequences see earlier ones)
    merged = np.concatenate([np.where(i >= 0, i + 100 * b, -1) for b, i in enumerate(ids_list)])
    R = sum(len(i) for i in ids_list)
    wrong = O.attention(q[None, :R], k[None, :R], v[None, :R], merged)[0]
    want = dense_rule_over_rows(q, k, v, ids_list, starts)
    with pytest.raises(AssertionError):
        for b in want:
            np.testing.assert_allclose(wrong[starts[b]:starts[b] + len(ids_list[b])], want[b],
                                       rtol=0, atol=1e-9)


def cfg_branches(seed, prompts, target):
    """Two or more CFG-like branches: [text p][image 6][text 2][image target] with prompts of
    different lengths, every branch ending in its target image block."""
    ids_list = [W.block_ids_from_segments((("text", p), ("image", 6), ("text", 2),
                                           ("image", target))) for p in prompts]
    lens = [len(i) for i in ids_list]
    starts = np.cumsum([0] + [n + 2 for n in lens])[:-1]       # a gap of 2 rows between branches
    R = int(starts[-1] + lens[-1] + 1)
    rng = np.random.default_rng(seed)
    q, k, v = (rng.standard_normal((R, 2, 128)) for _ in range(3))
    return q, k, v, ids_list, starts


def test_per_branch_caches_and_cached_step_reproduce_the_prefill_rows():
    """Per-branch caches laid end to end, then the batched cached step: each branch's target rows
    must equal its prefill rows under the rule built densely over all rows (a target row of the
    last image block sees every earlier row of its branch and its whole block)."""
    q, k, v, ids_list, starts = cfg_branches(5, [7, 13, 4], 9)
    kc, vc = O.prefix_cache_varlen(k, v, ids_list, starts)
    # the cache rows, position by position
    r = 0
    for b, ids in enumerate(ids_list):
        P = int(np.flatnonzero(np.asarray(ids) != ids[-1]).max()) + 1   # before the last block
        for j in range(P):
            assert np.array_equal(kc[r], k[starts[b] + j]) and np.array_equal(vc[r], v[starts[b] + j])
            r += 1
    assert r == kc.shape[0]
    # the targets, packed
    tgt = [np.arange(starts[b] + len(ids) - 9, starts[b] + len(ids)) for b, ids in enumerate(ids_list)]
    sel = np.concatenate(tgt)
    got = O.decode_varlen(q[sel], kc, vc, k[sel], v[sel], ids_list)
    want = dense_rule_over_rows(q, k, v, ids_list, starts)
    for b, ids in enumerate(ids_list):
        np.testing.assert_allclose(got[b], want[b][len(ids) - 9:], rtol=0, atol=1e-12)


def test_batched_cached_step_of_one_branch_is_the_plain_cached_step():
    q, k, v, ids_list, starts = cfg_branches(6, [11], 8)
    P = len(ids_list[0]) - 8
    got = O.decode_varlen(q[P:P + 8], k[:P], v[:P], k[P:P + 8], v[P:P + 8], ids_list)[0]
    want = O.decode(q[None, P:P + 8], k[None, :P], v[None, :P], k[None, P:P + 8], v[None, P:P + 8])[0]
    assert np.array_equal(got, want)


def test_planted_mistake_cache_rows_off_by_one_is_caught():
    q, k, v, ids_list, starts = cfg_branches(7, [5, 9], 7)
    kc, vc = O.prefix_cache_varlen(k, v, ids_list, starts)
    sel = np.concatenate([np.arange(starts[b] + len(i) - 7, starts[b] + len(i))
                          for b, i in enumerate(ids_list)])
    want = dense_rule_over_rows(q, k, v, ids_list, starts)
    # wrong: every cache row read one row off (c_b off by one)
    wrong = O.decode_varlen(q[sel], np.roll(kc, 1, axis=0), np.roll(vc, 1, axis=0), k[sel], v[sel],
                            ids_list)
    with pytest.raises(AssertionError):
        for b, ids in enumerate(ids_list):
            np.testing.assert_allclose(wrong[b], want[b][len(ids) - 7:], rtol=0, atol=1e-9)
