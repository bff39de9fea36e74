"""Pins of the CPU oracle against what the pages and the mathematics fix (CPU only).

Each check is written so that it does not reuse the oracle's own formula:

* the rule as the pages state it in words (text sees keys at or before itself; an image row sees
  everything before its block and its whole block, nothing after the block end), brute-forced
  over every run layout up to S = 8;
* the per-segment construction of the default processor (text segment: bottom-right aligned
  causal triangle; image segment: all earlier keys plus its own block);
* the pages' worked 3-query / 5-prefix example (tests/golden/bottom_right_causal_3x8.txt);
* closed forms (Q = 0 gives the mean of the visible values) and reductions to torch's
  scaled_dot_product_attention (unmasked, causal, piecewise segment calls);
* prefix invariance and decode == prefill rows;
* the pages' cache-size figures (tests/golden/cache_payload.txt).

The "planted mistake" tests plant plausible bugs in a copy of the oracle's rule on the CPU and
check that these pins catch every one of them.
"""
import itertools
import os

import numpy as np
import pytest
import torch

import bca_workloads as W
from oracle import bca_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------------------------------------
# helpers written independently of the oracle
# ---------------------------------------------------------------------------------------------
def all_layouts(S):
    """Every run layout of length S: runs are text or image; adjacent text runs would merge, so
    they are excluded; adjacent image runs get distinct ids."""
    out = []

    def rec(pos, prev_kind, acc):
        if pos == S:
            out.append(list(acc))
            return
        for n in range(1, S - pos + 1):
            for kind in ("text", "image"):
                if kind == "text" and prev_kind == "text":
                    continue
                rec(pos + n, kind, acc + [(kind, n)])

    rec(0, None, [])
    return [W.block_ids_from_segments(l) for l in out]


def block_of(ids, i):
    a = i
    while a > 0 and ids[a - 1] == ids[i]:
        a -= 1
    b = i + 1
    while b < len(ids) and ids[b] == ids[i]:
        b += 1
    return a, b


def rule_in_words(ids, i, j):
    """Text is strictly causal; an image row sees everything before its block and its whole block,
    and nothing after the end of its block."""
    if ids[i] < 0:
        return j <= i
    _, b = block_of(ids, i)
    return j < b


def words_mask(ids):
    S = len(ids)
    return np.array([[rule_in_words(ids, i, j) for j in range(S)] for i in range(S)], dtype=bool)


def piecewise_mask(ids):
    """One exact attention call per segment: a text segment [a, b) uses ones(b - a, b).tril(a)
    (bottom-right aligned: kv_len - q_len = a); an image segment uses ones(b - a, b)."""
    S = len(ids)
    m = np.zeros((S, S), dtype=bool)
    a = 0
    while a < S:
        _, b = block_of(ids, a)
        q_len, kv_len = b - a, b
        rows = np.tril(np.ones((q_len, kv_len), dtype=bool), kv_len - q_len) if ids[a] < 0 else \
            np.ones((q_len, kv_len), dtype=bool)
        m[a:b, :b] = rows
        a = b
    return m


def hi_closed_form(ids):
    """Row key limit from the segment structure: i + 1 for text, block end for image."""
    out = np.empty(len(ids), dtype=np.int64)
    for i in range(len(ids)):
        out[i] = i + 1 if ids[i] < 0 else block_of(ids, i)[1]
    return out


def load_golden_bits(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append([c == "1" for c in line])
    return np.array(rows, dtype=bool)


def rand_f64(rng, shape):
    return rng.standard_normal(shape)


# ---------------------------------------------------------------------------------------------
# pin checks, parameterised by the mask function so that planted mistakes can be fed in
# ---------------------------------------------------------------------------------------------
def check_rule_in_words(mask_fn, max_s=7):
    for S in range(1, max_s + 1):
        for ids in all_layouts(S):
            assert np.array_equal(mask_fn(ids), words_mask(ids)), ids


def check_piecewise(mask_fn, max_s=7):
    for S in range(1, max_s + 1):
        for ids in all_layouts(S):
            assert np.array_equal(mask_fn(ids), piecewise_mask(ids)), ids


def check_worked_case(mask_fn):
    golden = load_golden_bits("bottom_right_causal_3x8.txt")
    assert golden.shape == (3, 8)
    # all-text prefix of 5, and a prefix holding an image block of 4 after one text token
    for ids in (np.full(8, -1, dtype=np.int32), np.array([-1, 0, 0, 0, 0, -1, -1, -1], np.int32)):
        m = mask_fn(ids)
        assert np.array_equal(m[5:8, :], golden)
        # the top-left aligned variant the pages call wrong must differ
        assert not np.array_equal(m[5:8, :], np.tril(np.ones((3, 8), dtype=bool), 0))


def check_consequences(mask_fn):
    """The consequences the pages list, on the tiny workload's layout and on adjacent images."""
    ids = W.TINY.block_ids()  # [text 12][ref 64][text 6][target 64]
    m = mask_fn(ids)
    ref = slice(12, 76)
    later_text = slice(76, 82)
    target = slice(82, 146)
    assert not m[ref, 76:].any()                    # ref sees no later text, image or target
    assert m[ref, :76].all()                        # ... but all earlier text and itself
    assert m[later_text, ref].all()                 # later text reads the earlier reference
    assert m[target, :].all()                       # target reads prefix and whole target
    assert not m[:82, 82:].any()                    # the prefix never sees the target
    adj = W.block_ids_from_segments([("text", 3), ("image", 5), ("image", 4)])
    ma = mask_fn(adj)
    assert not ma[3:8, 8:].any()                    # earlier image can't read the adjacent one
    assert ma[8:, :].all()                          # the later one reads the earlier one


ALL_MASK_PINS = (check_rule_in_words, check_piecewise, check_worked_case, check_consequences)


# ---------------------------------------------------------------------------------------------
# the pins, run on the oracle
# ---------------------------------------------------------------------------------------------
def test_mask_equals_rule_in_words_every_layout():
    check_rule_in_words(O.visibility_mask, max_s=8)


def test_mask_equals_piecewise_construction_every_layout():
    check_piecewise(O.visibility_mask, max_s=8)


def test_worked_case_bottom_right_alignment():
    check_worked_case(O.visibility_mask)


def test_stated_consequences():
    check_consequences(O.visibility_mask)


def test_random_layouts_up_to_300():
    rng = np.random.default_rng(7)
    for _ in range(12):
        S = int(rng.integers(50, 301))
        ids = W.random_layout(rng, S)
        m = O.visibility_mask(ids)
        assert np.array_equal(m, piecewise_mask(ids))
        hi = O.row_key_limits(ids)
        assert np.array_equal(hi, hi_closed_form(ids))
        assert (np.diff(hi) >= 0).all() and (hi >= np.arange(1, S + 1)).all()


def test_block_id_validation():
    with pytest.raises(O.OracleInputError):
        O.validate_block_ids([-1, -2, 0])
    with pytest.raises(O.OracleInputError):
        O.validate_block_ids([0, 0, -1, 0])          # id reused in a second run
    with pytest.raises(O.OracleInputError):
        O.validate_block_ids([])
    O.validate_block_ids([3, 3, 1, 1, -1, 0])        # ids need not be increasing
    assert O.prefix_split([-1, -1, 0, 0, 1, 1, 1]) == (4, 3, True)
    assert O.prefix_split([-1, 0, 0, -1]) == (3, 1, False)


def test_q_zero_gives_mean_of_visible_values():
    """With Q = 0 every visible logit is 0, so each output row is the plain mean of V over the
    visible keys [0, hi(i))."""
    rng = np.random.default_rng(11)
    for ids in (W.TINY.block_ids(), W.random_layout(rng, 97)):
        S = len(ids)
        v = rand_f64(rng, (1, S, 2, 128))
        q = np.zeros_like(v)
        k = rand_f64(rng, (1, S, 2, 128))
        o = O.attention(q, k, v, ids)
        hi = hi_closed_form(ids)
        for i in range(S):
            np.testing.assert_allclose(o[0, i], v[0, :hi[i]].mean(axis=0), rtol=0, atol=1e-13)


def _sdpa(q, k, v, mask=None, causal=False, scale=None):
    """torch's reference attention on CPU in float64; q/k/v given as [S, D]."""
    t = lambda x: torch.from_numpy(np.ascontiguousarray(x))[None, None]
    m = None if mask is None else torch.from_numpy(mask)[None, None]
    return torch.nn.functional.scaled_dot_product_attention(
        t(q), t(k), t(v), attn_mask=m, is_causal=causal, scale=scale)[0, 0].numpy()


def test_single_image_block_is_unmasked_attention():
    rng = np.random.default_rng(12)
    S = 70
    q, k, v = (rand_f64(rng, (1, S, 1, 128)) for _ in range(3))
    o = O.attention(q, k, v, np.zeros(S, np.int32))
    ref = _sdpa(q[0, :, 0], k[0, :, 0], v[0, :, 0])
    np.testing.assert_allclose(o[0, :, 0], ref, rtol=0, atol=1e-12)


def test_all_text_is_causal_attention():
    rng = np.random.default_rng(13)
    S = 70
    q, k, v = (rand_f64(rng, (1, S, 1, 128)) for _ in range(3))
    o = O.attention(q, k, v, np.full(S, -1, np.int32), scale=0.3)
    ref = _sdpa(q[0, :, 0], k[0, :, 0], v[0, :, 0], causal=True, scale=0.3)
    np.testing.assert_allclose(o[0, :, 0], ref, rtol=0, atol=1e-12)


def test_equals_piecewise_segment_calls():
    """The default processor's procedure: one exact attention call per segment over keys
    [0, segment end), text segments with the bottom-right aligned causal mask."""
    rng = np.random.default_rng(14)
    for S in (40, 131):
        ids = W.random_layout(rng, S, max_seg=25)
        q, k, v = (rand_f64(rng, (2, S, 2, 128)) for _ in range(3))
        o = O.attention(q, k, v, ids)
        for b in range(2):
            for h in range(2):
                a = 0
                while a < S:
                    _, e = block_of(ids, a)
                    mask = None
                    if ids[a] < 0:
                        mask = torch.ones(e - a, e, dtype=torch.bool).tril(a).numpy()
                    ref = _sdpa(q[b, a:e, h], k[b, :e, h], v[b, :e, h], mask=mask)
                    np.testing.assert_allclose(o[b, a:e, h], ref, rtol=0, atol=1e-12)
                    a = e


def test_prefix_rows_invariant_to_target_perturbation():
    """Prefix states cannot depend on the target: perturbing Q/K/V at positions >= P leaves the
    prefix rows bit-for-bit unchanged."""
    rng = np.random.default_rng(15)
    ids = W.TINY.block_ids()
    P, N, ok = O.prefix_split(ids)
    assert (P, N, ok) == (82, 64, True)
    q, k, v = (rand_f64(rng, (1, 146, 2, 128)) for _ in range(3))
    o1 = O.attention(q, k, v, ids)
    q2, k2, v2 = q.copy(), k.copy(), v.copy()
    for x in (q2, k2, v2):
        x[:, P:] = 100.0 * rand_f64(rng, x[:, P:].shape)
    o2 = O.attention(q2, k2, v2, ids)
    assert np.array_equal(o1[:, :P], o2[:, :P])
    assert not np.array_equal(o1[:, P:], o2[:, P:])


def test_decode_equals_prefill_target_rows():
    rng = np.random.default_rng(16)
    for ids in (W.TINY.block_ids(), W.block_ids_from_segments([("image", 9), ("image", 30)])):
        S = len(ids)
        P, N, ok = O.prefix_split(ids)
        assert ok
        q, k, v = (rand_f64(rng, (2, S, 2, 128)) for _ in range(3))
        full = O.attention(q, k, v, ids)
        kc, vc = O.prefix_cache(k, v, ids)
        dec = O.decode(q[:, P:], kc, vc, k[:, P:], v[:, P:])
        np.testing.assert_allclose(dec, full[:, P:], rtol=0, atol=1e-12)


def test_prefix_cache_is_a_copy():
    rng = np.random.default_rng(17)
    ids = W.TINY.block_ids()
    k, v = rand_f64(rng, (1, 146, 2, 128)), rand_f64(rng, (1, 146, 2, 128))
    kc, vc = O.prefix_cache(k, v, ids)
    assert kc.shape == (1, 82, 2, 128) and np.array_equal(kc, k[:, :82])
    assert not np.shares_memory(kc, k) and not np.shares_memory(vc, v)


def test_cache_payload_figures():
    with open(os.path.join(GOLDEN, "cache_payload.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                L, B, P, H, D, bps, want = (int(x) for x in line.split())
                assert O.prefix_cache_bytes(L, B, P, H, D, bps) == want
    assert O.prefix_cache_bytes(32, 1, 1, 32, 128, 2) == 512 * 1024


def test_plan_from_mask_brute_force():
    rng = np.random.default_rng(18)
    for S in (1, 5, 33, 64, 65, 150):
        ids = W.random_layout(rng, S, max_seg=20)
        wm = words_mask(ids)
        for bm in (4, 16, 64):
            plan = O.plan_from_mask(ids, bm)
            hi = np.array([1 + max(j for j in range(S) if wm[i, j]) for i in range(S)])
            assert np.array_equal(plan["row_limit"], hi)
            nt = (S + bm - 1) // bm
            # tiles end at the sequence's end: only the first may be partial, and together they
            # cover every row once
            covered = []
            for t in range(nt):
                rows = range(max(0, S - (nt - t) * bm), S - (nt - 1 - t) * bm)
                assert plan["tile_first"][t] == S - (nt - t) * bm
                assert len(rows) == bm or (t == 0 and 0 < len(rows) < bm)
                covered.extend(rows)
                full = min(hi[r] for r in rows)
                end = max(hi[r] for r in rows)
                assert plan["kv_full"][t] == full and plan["kv_end"][t] == end
                # every key below kv_full is visible to every row; none at or past kv_end is
                assert all(wm[r, :full].all() and not wm[r, end:].any() for r in rows)
            assert covered == list(range(S))
            keys = [(-plan["kv_end"][t], t) for t in plan["order"]]
            assert keys == sorted(keys) and sorted(plan["order"]) == list(range(nt))
            assert plan["useful_pairs"] == wm.sum()


@pytest.mark.parametrize("name", ["tiny", "t2i_1024", "edit_2ref", "long_4ref"])
def test_workload_useful_pairs_closed_form(name):
    """Sum of row key limits against a closed form over the segments: a text run [a, b) adds
    sum(i + 1), an image run adds (b - a) * b."""
    lay = W.WORKLOADS[name]
    ids = lay.block_ids()
    total, a = 0, 0
    for kind, n in lay.segments:
        b = a + n
        total += (a + 1 + b) * n // 2 if kind == "text" else n * b
        a = b
    assert O.row_key_limits(ids).sum() == total


# ---------------------------------------------------------------------------------------------
# planted mistakes: every one must be caught by at least one pin
# ---------------------------------------------------------------------------------------------
def _mut_top_left(ids):
    """Text segment rows aligned top-left: a text row sees only keys up to its index within the
    segment (the alignment the pages call wrong)."""
    ids = np.asarray(ids)
    S = len(ids)
    m = O.visibility_mask(ids)
    for i in range(S):
        if ids[i] < 0:
            a, _ = block_of(ids, i)
            m[i, :] = np.arange(S) <= (i - a)
    return m


def _mut_text_same_block(ids):
    """'same block' without requiring an image id: all text mutually visible."""
    ids = np.asarray(ids)
    i = np.arange(len(ids))[:, None]
    j = np.arange(len(ids))[None, :]
    return (i >= j) | (ids[:, None] == ids[None, :])


def _mut_strict_causal(ids):
    ids = np.asarray(ids)
    i = np.arange(len(ids))[:, None]
    j = np.arange(len(ids))[None, :]
    return (i > j) | ((ids[:, None] >= 0) & (ids[:, None] == ids[None, :]))


def _mut_image_sees_next_run(ids):
    """An image row also sees the run right after its block."""
    ids = np.asarray(ids)
    m = O.visibility_mask(ids)
    for i in range(len(ids)):
        if ids[i] >= 0:
            _, b = block_of(ids, i)
            if b < len(ids):
                _, b2 = block_of(ids, b)
                m[i, :b2] = True
    return m


def _mut_adjacent_images_merged(ids):
    """Adjacent image blocks treated as one block."""
    ids = np.asarray(ids).copy()
    merged = np.where(ids >= 0, 0, -1)
    # keep distinct ids only across text gaps
    cur, out, prev = -1, [], -1
    for x in merged:
        if x >= 0 and prev < 0:
            cur += 1
        out.append(cur if x >= 0 else -1)
        prev = x
    return O.visibility_mask(np.array(out))


@pytest.mark.parametrize("mutant", [_mut_top_left, _mut_text_same_block, _mut_strict_causal,
                                    _mut_image_sees_next_run, _mut_adjacent_images_merged])
def test_planted_mask_mistakes_are_caught(mutant):
    caught = 0
    for pin in ALL_MASK_PINS:
        try:
            pin(mutant)
        except AssertionError:
            caught += 1
    assert caught >= 1, f"{mutant.__name__} passed every pin"


def test_planted_softmax_mistakes_are_caught(monkeypatch):
    """Numeric mistakes planted in the oracle's softmax attention: a dropped scale, the row max
    not subtracted per row, and normalisation over the wrong axis."""
    rng = np.random.default_rng(19)
    S = 40
    q, k, v = (rand_f64(rng, (1, S, 1, 128)) for _ in range(3))
    ids = np.zeros(S, np.int32)
    ref = _sdpa(q[0, :, 0], k[0, :, 0], v[0, :, 0])

    def no_scale(qq, kk, vv, scale, mask):
        s = qq @ kk.T
        p = np.exp(s - s.max(axis=1, keepdims=True))
        return (p / p.sum(axis=1, keepdims=True)) @ vv

    def wrong_axis(qq, kk, vv, scale, mask):
        s = (qq @ kk.T) * scale
        p = np.exp(s - s.max())
        return (p / p.sum(axis=0, keepdims=True)) @ vv

    for bad in (no_scale, wrong_axis):
        monkeypatch.setattr(O, "_softmax_attention", bad)
        o = O.attention(q, k, v, ids)
        assert not np.allclose(o[0, :, 0], ref, rtol=0, atol=1e-6)
    monkeypatch.undo()
    np.testing.assert_allclose(O.attention(q, k, v, ids)[0, :, 0], ref, rtol=0, atol=1e-12)
