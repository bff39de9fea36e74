"""Pins of the oracle's Q/K prologue (per-head RMS norm, three-axis RoPE, positions), CPU only.

Each function is pinned to something other than its own formula:
* positions: the rule in words (text advances all three coordinates together, an image keeps
  the frame reached so far and a zero-centred grid) checked token by token, and the pages' stated
  consequence that moving a reference later changes its frame but not its height/width grid;
* angles: closed forms of the frequencies (frame pair k turns by 10^(-k/2) per unit, height and
  width pair k by 10^(-k/7), since 10000^(2/16) = 10^(1/2) and 10000^(2/56) = 10^(1/7)), seen
  through unit vectors, which also fixes the pairing and the section boundaries;
* rotation: length preserved per pair, and the relative-position property (a dot product of two
  rotated vectors depends on the positions only through their difference on every axis);
* RMS norm: unit mean square for w = 1, eps = 0; invariance to positive scaling; a constant row.
Planted mistakes (rotate-half pairing, swapped sections, frequencies over d instead of d/2,
text that does not advance, an uncentred grid, the frame advancing inside an image) are caught.
"""
import math

import numpy as np
import pytest

import bca_workloads as W
from oracle import bca_oracle as O


# ---------------------------------------------------------------------------------------------
# positions
# ---------------------------------------------------------------------------------------------
def check_positions(pos_fn):
    ids = W.block_ids_from_segments([("text", 5), ("image", 12), ("text", 3), ("image", 4),
                                     ("image", 9), ("text", 2)])
    hw = [(3, 4), (2, 2), (3, 3)]
    pos = pos_fn(ids, hw)
    assert pos.shape == (len(ids), 3)
    # text: (c, c, c), consecutive text tokens advance by one
    for i in range(5):
        assert tuple(pos[i]) == (i, i, i)
    # first image 3 x 4: frame 5 (five text tokens before it), grid centred on zero, row-major
    blk = pos[5:17]
    assert (blk[:, 0] == 5).all()
    assert [tuple(x) for x in blk[:, 1:]] == [(h - 1, w - 2) for h in range(3) for w in range(4)]
    # text after it continues at 6
    assert [tuple(x) for x in pos[17:20]] == [(6, 6, 6), (7, 7, 7), (8, 8, 8)]
    # two adjacent images: frames 9 and 10, each with its own centred grid
    assert (pos[20:24, 0] == 9).all() and (pos[24:33, 0] == 10).all()
    assert [tuple(x) for x in pos[20:24, 1:]] == [(-1, -1), (-1, 0), (0, -1), (0, 0)]
    assert [tuple(x) for x in pos[24:33, 1:]] == [(h - 1, w - 1) for h in range(3) for w in range(3)]
    assert [tuple(x) for x in pos[33:35]] == [(11, 11, 11), (12, 12, 12)]


def test_positions_follow_the_rule():
    check_positions(O.rope_positions)


def test_moving_a_reference_later_changes_only_its_frame():
    a = W.block_ids_from_segments([("text", 4), ("image", 16), ("text", 2), ("image", 16)])
    b = W.block_ids_from_segments([("text", 9), ("image", 16), ("text", 2), ("image", 16)])
    pa, pb = O.rope_positions(a), O.rope_positions(b)
    ra, rb = pa[4:20], pb[9:25]
    assert (rb[:, 0] - ra[:, 0] == 5).all()          # frame moved with the reference
    assert np.array_equal(ra[:, 1:], rb[:, 1:])      # its height/width grid did not
    assert np.array_equal(pa[-16:, 1:], pb[-16:, 1:])


def test_workload_positions():
    pos = O.rope_positions(W.EDIT_2REF.block_ids())
    # [t48][ref 64x64][t40][ref 64x64][t24][target 64x64]
    assert tuple(pos[47]) == (47, 47, 47)
    assert (pos[48:48 + 4096, 0] == 48).all()
    assert pos[48:48 + 4096, 1].min() == -32 and pos[48:48 + 4096, 1].max() == 31
    assert tuple(pos[4144]) == (49, 49, 49)
    assert (pos[-4096:, 0] == 48 + 1 + 40 + 1 + 24).all()


def test_positions_reject_a_wrong_shape():
    with pytest.raises(ValueError):
        O.rope_positions(W.block_ids_from_segments([("image", 12)]))        # not square
    with pytest.raises(ValueError):
        O.rope_positions(W.block_ids_from_segments([("image", 12)]), [(3, 5)])


# ---------------------------------------------------------------------------------------------
# rotation
# ---------------------------------------------------------------------------------------------
def unit(d):
    x = np.zeros((1, 1, 1, 128))
    x[..., d] = 1.0
    return x


def check_rotation(rope_fn):
    """Unit vector e_d at position p: the pair holding d turns by p times its frequency."""
    p = 3.0
    cases = [
        (0, (p, 0, 0), 1.0),                    # frame pair 0
        (2, (p, 0, 0), 10 ** -0.5),             # frame pair 1: 10^(-1/2)
        (14, (p, 0, 0), 10 ** -3.5),            # frame pair 7
        (16, (0, p, 0), 1.0),                   # height pair 0 starts at dim 16
        (18, (0, p, 0), 10 ** (-1 / 7)),        # height pair 1
        (70, (0, p, 0), 10 ** (-27 / 7)),       # height pair 27 (last)
        (72, (0, 0, p), 1.0),                   # width pair 0 starts at dim 72
        (126, (0, 0, p), 10 ** (-27 / 7)),      # width pair 27 (last)
    ]
    for d, pos, f in cases:
        got = rope_fn(unit(d), np.array([pos]))[0, 0, 0]
        want = np.zeros(128)
        want[d] = math.cos(p * f)
        want[d + 1] = math.sin(p * f)
        assert np.allclose(got, want, atol=1e-12), (d, pos)
    # a position on one axis does not move the other axes' dims
    got = rope_fn(unit(20), np.array([(5.0, 0, 0)]))[0, 0, 0]
    assert np.allclose(got, unit(20)[0, 0, 0], atol=1e-15)


def oracle_rope(x, pos):
    return O.apply_rope(x, O.rope_angles(pos))


def test_rotation_closed_forms():
    check_rotation(oracle_rope)


def test_rotation_preserves_pair_lengths_and_is_relative():
    rng = np.random.default_rng(1)
    q = rng.standard_normal((1, 1, 1, 128))
    k = rng.standard_normal((1, 1, 1, 128))
    p1, p2, t = np.array([[3, -7, 11]]), np.array([[40, 2, -5]]), np.array([[17, -9, 4]])
    rq = oracle_rope(q, p1)
    pair_len = lambda x: x[..., 0::2] ** 2 + x[..., 1::2] ** 2
    assert np.allclose(pair_len(rq), pair_len(q), atol=1e-12)
    d1 = np.sum(oracle_rope(q, p1) * oracle_rope(k, p2))
    d2 = np.sum(oracle_rope(q, p1 + t) * oracle_rope(k, p2 + t))
    assert abs(d1 - d2) < 1e-10
    d3 = np.sum(oracle_rope(q, p1 + t) * oracle_rope(k, p2))   # not a common shift
    assert abs(d1 - d3) > 1e-3


# ---------------------------------------------------------------------------------------------
# RMS norm
# ---------------------------------------------------------------------------------------------
def test_rms_norm_closed_forms():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((2, 5, 3, 128)) * rng.uniform(0.1, 10, size=(2, 5, 3, 1))
    ones = np.ones(128)
    y = O.rms_norm(x, ones, eps=0.0)
    assert np.allclose(np.mean(y * y, axis=-1), 1.0, atol=1e-12)
    assert np.allclose(O.rms_norm(7.5 * x, ones, eps=0.0), y, atol=1e-12)
    c = np.full((1, 1, 1, 128), -2.5)
    assert np.allclose(O.rms_norm(c, ones, eps=0.0), -1.0, atol=1e-15)
    w = rng.uniform(0.5, 1.5, size=128)
    assert np.allclose(O.rms_norm(x, w, eps=0.0), y * w, atol=1e-12)
    # eps only matters at tiny scale: mean square 1e-6 and eps 1e-6 halve the mean square
    tiny = np.full((1, 1, 1, 128), 1e-3)
    assert np.allclose(O.rms_norm(tiny, ones, eps=1e-6), 1e-3 / math.sqrt(2e-6), atol=1e-12)


def test_prologue_is_norm_then_rope():
    """RoPE keeps pair lengths, so the prologue's per-head RMS is the norm's (w = 1); and a
    head rotated back by the same angles gives the normalised input."""
    rng = np.random.default_rng(3)
    ids = W.TINY.block_ids()
    q = rng.standard_normal((1, 146, 2, 128)) * 4
    k = rng.standard_normal((1, 146, 2, 128)) * 0.3
    ones = np.ones(128)
    pos = O.rope_positions(ids)
    qo, ko = O.qk_prologue(q, k, ones, ones, pos, eps=0.0)
    assert np.allclose(np.mean(qo * qo, axis=-1), 1.0, atol=1e-12)
    back = O.apply_rope(ko, -O.rope_angles(pos))
    assert np.allclose(back, O.rms_norm(k, ones, eps=0.0), atol=1e-12)


# ---------------------------------------------------------------------------------------------
# planted mistakes
# ---------------------------------------------------------------------------------------------
def _rope_rotate_half(x, pos):
    a = O.rope_angles(pos)[None, :, None, :]
    x = np.asarray(x, dtype=np.float64)
    x0, x1 = x[..., :64], x[..., 64:]
    return np.concatenate([x0 * np.cos(a) - x1 * np.sin(a), x0 * np.sin(a) + x1 * np.cos(a)], -1)


def _rope_swapped_sections(x, pos):
    return O.apply_rope(x, O.rope_angles(np.asarray(pos)[:, ::-1], sections=(56, 56, 16)))


def _rope_freq_over_d(x, pos):
    pos = np.asarray(pos, dtype=np.float64)
    cols = []
    for axis, d in enumerate(O.ROPE_SECTIONS):
        k = np.arange(d // 2, dtype=np.float64)
        cols.append(pos[:, axis:axis + 1] * (O.ROPE_BASE ** (-k / d))[None, :])
    return O.apply_rope(x, np.concatenate(cols, 1))


@pytest.mark.parametrize("bad", [_rope_rotate_half, _rope_swapped_sections, _rope_freq_over_d])
def test_planted_rotation_mistakes_are_caught(bad):
    with pytest.raises(AssertionError):
        check_rotation(bad)


def _pos_text_frozen(ids, hw):
    p = O.rope_positions(ids, hw)
    p[p[:, 0] == p[:, 1]] = 0
    return p


def _pos_uncentred(ids, hw):
    p = O.rope_positions(ids, hw).copy()
    img = ~((p[:, 0] == p[:, 1]) & (p[:, 1] == p[:, 2]))
    p[img, 1] -= p[img, 1].min()
    return p


def _pos_frame_per_row(ids, hw):
    p = O.rope_positions(ids, hw).copy()
    img = ~((p[:, 0] == p[:, 1]) & (p[:, 1] == p[:, 2]))
    p[img, 0] += p[img, 1] + 1
    return p


@pytest.mark.parametrize("bad", [_pos_text_frozen, _pos_uncentred, _pos_frame_per_row])
def test_planted_position_mistakes_are_caught(bad):
    with pytest.raises(AssertionError):
        check_positions(bad)
