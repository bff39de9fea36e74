"""CPU tests of the prologue's host side: RoPE positions and table against the oracle, and the
argument checks of bca_rope_positions, bca_rope_table and bca_qk_prologue (no GPU needed: every
call here is rejected before anything is launched)."""
import ctypes

import numpy as np
import pytest

import bca_workloads as W
from oracle import bca_oracle as O

bca = pytest.importorskip("block_causal_attention_amd")
from block_causal_attention_amd import _lib  # noqa: E402


def image_shapes(ids):
    """(H, W) per image run: the most nearly square factorisation."""
    hw = []
    for a, e, bid in O.runs(ids):
        if bid >= 0:
            n = e - a
            H = max(d for d in range(1, int(np.sqrt(n)) + 1) if n % d == 0)
            hw.append((H, n // H))
    return hw


@pytest.mark.parametrize("name", ["tiny", "t2i_1024", "edit_2ref", "long_4ref"])
def test_positions_bit_exact_on_workloads(name):
    ids = W.WORKLOADS[name].block_ids()
    got = bca.rope_positions(ids)
    assert np.array_equal(got.astype(np.int64), O.rope_positions(ids))


def test_positions_bit_exact_fuzz_with_shapes():
    rng = np.random.default_rng(31)
    for _ in range(30):
        ids = W.random_layout(rng, int(rng.integers(1, 500)), p_text=float(rng.random()),
                              max_seg=int(rng.integers(1, 120)))
        hw = image_shapes(ids)
        got = bca.rope_positions(ids, hw if hw else None)
        assert np.array_equal(got.astype(np.int64), O.rope_positions(ids, hw if hw else None))


def test_table_matches_oracle_angles():
    for ids in (W.TINY.block_ids(), W.EDIT_2REF.block_ids()):
        pos = bca.rope_positions(ids)
        tab = bca.rope_table(pos).astype(np.float64)
        ang = O.rope_angles(O.rope_positions(ids))
        # float rounding of the exact cos / sin: within half a float ulp (2^-25 below 1)
        assert np.abs(tab[..., 0] - np.cos(ang)).max() <= 2.0 ** -24
        assert np.abs(tab[..., 1] - np.sin(ang)).max() <= 2.0 ** -24


def test_host_argument_errors():
    with pytest.raises(bca.BcaError) as e:
        bca.rope_positions(W.block_ids_from_segments([("image", 12)]))       # not square
    assert e.value.status == _lib.BCA_ERR_ARG
    with pytest.raises(bca.BcaError) as e:
        bca.rope_positions(W.block_ids_from_segments([("image", 12)]), [(3, 5)])
    assert e.value.status == _lib.BCA_ERR_ARG
    with pytest.raises(bca.BcaError) as e:                                   # wrong count
        bca.rope_positions(W.block_ids_from_segments([("image", 12)]), [(3, 4), (1, 1)])
    assert e.value.status == _lib.BCA_ERR_ARG
    with pytest.raises(bca.BcaError) as e:
        bca.rope_positions([0, -1, 0])
    assert e.value.status == _lib.BCA_ERR_BLOCK_IDS
    lib = _lib.load()
    pos = np.zeros((2, 3), np.int32)
    out = np.zeros((2, 64, 2), np.float32)
    ip = pos.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
    fp = out.ctypes.data_as(ctypes.POINTER(ctypes.c_float))
    assert lib.bca_rope_table(ip, 2, 1.0, fp) == _lib.BCA_ERR_ARG
    assert lib.bca_rope_table(ip, 2, float("inf"), fp) == _lib.BCA_ERR_ARG
    assert lib.bca_rope_table(None, 2, 1e4, fp) == _lib.BCA_ERR_ARG
    assert lib.bca_rope_table(ip, 2, 1e4, fp) == _lib.BCA_OK
    assert (out[..., 0] == 1).all() and (out[..., 1] == 0).all()            # position 0


def test_prologue_argument_errors():
    lib = _lib.load()
    t = lambda ptr=0x10000, ss=4096: ctypes.byref(_lib.BcaTensor(ptr, 8 * 4096, ss, 128))
    v = ctypes.c_void_p(0x20000)

    def call(B=1, S=8, H=2, D=128, eps=1e-6, q=None, wq=v, table=v):
        return lib.bca_qk_prologue(B, S, H, D, eps, q or t(), t(), t(), t(), wq, v, table, None)

    assert call(D=64) == _lib.BCA_ERR_UNSUPPORTED
    assert call(B=0) == _lib.BCA_ERR_ARG
    assert call(S=0) == _lib.BCA_ERR_ARG
    assert call(eps=-1.0) == _lib.BCA_ERR_ARG
    assert call(eps=float("nan")) == _lib.BCA_ERR_ARG
    assert call(q=t(ptr=0x10008)) == _lib.BCA_ERR_ARG
    assert call(q=t(ss=4100)) == _lib.BCA_ERR_ARG
    assert call(wq=None) == _lib.BCA_ERR_ARG
    assert call(table=ctypes.c_void_p(0x20004)) == _lib.BCA_ERR_ARG
    assert b"16-byte" in lib.bca_last_error()
