"""CPU tests of bca_prefill_layout: when a single-sequence prefill hands its target rows to the
cached step's kernels (two launches) and when it runs as one launch.  Host-only plans; no GPU."""
import numpy as np
import pytest

import bca_workloads as W

bca = pytest.importorskip("block_causal_attention_amd")
from block_causal_attention_amd import _lib  # noqa: E402


def cdiv(a, b):
    return -(-a // b)


def expected(plan, B, H, cus):
    """The rule as bca.h states it."""
    info = plan.info
    P, N, nt = info.prefix_len, info.target_len, info.n_qtiles
    two = (info.n_sequences == 1 and info.decode_ok and P > 0 and nt * B * H < 2 * cus
           and cdiv(N, 384) * B * H >= cus and bca.decode_layout(N, B * H, 1, 0, cus)[0] == 12)
    return (2, cdiv(P, info.block_m), N) if two else (1, nt, 0)


def test_text_to_image_hands_off_at_one_batch_item():
    plan = bca.Plan(W.T2I_1024.block_ids(), host_only=True)
    assert bca.prefill_layout(plan, 1, 32, 256) == (2, 1, 4096)
    # twice the grid fills two rounds: one launch
    assert bca.prefill_layout(plan, 2, 32, 256) == (1, 12, 0)


def test_target_under_one_round_keeps_one_launch():
    # 2,304 target rows: one 12-wave round of its own, no better than the one-launch prefill
    ids = W.block_ids_from_segments([("text", 256), ("image", 2304)])
    plan = bca.Plan(ids, host_only=True)
    assert bca.decode_layout(2304, 32, 1, 0, 256)[0] == 12
    assert bca.prefill_layout(plan, 1, 32, 256) == (1, plan.info.n_qtiles, 0)


def test_headline_layouts_take_one_launch():
    for lay in (W.EDIT_2REF, W.LONG_4REF, W.TINY):
        plan = bca.Plan(lay.block_ids(), host_only=True)
        assert bca.prefill_layout(plan, 1, lay.heads, 256)[0] == 1


def test_text_last_and_batches_of_sequences_take_one_launch():
    ids = W.block_ids_from_segments([("text", 100), ("image", 300), ("text", 20)])
    plan = bca.Plan(ids, host_only=True)
    assert bca.prefill_layout(plan, 1, 32, 256) == (1, plan.info.n_qtiles, 0)
    t2i = W.T2I_1024.block_ids()
    vplan = bca.Plan.varlen([t2i], host_only=True)
    assert bca.prefill_layout(vplan, 1, 32, 256)[0] == 1


@pytest.mark.parametrize("seed", range(40))
def test_rule_on_random_layouts(seed):
    rng = np.random.default_rng(500 + seed)
    S = int(rng.integers(1, 9000))
    ids = W.random_layout(rng, S, p_text=float(rng.uniform(0.1, 0.9)), max_seg=max(1, S // 3))
    if rng.integers(0, 2):
        ids[-max(1, int(S * rng.uniform(0.05, 0.9))):] = 10 ** 6  # an image block last
    plan = bca.Plan(ids, host_only=True)
    for B, H, cus in ((1, 32, 256), (2, 32, 256), (1, 8, 80), (1, 16, 304), (3, 24, 256)):
        got = bca.prefill_layout(plan, B, H, cus)
        assert got == expected(plan, B, H, cus), (S, B, H, cus)
        if got[0] == 2:
            assert got[1] * plan.info.block_m >= plan.info.prefix_len > 0


@pytest.mark.parametrize("args", [(0, 32, 256), (1, 0, 256), (1, 32, -1)])
def test_bad_arguments(args):
    plan = bca.Plan(W.T2I_1024.block_ids(), host_only=True)
    with pytest.raises(bca.BcaError) as e:
        bca.prefill_layout(plan, *args)
    assert e.value.status == _lib.BCA_ERR_ARG
