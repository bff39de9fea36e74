"""GPU parity of the Q/K prologue (bca_qk_prologue) against the oracle, and of the whole chain
prologue -> prefill (storing post-RoPE K in the prefix cache) -> cached decode.

The prologue's bf16 outputs are compared element by element with the float64 oracle: at most
one bf16 ulp of the exact value (fp32 arithmetic, then one RNE rounding), or 1e-6 absolute for
values next to zero.  In-place calls match out-of-place calls bit for bit.
"""
import numpy as np
import pytest

import bca_workloads as W
from oracle import bca_oracle as O

torch = pytest.importorskip("torch")
bca = pytest.importorskip("block_causal_attention_amd")

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
MAX_TOL, MEAN_TOL = 1e-2, 1e-3


def say(*a):
    print(*a, flush=True)


def to_dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(DEV)


def from_dev(t):
    return W.bf16_bits_to_f32(t.cpu().view(torch.int16).numpy().view(np.uint16))


def f32(bits):
    return W.bf16_bits_to_f32(bits)


def bf16_ulp(x):
    a = np.abs(np.asarray(x, dtype=np.float64))
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    return np.where(a > 0, 2.0 ** (e - 7), 0.0)


def check_ulp(got, ref, what):
    err = np.abs(np.asarray(got, np.float64) - ref)
    tol = np.maximum(bf16_ulp(ref), 1e-6)
    bad = err > tol
    say(f"  {what}: max err/ulp = {(err / tol).max():.3f}, n = {err.size}")
    assert not bad.any(), (what, np.argwhere(bad)[:5])


def check(got, ref, what):
    err = np.abs(np.asarray(got, np.float64) - np.asarray(ref, np.float64))
    say(f"  {what}: max|err|={err.max():.3e} mean|err|={err.mean():.3e}")
    assert np.isfinite(got).all() and err.max() <= MAX_TOL and err.mean() <= MEAN_TOL, what


def run_prologue(ids, seed, B, H, image_hw=None, in_place=False):
    S = len(ids)
    qb, kb, wq, wk = W.prologue_inputs(seed, B, S, H)
    pos = bca.rope_positions(ids, image_hw)
    table = torch.from_numpy(bca.rope_table(pos)).to(DEV)
    q, k = to_dev(qb), to_dev(kb)
    wqd, wkd = torch.from_numpy(wq).to(DEV), torch.from_numpy(wk).to(DEV)
    if in_place:
        qo, ko = bca.qk_prologue(q, k, wqd, wkd, table, q_out=q, k_out=k)
    else:
        qo, ko = bca.qk_prologue(q, k, wqd, wkd, table)
    torch.cuda.synchronize()
    return qb, kb, wq, wk, qo, ko


@pytest.mark.parametrize("seed,S,B,H", [(61, 1, 1, 1), (62, 37, 2, 3), (63, 146, 1, 2),
                                         (64, 700, 2, 2)])
def test_prologue_matches_oracle(seed, S, B, H):
    rng = np.random.default_rng(seed)
    ids = W.TINY.block_ids() if S == 146 else W.random_layout(rng, S, max_seg=max(1, S // 4))
    hw = [(1, e - a) for a, e, bid in O.runs(ids) if bid >= 0] if S != 146 else None
    say(f"case: prologue seed={seed} S={S} B={B} H={H}")
    qb, kb, wq, wk, qo, ko = run_prologue(ids, seed, B, H, hw)
    rq, rk = O.qk_prologue(f32(qb), f32(kb), wq, wk, O.rope_positions(ids, hw))
    check_ulp(from_dev(qo), rq, "q'")
    check_ulp(from_dev(ko), rk, "k'")
    _, _, _, _, qi, ki = run_prologue(ids, seed, B, H, hw, in_place=True)
    assert torch.equal(qi, qo) and torch.equal(ki, ko)


def test_prologue_full_size_sampled_rows():
    lay = W.EDIT_2REF
    ids = lay.block_ids()
    say("case: prologue two-reference edit, S=12400 H=32")
    qb, kb, wq, wk, qo, ko = run_prologue(ids, 71, 1, lay.heads)
    rows = np.unique(np.r_[np.arange(0, lay.seq_len, 97), [lay.seq_len - 1, 47, 48, 4143, 4144]])
    pos = O.rope_positions(ids)[rows]
    rq, rk = O.qk_prologue(f32(qb[:, rows]), f32(kb[:, rows]), wq, wk, pos)
    idx = torch.from_numpy(rows).to(DEV)
    check_ulp(from_dev(qo[:, idx]), rq, "q' sampled rows")
    check_ulp(from_dev(ko[:, idx]), rk, "k' sampled rows")


@pytest.mark.parametrize("name", ["tiny", "random"])
def test_prologue_prefill_cache_decode_chain(name):
    """Prologue in place -> prefill storing the prefix cache -> prologue of a fresh target ->
    cached decode; the cache holds post-RoPE K bit for bit, and both outputs match the oracle
    run on the oracle's own prologue."""
    rng = np.random.default_rng(81)
    if name == "tiny":
        ids, hw, B, H = W.TINY.block_ids(), None, 1, 2
    else:
        ids = W.random_layout(rng, 520, max_seg=90)
        ids[-100:] = 10 ** 6
        hw = [(1, e - a) if e - a != 100 else (10, 10) for a, e, bid in O.runs(ids) if bid >= 0]
        B, H = 2, 2
    say(f"case: chain {name} S={len(ids)}")
    plan = bca.Plan(ids)
    P, N = plan.info.prefix_len, plan.info.target_len
    pos = bca.rope_positions(ids, hw)
    table = torch.from_numpy(bca.rope_table(pos)).to(DEV)
    qb, kb, wq, wk = W.prologue_inputs(82, B, len(ids), H)
    vb = W.qkv(83, B, len(ids), H, scaled=False)[2]
    q, k, v = to_dev(qb), to_dev(kb), to_dev(vb)
    wqd, wkd = torch.from_numpy(wq).to(DEV), torch.from_numpy(wk).to(DEV)
    bca.qk_prologue(q, k, wqd, wkd, table, q_out=q, k_out=k)
    cache = bca.KVCache.empty(plan, B, H, bca.KVCache.BF16, device=DEV)
    o = bca.prefill_ex(plan, q, k, v, cache)
    torch.cuda.synchronize()
    assert torch.equal(cache.k, k[:, :P]) and torch.equal(cache.v, v[:, :P])
    opos = O.rope_positions(ids, hw)
    rq, rk = O.qk_prologue(f32(qb), f32(kb), wq, wk, opos)
    ref = O.attention(rq, rk, f32(vb), ids)
    check(o.cpu().numpy(), ref, "prefill after prologue")
    # a fresh cached step: the target's raw Q/K go through the prologue with the target's rows
    qt_b, kt_b, _, _ = W.prologue_inputs(84, B, N, H)
    vt_b = W.qkv(85, B, N, H, scaled=False)[2]
    qt, kt = to_dev(qt_b), to_dev(kt_b)
    bca.qk_prologue(qt, kt, wqd, wkd, table[P:].contiguous(), q_out=qt, k_out=kt)
    od = bca.decode_ex(plan, qt, cache, kt, to_dev(vt_b))
    torch.cuda.synchronize()
    rqt, rkt = O.qk_prologue(f32(qt_b), f32(kt_b), wq, wk, opos[P:])
    refd = O.decode(rqt, rk[:, :P], f32(vb[:, :P]), rkt, f32(vt_b))
    check(od.cpu().numpy(), refd, "cached step after prologue")
