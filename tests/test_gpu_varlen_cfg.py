"""GPU parity of per-branch prefix caches (bca_prefill_varlen with caches) and the batched
cached step over them (bca_decode_varlen): CFG branches whose prompts differ in length, each
with its own cache (the guide's section "The prefix cache is a compute-for-memory trade").

* Small and mid-size batches (several query and key tiles, ragged ends, gaps between the
  branches' rows, a branch with an empty prefix): caches bitwise equal to each branch's prefix
  rows, the prefill and the cached step compared in full with the oracle, and the batched step
  bitwise equal to the single-branch decode of each branch.
* The full-size pair (the 2-ref 1024^2 edit as the cond branch, S = 12,400, and an uncond branch
  with an 8-position prompt, S = 12,360; H = 32): caches bitwise, prefill and cached step on
  sampled rows against the oracle, and the batched step bitwise equal to per-branch decodes.
* Strided views (Q/K/V rows of one packed buffer, caches and outputs inside wider buffers) give
  bitwise the contiguous results, and a one-sequence plan through bca_decode_varlen is bitwise
  the plain decode.
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


def f32(bits):
    return W.bf16_bits_to_f32(bits)


def check(got, ref, what):
    err = np.abs(np.asarray(got, np.float64) - np.asarray(ref, np.float64))
    say(f"  {what}: max|err|={err.max():.3e} mean|err|={err.mean():.3e} n={err.size}")
    assert np.isfinite(got).all() and err.max() <= MAX_TOL and err.mean() <= MEAN_TOL, what


def branch_layout(prompt, ref, gap_text, target):
    segs = ([("text", prompt)] if prompt else []) + ([("image", ref)] if ref else []) + \
        ([("text", gap_text)] if gap_text else []) + [("image", target)]
    return W.block_ids_from_segments(segs)


def run_branches(ids_list, starts, H, seed, rows_of=None, heads=None, full=True):
    """Prefill with per-branch caches, then one cached step with fresh targets; returns what the
    checks need."""
    lens = [len(i) for i in ids_list]
    R = int(max(a + n for a, n in zip(starts, lens))) + 5
    rng = np.random.default_rng(seed)
    q, k, v = (W.draw_bf16(rng, (R, H, 128)) for _ in range(3))
    plan = bca.Plan.varlen(ids_list, row_start=starts)
    sq = plan.sequences()
    off = O.varlen_offsets(ids_list)
    assert np.array_equal(sq[:, 2], off["P"]) and np.array_equal(sq[:, 3], off["N"])
    P, N = plan.info.prefix_len, plan.info.target_len
    say(f"  branches={len(ids_list)} lens={lens} P_b={off['P'].tolist()} H={H}")
    kc = torch.full((P, H, 128), 3.0, dtype=torch.bfloat16, device=DEV)
    vc = torch.full_like(kc, 3.0)
    o = bca.prefill_varlen(plan, to_dev(q), to_dev(k), to_dev(v), k_cache=kc, v_cache=vc)
    # fresh target Q/K/V for the cached step, packed
    qt, kt, vt = (W.draw_bf16(rng, (N, H, 128)) for _ in range(3))
    od = bca.decode_varlen(plan, to_dev(qt), kc, vc, to_dev(kt), to_dev(vt))
    torch.cuda.synchronize()
    return dict(q=q, k=k, v=v, plan=plan, kc=kc, vc=vc, o=o.cpu().numpy(), qt=qt, kt=kt, vt=vt,
                od=od.cpu().numpy(), off=off, starts=starts, lens=lens)


def check_caches(r, ids_list):
    kc_want, vc_want = O.prefix_cache_varlen(r["k"], r["v"], ids_list, r["starts"])
    got_k = r["kc"].view(torch.int16).cpu().numpy().view(np.uint16)
    got_v = r["vc"].view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(got_k, kc_want) and np.array_equal(got_v, vc_want), "cache rows"


def check_per_branch_decode(r, ids_list, H):
    """The batched step must be bitwise the single-branch decode of each branch."""
    off = r["off"]
    for b, ids in enumerate(ids_list):
        c, P, t, N = (int(off[x][b]) for x in ("c", "P", "t", "N"))
        plan1 = bca.Plan(ids)
        sl = lambda a, lo, n: to_dev(a[lo:lo + n])[None]
        kc1 = r["kc"][c:c + P][None].contiguous()
        vc1 = r["vc"][c:c + P][None].contiguous()
        o1 = bca.decode(plan1, sl(r["qt"], t, N), kc1 if P else None, vc1 if P else None,
                        sl(r["kt"], t, N), sl(r["vt"], t, N))
        torch.cuda.synchronize()
        assert np.array_equal(o1.cpu().numpy()[0], r["od"][t:t + N]), f"branch {b}"


@pytest.mark.parametrize("seed,branches,H", [
    (301, [(37, 300, 5, 700), (3, 300, 5, 700)], 3),            # CFG pair: prompts 37 vs 3
    (302, [(90, 500, 17, 420), (0, 500, 17, 420), (0, 0, 0, 420)], 2),  # empty prefix last
    (303, [(5, 0, 0, 33), (260, 129, 3, 800), (11, 40, 2, 65), (1, 1, 1, 1)], 2),
])
def test_cfg_branches_against_oracle(seed, branches, H):
    ids_list = [branch_layout(*b) for b in branches]
    lens = [len(i) for i in ids_list]
    starts = np.cumsum([3] + [n + 7 for n in lens])[:-1]        # gaps between the branches
    say(f"test_cfg_branches_against_oracle seed={seed}")
    r = run_branches(ids_list, starts, H, seed)
    check_caches(r, ids_list)
    want = O.attention_varlen(f32(r["q"]), f32(r["k"]), f32(r["v"]), ids_list, starts)
    for b, ids in enumerate(ids_list):
        a = int(starts[b])
        check(r["o"][a:a + len(ids)], want[b], f"prefill branch {b}")
    kc_w, vc_w = O.prefix_cache_varlen(f32(r["k"]), f32(r["v"]), ids_list, starts)
    dwant = O.decode_varlen(f32(r["qt"]), kc_w, vc_w, f32(r["kt"]), f32(r["vt"]), ids_list)
    off = r["off"]
    for b in range(len(ids_list)):
        t, N = int(off["t"][b]), int(off["N"][b])
        check(r["od"][t:t + N], dwant[b], f"cached step branch {b}")
    check_per_branch_decode(r, ids_list, H)


def test_cfg_full_size_pair():
    """The 2-ref edit under CFG with prompts of different lengths, at full size."""
    ids_list = [lay.block_ids() for lay in W.CFG_VARLEN]
    H = W.EDIT_2REF.heads
    lens = [len(i) for i in ids_list]
    starts = O.packed_row_starts(lens)
    say(f"test_cfg_full_size_pair lens={lens}")
    r = run_branches(ids_list, starts, H, W.SEEDS["cfg_varlen"])
    check_caches(r, ids_list)
    heads = [0, 17, 31]
    rows_of = {b: np.unique(np.r_[np.arange(0, n, 97), n - 1]) for b, n in enumerate(lens)}
    want = O.attention_varlen(f32(r["q"]), f32(r["k"]), f32(r["v"]), ids_list, starts,
                              rows_of=rows_of, heads=heads)
    for b in range(len(ids_list)):
        got = r["o"][int(starts[b]) + rows_of[b]][:, heads]
        check(got, want[b], f"prefill branch {b} (sampled rows)")
    off = r["off"]
    kc_w, vc_w = O.prefix_cache_varlen(f32(r["k"]), f32(r["v"]), ids_list, starts)
    drows = {b: np.unique(np.r_[np.arange(0, int(off["N"][b]), 61), int(off["N"][b]) - 1])
             for b in range(len(ids_list))}
    dwant = O.decode_varlen(f32(r["qt"]), kc_w, vc_w, f32(r["kt"]), f32(r["vt"]), ids_list,
                            rows_of=drows, heads=heads)
    for b in range(len(ids_list)):
        got = r["od"][int(off["t"][b]) + drows[b]][:, heads]
        check(got, dwant[b], f"cached step branch {b} (sampled rows)")
    check_per_branch_decode(r, ids_list, H)


def test_cfg_strided_views_and_single_plan():
    """Strided inputs (packed QKV rows), strided cache views and a strided output give bitwise the
    contiguous results; a single-sequence plan through bca_decode_varlen is the plain decode."""
    ids_list = [branch_layout(*b) for b in [(29, 130, 3, 200), (5, 130, 3, 200)]]
    lens = [len(i) for i in ids_list]
    starts = O.packed_row_starts(lens)
    H = 2
    say("test_cfg_strided_views_and_single_plan")
    r = run_branches(ids_list, starts, H, 311)
    plan = r["plan"]
    P, N = plan.info.prefix_len, plan.info.target_len
    R = r["q"].shape[0]
    # Q, K, V as slices of one packed [R, 3, H, 128] buffer; caches inside wider buffers
    qkv = torch.stack([to_dev(r["q"]), to_dev(r["k"]), to_dev(r["v"])], dim=1)
    q, k, v = qkv[:, 0], qkv[:, 1], qkv[:, 2]
    kc_big = torch.zeros((P, H + 1, 128), dtype=torch.bfloat16, device=DEV)
    vc_big = torch.zeros((P, 2, H, 128), dtype=torch.bfloat16, device=DEV)
    kc, vc = kc_big[:, :H], vc_big[:, 1]
    o_big = torch.zeros((R, H, 2, 128), dtype=torch.float32, device=DEV)
    o = o_big[:, :, 1]
    bca.prefill_varlen(plan, q, k, v, k_cache=kc, v_cache=vc, out=o)
    t = torch.stack([to_dev(r["qt"]), to_dev(r["kt"]), to_dev(r["vt"])], dim=2)
    od_big = torch.zeros((N, 2, H, 128), dtype=torch.float32, device=DEV)
    od = bca.decode_varlen(plan, t[:, :, 0], kc, vc, t[:, :, 1], t[:, :, 2], out=od_big[:, 0])
    torch.cuda.synchronize()
    for a, bq in ((o, r["o"]), (od, r["od"])):
        assert np.array_equal(a.cpu().numpy()[:bq.shape[0]], bq)
    assert torch.equal(kc.cpu(), r["kc"].cpu()) and torch.equal(vc.cpu(), r["vc"].cpu())
    # one sequence, planned with bca_plan: bca_decode_varlen is the plain decode
    ids = ids_list[0]
    plan1 = bca.Plan(ids)
    P1, N1 = plan1.info.prefix_len, plan1.info.target_len
    qb, kb, vb = (to_dev(x[:len(ids)]) for x in (r["q"], r["k"], r["v"]))
    kc1 = kb[:P1].contiguous()
    vc1 = vb[:P1].contiguous()
    od1 = bca.decode_varlen(plan1, qb[P1:], kc1, vc1, kb[P1:], vb[P1:])
    od2 = bca.decode(plan1, qb[None, P1:], kc1[None], vc1[None], kb[None, P1:], vb[None, P1:])
    torch.cuda.synchronize()
    assert np.array_equal(od1.cpu().numpy(), od2.cpu().numpy()[0])


@pytest.mark.parametrize("seed,branches", [
    # two sequences x 32 heads: 8 x 384 rows in the 12-wave launch, then 4 x 256 in the tail
    # launch; the second sequence ends inside the first tail tile
    (321, [(20, 100, 3, 4000), (7, 100, 3, 3300)]),
    # three sequences: every row in the tail launch; the third ends inside its fourth tile
    (322, [(20, 100, 3, 4000), (7, 100, 3, 3300), (5, 60, 0, 1000)]),
])
def test_batched_step_through_the_tail_launch(seed, branches):
    """bca_decode_varlen whose longest target takes the two-launch layout: sequences with fewer
    target rows leave tiles of either launch empty or part empty.  Caches bitwise, the batched
    step bitwise equal to each sequence's own decode, sampled rows against the oracle."""
    H = 32
    ids_list = [branch_layout(*b) for b in branches]
    lens = [len(i) for i in ids_list]
    starts = O.packed_row_starts(lens)
    off = O.varlen_offsets(ids_list)
    n_max = int(off["N"].max())
    layout = bca.decode_layout(n_max, len(ids_list) * H)
    assert layout[4] > 0, layout
    say(f"test_batched_step_through_the_tail_launch seed={seed} N_b={off['N'].tolist()} "
        f"layout={layout}")
    r = run_branches(ids_list, starts, H, seed)
    check_caches(r, ids_list)
    check_per_branch_decode(r, ids_list, H)
    heads = [0, 31]
    kc_w, vc_w = O.prefix_cache_varlen(f32(r["k"]), f32(r["v"]), ids_list, starts)
    drows = {}
    for b in range(len(ids_list)):
        n = int(off["N"][b])
        edges = [x for x in (3071, 3072, 3327, 3328, n - 1) if x < n]
        drows[b] = np.unique(np.r_[np.arange(0, n, 89), edges])
    dwant = O.decode_varlen(f32(r["qt"]), kc_w, vc_w, f32(r["kt"]), f32(r["vt"]), ids_list,
                            rows_of=drows, heads=heads)
    for b in range(len(ids_list)):
        got = r["od"][int(off["t"][b]) + drows[b]][:, heads]
        check(got, dwant[b], f"cached step branch {b} (sampled rows)")
