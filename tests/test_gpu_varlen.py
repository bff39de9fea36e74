"""GPU parity of the batch-of-sequences prefill (bca_plan_varlen + bca_prefill_varlen).

* Full comparison with the oracle on random batches, packed and with gaps; rows outside every
  sequence keep their sentinel value.
* A single-sequence plan through the varlen entry point gives bitwise the plain prefill.
* Exact counting probe over a whole batch (Q = 0, V = key-index bits and run indicators):
  closed form count / hi(i) per sequence, to 2 ulp, which catches any key read across a sequence
  boundary or off by one.
* Leak probe: rewriting every row outside sequence b leaves b's rows bitwise unchanged.
* A NEO-like batch at full size (batch 8, max_seq_len 4,096, 88 image tokens; H = 32 assumed):
  sampled rows against the oracle.
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
SENTINEL = 7.25


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


def rows_draw(seed, R, H, scaled=False):
    q, k, v = W.qkv(seed, 1, R, H, scaled)
    return q[0], k[0], v[0]


def run(ids_list, starts, qb, kb, vb):
    plan = bca.Plan.varlen(ids_list, row_start=starts)
    R, H, _ = qb.shape
    out = torch.full((R, H, 128), SENTINEL, dtype=torch.float32, device=DEV)
    bca.prefill_varlen(plan, to_dev(qb), to_dev(kb), to_dev(vb), out=out)
    torch.cuda.synchronize()
    return plan, out.cpu().numpy()


def covered(ids_list, starts, R):
    m = np.zeros(R, bool)
    for ids, a in zip(ids_list, starts):
        m[a:a + len(ids)] = True
    return m


@pytest.mark.parametrize("seed,n_seq,max_len,gaps", [(91, 1, 300, False), (92, 3, 700, False),
                                                     (93, 5, 400, True), (94, 7, 260, True)])
def test_varlen_random_batches(seed, n_seq, max_len, gaps):
    rng = np.random.default_rng(seed)
    ids_list = [W.random_layout(rng, int(rng.integers(1, max_len)), max_seg=90) for _ in range(n_seq)]
    lens = [len(i) for i in ids_list]
    if gaps:
        # sequences laid out in a shuffled order with gaps between them
        order = rng.permutation(n_seq)
        starts = np.zeros(n_seq, np.int64)
        r = int(rng.integers(0, 40))
        for b in order:
            starts[b] = r
            r += lens[b] + int(rng.integers(0, 40))
        R = r + 3
    else:
        starts = O.packed_row_starts(lens)
        R = int(sum(lens))
    H = 2
    say(f"case: varlen seed={seed} lens={lens} gaps={gaps}")
    qb, kb, vb = rows_draw(seed, R, H)
    plan, got = run(ids_list, starts, qb, kb, vb)
    ref = O.attention_varlen(f32(qb), f32(kb), f32(vb), ids_list, starts)
    for b, (ids, a) in enumerate(zip(ids_list, starts)):
        check(got[a:a + len(ids)], ref[b], f"sequence {b} (len {len(ids)})")
    pad = ~covered(ids_list, starts, R)
    assert (got[pad] == SENTINEL).all()


def test_single_sequence_plan_through_varlen_is_the_prefill():
    ids = W.TINY.block_ids()
    qb, kb, vb = W.qkv(95, 1, len(ids), 2, scaled=False)
    plan = bca.Plan(ids)
    o1 = bca.prefill(plan, to_dev(qb), to_dev(kb), to_dev(vb))
    o2 = bca.prefill_varlen(plan, to_dev(qb[0]), to_dev(kb[0]), to_dev(vb[0]))
    torch.cuda.synchronize()
    assert torch.equal(o1[0], o2)


def test_varlen_count_probe_exact():
    rng = np.random.default_rng(96)
    ids_list = [W.random_layout(rng, int(n), max_seg=400) for n in (1500, 130, 2200, 64, 900)]
    starts = np.array([5000, 0, 200, 2600, 2700], np.int64)   # gaps, not in sequence order
    R = 6510                                                  # seq 0 ends at 6500
    H = 2
    v = np.zeros((R, 128), np.float32)
    want = {}
    for b, (ids, a) in enumerate(zip(ids_list, starts)):
        n = len(ids)
        segs = O.runs(ids)
        assert len(segs) <= 48
        vv = np.zeros((n, 128), np.float32)
        for c, (s0, s1, _) in enumerate(segs):
            vv[s0:s1, c] = 1.0
        j = np.arange(n)
        for bit in range(12):
            vv[:, 64 + bit] = (j >> bit) & 1
        vv[:, 100] = b + 1                                       # identifies the sequence
        v[a:a + n] = vv
        hi = O.row_key_limits(ids)
        cum = np.concatenate([np.zeros((1, 128)), np.cumsum(vv.astype(np.float64), axis=0)])
        want[b] = cum[hi] / hi[:, None]
    vb = np.broadcast_to(W.f32_to_bf16_bits(v)[:, None, :], (R, H, 128)).copy()
    qb = np.zeros((R, H, 128), np.uint16)
    kb = rows_draw(97, R, H)[1]
    say("case: varlen count probe")
    _, got = run(ids_list, starts, qb, kb, vb)
    for b, (ids, a) in enumerate(zip(ids_list, starts)):
        g = got[a:a + len(ids)]
        tol = 2 * np.spacing(np.abs(want[b]).astype(np.float32)).astype(np.float64)
        for h in range(H):
            bad = np.abs(g[:, h] - want[b]) > tol
            assert not bad.any(), (b, h, np.argwhere(bad)[:5])


def test_varlen_leak_probe_bitwise():
    rng = np.random.default_rng(98)
    ids_list = [W.random_layout(rng, int(n), max_seg=200) for n in (700, 333, 1024)]
    lens = [len(i) for i in ids_list]
    starts = O.packed_row_starts(lens)
    R, H = sum(lens), 2
    qb, kb, vb = rows_draw(98, R, H)
    _, base = run(ids_list, starts, qb, kb, vb)
    say("case: varlen leak probe")
    for b, a in enumerate(starts):
        q2, k2, v2 = qb.copy(), kb.copy(), vb.copy()
        outside = np.ones(R, bool)
        outside[a:a + lens[b]] = False
        big = W.f32_to_bf16_bits(30 * rng.standard_normal((int(outside.sum()), H, 128),
                                                          dtype=np.float32))
        for t in (q2, k2, v2):
            t[outside] = big
        _, got = run(ids_list, starts, q2, k2, v2)
        assert np.array_equal(got[a:a + lens[b]], base[a:a + lens[b]]), b


def test_neo_like_batch_full_size_sampled():
    ids_list, lens = W.neo_like_batch(99, 8, 4096, 88)
    starts = O.packed_row_starts(lens)
    R, H = int(sum(lens)), 32
    say(f"case: NEO-like batch 8 x <=4096, R={R}, H={H}")
    qb, kb, vb = rows_draw(99, R, H, scaled=False)
    plan, got = run(ids_list, starts, qb, kb, vb)
    rows_of = {}
    for b, ids in enumerate(ids_list):
        n = len(ids)
        r = set(range(0, n, 389)) | {n - 1}
        for s0, s1, bid in O.runs(ids):
            if bid >= 0:
                r |= {s0, s1 - 1, min(n - 1, s1)}
        rows_of[b] = np.array(sorted(r))
    heads = [0, 31]
    ref = O.attention_varlen(f32(qb), f32(kb), f32(vb), ids_list, starts, rows_of=rows_of,
                             heads=heads)
    for b, a in enumerate(starts):
        check(got[a + rows_of[b]][:, heads], ref[b], f"sequence {b} sampled rows")
