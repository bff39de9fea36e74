"""GPU test of the allocation-free split decode (bca_decode_split_noalloc), through the C ABI.

Its kernels are those of bca_decode_split; only the partial results move from a caller
workspace to the library's own device scratch.  So on every call its output must equal
bca_decode_split's on the same inputs and range count bit for bit.  Two calls in a row, the
second on a smaller input (the scratch keeps the first call's contents, none of which may leak
into the second), then an unsplit call (no scratch) and a split too large for the scratch, which
must be rejected on the host with nothing enqueued.
"""
import numpy as np
import pytest

import bca_workloads as W
from oracle import bca_oracle as O

torch = pytest.importorskip("torch")
bca = pytest.importorskip("block_causal_attention_amd")
from block_causal_attention_amd import _lib  # noqa: E402

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def say(*a):
    print(*a, flush=True)


def to_dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(DEV)


def case(ids, B, H, seed):
    plan = bca.Plan(ids)
    P = plan.info.prefix_len
    qb, kb, vb = W.qkv(seed, B, len(ids), H, scaled=False)
    cache = bca.KVCache(bca.KVCache.BF16, to_dev(kb[:, :P]), to_dev(vb[:, :P]))
    q, k, v = (to_dev(x[:, P:]) for x in (qb, kb, vb))
    return plan, cache, q, k, v, (qb, kb, vb)


def both(plan, cache, q, k, v, n_split):
    nbytes, used = bca.split_workspace(plan, q.shape[0], q.shape[2], n_split)
    want = bca.decode_split(plan, q, cache, k, v, n_split=n_split)
    got = torch.full_like(want, float("nan"))
    bca.decode_split_noalloc(plan, q, cache, k, v, n_split=n_split, out=got)
    torch.cuda.synchronize()
    return want, got, nbytes, used


def test_noalloc_split_decode_matches_the_workspace_call():
    # call 1: the 512^2 target under two 1024^2 references (B = 1, H = 32), library-chosen ranges
    lay = W.EDIT_2REF_T512
    say(f"case: no-alloc split decode, call 1: {lay.name}, B=1 H={lay.heads}")
    plan, cache, q, k, v, (qb, kb, vb) = case(lay.block_ids(), 1, lay.heads, 6001)
    want, got, nbytes, used = both(plan, cache, q, k, v, 0)
    say(f"  ranges {used}, partial results {nbytes} bytes of {_lib.BCA_SCRATCH_BYTES}")
    assert used > 1 and 0 < nbytes <= _lib.BCA_SCRATCH_BYTES
    assert torch.equal(got, want)
    P, N = plan.info.prefix_len, plan.info.target_len
    rows = np.unique(np.concatenate([np.arange(0, N, 97), [N - 1]]))
    heads = [0, 17, 31]
    f32 = W.bf16_bits_to_f32
    ref = O.decode(f32(qb[:, P:]), f32(kb[:, :P]), f32(vb[:, :P]), f32(kb[:, P:]), f32(vb[:, P:]),
                   rows=rows, heads=heads)
    err = np.abs(got[:, torch.from_numpy(rows).to(DEV)][:, :, heads].cpu().numpy() - ref)
    say(f"  vs oracle: max|err|={err.max():.3e} mean={err.mean():.3e}")
    assert err.max() <= 1e-2 and err.mean() <= 1e-3

    # call 2, smaller: a random layout (B = 2, H = 2), 2 ranges
    rng = np.random.default_rng(5)
    ids = W.random_layout(rng, 700, max_seg=120)
    ids[-150:] = 10 ** 6
    say("case: no-alloc split decode, call 2: random layout S=700, B=2 H=2, 2 ranges")
    plan2, cache2, q2, k2, v2, _ = case(ids, 2, 2, 8)
    want2, got2, nbytes2, used2 = both(plan2, cache2, q2, k2, v2, 2)
    assert used2 == 2 and 0 < nbytes2 < nbytes
    assert torch.equal(got2, want2)

    # one range: no scratch, the plain decode's result
    want3, got3, nbytes3, used3 = both(plan2, cache2, q2, k2, v2, 1)
    assert used3 == 1 and nbytes3 == 0
    assert torch.equal(got3, want3)
    assert torch.equal(got3, bca.decode_ex(plan2, q2, cache2, k2, v2))

    # too large for the scratch (the 512^2 target at B = 2 with 3 ranges): rejected on the host
    q4, k4, v4 = (torch.cat([t, t]) for t in (q, k, v))
    cache4 = bca.KVCache(bca.KVCache.BF16, torch.cat([cache.k, cache.k]),
                         torch.cat([cache.v, cache.v]))
    need, _ = bca.split_workspace(plan, 2, lay.heads, 3)
    assert need > _lib.BCA_SCRATCH_BYTES
    out4 = torch.full((2, N, lay.heads, 128), float("nan"), dtype=torch.float32, device=DEV)
    with pytest.raises(bca.BcaError) as exc:
        bca.decode_split_noalloc(plan, q4, cache4, k4, v4, n_split=3, out=out4)
    assert exc.value.status == _lib.BCA_ERR_ARG
    torch.cuda.synchronize()
    assert torch.isnan(out4).all()
    # and the scratch still serves the next call
    got5 = torch.empty_like(want2)
    bca.decode_split_noalloc(plan2, q2, cache2, k2, v2, n_split=2, out=got5)
    torch.cuda.synchronize()
    assert torch.equal(got5, want2)
    plan.free()
    plan2.free()
