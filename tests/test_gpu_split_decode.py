"""GPU parity of the split-KV decode (bca_decode_split) against the oracle's decode.

The split path computes the same softmax as the plain decode with the key axis cut into ranges,
so the oracle is the plain (pinned) decode.  Checked:
* small layouts in full, with 2, 3, automatic and clamped range counts, and ranges that straddle
  the cache/target split or the end;
* one range is the plain decode, bit for bit; more ranges agree with it to the tolerance (each
  range rounds p to bf16 against its own running max);
* an exact counting probe: with Q = 0 every range has running max 0, so the merge is a sum of
  exact integer counts and O must equal the mean of V to 2 ulp;
* FP8 caches through the split path against the oracle's decode over its own FP8 cache;
* the 512^2-target editing shape (N = 1,024 under P = 8,304) at B = 1 and 2, sampled rows.
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


def bf16_cache(kb, vb, P):
    c = bca.KVCache(bca.KVCache.BF16, to_dev(kb[:, :P]), to_dev(vb[:, :P]))
    return c


@pytest.mark.parametrize("seed,S,tgt,B,H", [(101, 300, 70, 1, 2), (102, 777, 129, 2, 2),
                                            (103, 1500, 64, 1, 3), (104, 146, 64, 1, 2)])
def test_split_decode_small_layouts(seed, S, tgt, B, H):
    rng = np.random.default_rng(seed)
    ids = W.TINY.block_ids() if S == 146 else W.random_layout(rng, S, max_seg=120)
    ids[-tgt:] = 10 ** 6
    plan = bca.Plan(ids)
    P, N = plan.info.prefix_len, plan.info.target_len
    qb, kb, vb = W.qkv(seed, B, S, H, scaled=False)
    cache = bf16_cache(kb, vb, P)
    q, k, v = to_dev(qb[:, P:]), to_dev(kb[:, P:]), to_dev(vb[:, P:])
    ref = O.decode(f32(qb[:, P:]), f32(kb[:, :P]), f32(vb[:, :P]), f32(kb[:, P:]), f32(vb[:, P:]))
    plain = bca.decode_ex(plan, q, cache, k, v)
    for n_split in (2, 3, 0, 10 ** 4):
        _, used = bca.split_workspace(plan, B, H, n_split)
        say(f"case: split decode seed={seed} P={P} N={N} n_split={n_split} -> {used}")
        got = bca.decode_split(plan, q, cache, k, v, n_split=n_split)
        torch.cuda.synchronize()
        check(got.cpu().numpy(), ref, f"{used} ranges vs oracle")
        # each range rounds p to bf16 against its own running max: the two paths agree to the
        # same tolerance, not bitwise
        check(got.cpu().numpy(), plain.cpu().numpy(), f"{used} ranges vs the plain decode")
    one = bca.decode_split(plan, q, cache, k, v, n_split=1)
    torch.cuda.synchronize()
    assert torch.equal(one, plain)


def test_split_decode_count_probe_exact():
    ids = W.EDIT_2REF_T512.block_ids()
    plan = bca.Plan(ids)
    P, N = plan.info.prefix_len, plan.info.target_len
    B, H = 1, 2
    S = len(ids)
    v = np.zeros((S, 128), np.float32)
    j = np.arange(S)
    for bit in range(14):
        v[:, bit] = (j >> bit) & 1
    v[:, 20] = (j < P)                                       # cache rows
    vb = np.broadcast_to(W.f32_to_bf16_bits(v)[None, :, None, :], (B, S, H, 128)).copy()
    kb = W.qkv(105, B, S, H)[1]
    qb = np.zeros((B, N, H, 128), np.uint16)
    cache = bf16_cache(kb, vb, P)
    want = v.astype(np.float64).mean(axis=0)
    tol = 2 * np.spacing(np.abs(want).astype(np.float32)).astype(np.float64)
    for n_split in (0, 7, 146):
        got = bca.decode_split(plan, to_dev(qb), cache, to_dev(kb[:, P:]), to_dev(vb[:, P:]),
                               n_split=n_split)
        torch.cuda.synchronize()
        g = got.cpu().numpy()
        say(f"case: split count probe n_split={n_split}")
        assert (np.abs(g - want) <= tol).all(), n_split


@pytest.mark.parametrize("fmt", [bca.KVCache.FP8_V, bca.KVCache.FP8_KV])
def test_split_decode_fp8_cache(fmt):
    rng = np.random.default_rng(106)
    ids = W.random_layout(rng, 900, max_seg=200)
    ids[-130:] = 10 ** 6
    plan = bca.Plan(ids)
    P, N = plan.info.prefix_len, plan.info.target_len
    B, H = 2, 2
    qb, kb, vb = W.qkv(106, B, len(ids), H, scaled=False)
    cache = bca.KVCache.empty(plan, B, H, fmt, device=DEV)
    bca.prefill_ex(plan, to_dev(qb), to_dev(kb), to_dev(vb), cache)
    got = bca.decode_split(plan, to_dev(qb[:, P:]), cache, to_dev(kb[:, P:]), to_dev(vb[:, P:]),
                           n_split=3)
    torch.cuda.synchronize()
    oc = O.prefix_cache_fp8(f32(kb), f32(vb), ids, fmt)
    ref = O.decode_cached(f32(qb[:, P:]), oc, f32(kb[:, P:]), f32(vb[:, P:]))
    say(f"case: split decode FP8 format {fmt}")
    check(got.cpu().numpy(), ref, "split over FP8 cache vs oracle")


@pytest.mark.parametrize("B", [1, 2])
def test_split_decode_small_target_full_size(B):
    lay = W.EDIT_2REF_T512
    ids = lay.block_ids()
    H = lay.heads
    plan = bca.Plan(ids)
    P, N = plan.info.prefix_len, plan.info.target_len
    assert (P, N) == (8304, 1024)
    qb, kb, vb = W.qkv(W.SEEDS["edit_2ref_t512"], B, len(ids), H, scaled=False)
    cache = bf16_cache(kb, vb, P)
    _, used = bca.split_workspace(plan, B, H)
    say(f"case: 512^2 target B={B}: {used} ranges")
    got = bca.decode_split(plan, to_dev(qb[:, P:]), cache, to_dev(kb[:, P:]), to_dev(vb[:, P:]))
    torch.cuda.synchronize()
    rows = np.unique(np.r_[np.arange(0, N, 37), [N - 1]])
    heads = [0, 31]
    g = got[:, torch.from_numpy(rows).to(DEV)][:, :, heads].cpu().numpy()
    ref = O.decode(f32(qb[:, P:][:, :, heads]), f32(kb[:, :P][:, :, heads]),
                   f32(vb[:, :P][:, :, heads]), f32(kb[:, P:][:, :, heads]),
                   f32(vb[:, P:][:, :, heads]), rows=rows)
    check(g, ref, f"{used} ranges, sampled rows")
