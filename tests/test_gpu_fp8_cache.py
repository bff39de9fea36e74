"""GPU parity of the FP8 prefix cache (bca_prefill_ex / bca_decode_ex) against the oracle.

* The codes and scales the prefill writes are bit-exact with ``oracle.quantize_fp8_rows`` on the
  same bf16 K/V, including an all-zero row and rows of bf16 subnormals (the scale floor).
* The prefill output does not depend on the cache format: bitwise equal to the prefill that
  writes a bf16 cache, and the unquantised K of the V-only format is a bitwise copy.
* The decode over an FP8 cache matches ``oracle.decode_cached`` over the oracle's own cache
  (quantised on the CPU from the same inputs) within the suite's tolerance, on both input
  distributions: in full at small sizes and ragged prefixes, on sampled rows at the CFG editing
  workload's full size.
* Strided cache views give bitwise the same decode as contiguous ones; P = 0 needs no cache.
"""
import numpy as np
import pytest

import bca_workloads as W
from oracle import bca_oracle as O

torch = pytest.importorskip("torch")
bca = pytest.importorskip("block_causal_attention_amd")

pytestmark = pytest.mark.gpu

MAX_TOL, MEAN_TOL = 1e-2, 1e-3
DEV = "cuda:0"
FORMATS = [("fp8_v", O.CACHE_FP8_V), ("fp8_kv", O.CACHE_FP8_KV)]


def say(*a):
    print(*a, flush=True)


def to_dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(DEV)


def f32(bits):
    return W.bf16_bits_to_f32(bits)


def check(got, ref, what):
    err = np.abs(np.asarray(got, dtype=np.float64) - np.asarray(ref, dtype=np.float64))
    say(f"  {what}: max|err|={err.max():.3e} mean|err|={err.mean():.3e} n={err.size}")
    assert np.isfinite(got).all(), what
    assert err.max() <= MAX_TOL and err.mean() <= MEAN_TOL, what


def poison_cache(plan, B, H, fmt):
    """A cache of the format whose every byte is garbage before the prefill writes it."""
    c = bca.KVCache.empty(plan, B, H, fmt, device=DEV)
    for t in (c.k, c.v):
        if t.dtype == torch.uint8:
            t.fill_(0x7F)  # the NaN code
        else:
            t.fill_(float("nan"))
    for t in (c.k_scale, c.v_scale):
        if t is not None:
            t.fill_(float("nan"))
    return c


def check_cache_exact(cache, kb, vb, P, heads=None):
    """Codes and scales bit-exact with the oracle's quantiser; bf16 tensors bit copies."""
    sel = slice(None) if heads is None else heads
    for name, t, sc, src, q in (("k", cache.k, cache.k_scale, kb, cache.k_quantized),
                                ("v", cache.v, cache.v_scale, vb, cache.v_quantized)):
        x = src[:, :P][:, :, sel]
        got = t[:, :, sel].cpu()
        if not q:
            assert torch.equal(got.view(torch.int16), torch.from_numpy(x.view(np.int16))), name
            continue
        codes, scales = O.quantize_fp8_rows(f32(x))
        gc = got.numpy()
        gs = sc[:, :, sel].cpu().numpy()
        bad = np.argwhere(gc != codes)
        assert bad.size == 0, (name, "codes differ at", bad[:5], gc[tuple(bad[0])], codes[tuple(bad[0])])
        assert np.array_equal(gs.view(np.uint32), scales.view(np.uint32)), (name, "scales differ")
        say(f"  cache.{name}: {codes.size} codes and {scales.size} scales bit-exact")


def oracle_cache(kb, vb, ids, fmt, heads=None):
    sel = slice(None) if heads is None else heads
    return O.prefix_cache_fp8(f32(kb[:, :, sel]), f32(vb[:, :, sel]), ids, fmt)


def plant_edge_rows(kb, vb, P):
    """An all-zero row and rows of bf16 subnormals inside the prefix (head 0)."""
    rng = np.random.default_rng(11)
    kb, vb = kb.copy(), vb.copy()
    for t in (kb, vb):
        t[:, min(3, P - 1), 0, :] = 0
        sub = rng.integers(1, 0x80, size=t[:, 0, 0, :].shape).astype(np.uint16)
        sub |= (rng.integers(0, 2, size=sub.shape).astype(np.uint16) << 15)
        t[:, min(5, P - 1), 0, :] = sub
        t[:, min(7, P - 1), 0, :] = sub | 0x0380  # normals near 2^-120: amax / 448 below the floor
    return kb, vb


# ---------------------------------------------------------------------------------------------
@pytest.mark.parametrize("fname,fmt", FORMATS)
@pytest.mark.parametrize("scaled", [True, False])
def test_tiny_fp8_prefill_codes_and_decode(fname, fmt, scaled):
    lay = W.TINY
    ids = lay.block_ids()
    say(f"case: tiny {fname} scaled={scaled}")
    qb, kb, vb = W.qkv(W.SEEDS["tiny"], lay.batch, lay.seq_len, lay.heads, scaled)
    plan = bca.Plan(ids)
    P = plan.info.prefix_len
    kb, vb = plant_edge_rows(kb, vb, P)
    B, S, H = lay.batch, lay.seq_len, lay.heads
    q, k, v = to_dev(qb), to_dev(kb), to_dev(vb)
    o_plain = bca.prefill(plan, q, k, v)
    cache = poison_cache(plan, B, H, fmt)
    o = bca.prefill_ex(plan, q, k, v, cache)
    torch.cuda.synchronize()
    assert torch.equal(o, o_plain), "the cache format changed the prefill output"
    check_cache_exact(cache, kb, vb, P)
    od = bca.decode_ex(plan, to_dev(qb[:, P:]), cache, to_dev(kb[:, P:]), to_dev(vb[:, P:]))
    torch.cuda.synchronize()
    ref = O.decode_cached(f32(qb[:, P:]), oracle_cache(kb, vb, ids, fmt), f32(kb[:, P:]),
                          f32(vb[:, P:]))
    check(od.cpu().numpy(), ref, "decode over FP8 cache vs oracle")


RANDOM_CASES = [(51, 40, 1, 2), (52, 129, 2, 2), (53, 300, 2, 3), (54, 777, 1, 2),
                (55, 1500, 2, 1)]


@pytest.mark.parametrize("fname,fmt", FORMATS)
@pytest.mark.parametrize("seed,S,B,H", RANDOM_CASES)
def test_random_layouts_fp8(fname, fmt, seed, S, B, H):
    rng = np.random.default_rng(seed)
    ids = W.random_layout(rng, S, p_text=0.5, max_seg=max(1, S // 3))
    ids[-max(1, S // 5):] = 10 ** 6  # a target image block last, so decode applies
    say(f"case: random layout {fname} seed={seed} S={S} B={B} H={H}")
    plan = bca.Plan(ids)
    P, N = plan.info.prefix_len, plan.info.target_len
    assert plan.info.decode_ok and P > 0
    qb, kb, vb = W.qkv(seed, B, S, H, scaled=False)
    q, k, v = to_dev(qb), to_dev(kb), to_dev(vb)
    cache = poison_cache(plan, B, H, fmt)
    o = bca.prefill_ex(plan, q, k, v, cache)
    torch.cuda.synchronize()
    assert torch.equal(o, bca.prefill(plan, q, k, v))
    check_cache_exact(cache, kb, vb, P)
    qt, kt, vt = W.qkv(seed + 1, B, N, H, scaled=False)
    od = bca.decode_ex(plan, to_dev(qt), cache, to_dev(kt), to_dev(vt))
    torch.cuda.synchronize()
    ref = O.decode_cached(f32(qt), oracle_cache(kb, vb, ids, fmt), f32(kt), f32(vt))
    check(od.cpu().numpy(), ref, "fresh-step decode over FP8 cache (sharp)")


@pytest.mark.parametrize("fname,fmt", FORMATS)
def test_cfg_fp8_full_size(fname, fmt):
    """The CFG editing workload (B = 2, S = 12,400, P = 8,304, N = 4,096, H = 32): the whole
    prefill writes the FP8 cache; three heads are checked bit-exact, and a fresh cached step on
    sampled rows against the oracle."""
    lay = W.EDIT_2REF_CFG
    ids = lay.block_ids()
    B, S, H = lay.batch, lay.seq_len, lay.heads
    say(f"case: CFG {fname} full size")
    qb, kb, vb = W.qkv(W.SEEDS["edit_2ref_cfg"], B, S, H, scaled=False)
    plan = bca.Plan(ids)
    P, N = plan.info.prefix_len, plan.info.target_len
    q, k, v = to_dev(qb), to_dev(kb), to_dev(vb)
    cache = poison_cache(plan, B, H, fmt)
    o = bca.prefill_ex(plan, q, k, v, cache)
    o_plain = bca.prefill(plan, q, k, v)
    torch.cuda.synchronize()
    assert torch.equal(o, o_plain)
    heads = [0, 17, 31]
    check_cache_exact(cache, kb, vb, P, heads=heads)
    for t in (cache.k, cache.v):  # no NaN code anywhere: every row was written
        if t.dtype == torch.uint8:
            assert not ((t & 0x7F) == 0x7F).any()
    for t in (cache.k_scale, cache.v_scale):
        if t is not None:
            assert torch.isfinite(t).all() and (t > 0).all()
    qt, kt, vt = W.decode_step_qkv(1, B, N, H, scaled=False)
    od = bca.decode_ex(plan, to_dev(qt), cache, to_dev(kt), to_dev(vt))
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([np.arange(0, N, 61), [N - 1]]))
    got = od[:, torch.from_numpy(rows).to(DEV)][:, :, heads].cpu().numpy()
    oc = oracle_cache(kb[:, :P], vb[:, :P], ids, fmt, heads=heads)
    ref = O.decode_cached(f32(qt[:, :, heads]), oc, f32(kt[:, :, heads]), f32(vt[:, :, heads]),
                          rows=rows)
    check(got, ref, "fresh-step decode over FP8 cache vs oracle")
    # Heads are independent: two of them as strided views make a grid small enough for the
    # 4-wave decode (the full one runs 12-wave workgroups in 384- and 256-row tiles); a row's
    # arithmetic is the same.
    two = slice(0, 2)
    sub = bca.KVCache(fmt, cache.k[:, :, two], cache.v[:, :, two],
                      None if cache.k_scale is None else cache.k_scale[:, :, two],
                      None if cache.v_scale is None else cache.v_scale[:, :, two])
    od2 = bca.decode_ex(plan, to_dev(qt)[:, :, two], sub, to_dev(kt)[:, :, two],
                        to_dev(vt)[:, :, two])
    torch.cuda.synchronize()
    assert torch.equal(od[:, :, two], od2)


def test_fp8_strided_cache_views():
    """Codes inside a wider buffer and scales as a [B, H, P] buffer seen as [B, P, H]: the
    prefill fills the views and the decode reads them bit-identically to contiguous ones."""
    rng = np.random.default_rng(8)
    S, B, H = 400, 2, 3
    ids = W.random_layout(rng, S, max_seg=90)
    ids[-70:] = 10 ** 6
    say("case: FP8 strided cache views")
    plan = bca.Plan(ids)
    P, N = plan.info.prefix_len, plan.info.target_len
    qb, kb, vb = W.qkv(8, B, S, H, scaled=False)
    q, k, v = to_dev(qb), to_dev(kb), to_dev(vb)
    fmt = bca.KVCache.FP8_KV
    dense = poison_cache(plan, B, H, fmt)
    bca.prefill_ex(plan, q, k, v, dense)
    kbuf = torch.zeros((B, P, H + 2, 128), dtype=torch.uint8, device=DEV)
    vbuf = torch.zeros((B, P, H + 2, 128), dtype=torch.uint8, device=DEV)
    ks = torch.zeros((B, H, P), dtype=torch.float32, device=DEV).transpose(1, 2)
    vs = torch.zeros((B, H, P), dtype=torch.float32, device=DEV).transpose(1, 2)
    strided = bca.KVCache(fmt, kbuf[:, :, 1:H + 1], vbuf[:, :, 1:H + 1], ks, vs)
    bca.prefill_ex(plan, q, k, v, strided)
    torch.cuda.synchronize()
    for a, b in ((dense.k, strided.k), (dense.v, strided.v), (dense.k_scale, strided.k_scale),
                 (dense.v_scale, strided.v_scale)):
        assert torch.equal(a, b)
    assert int(kbuf[:, :, 0].count_nonzero()) == 0 and int(kbuf[:, :, H + 1].count_nonzero()) == 0
    tq, tk, tv = to_dev(qb[:, P:]), to_dev(kb[:, P:]), to_dev(vb[:, P:])
    d1 = bca.decode_ex(plan, tq, dense, tk, tv)
    d2 = bca.decode_ex(plan, tq, strided, tk, tv)
    torch.cuda.synchronize()
    assert torch.equal(d1, d2)


def test_fp8_decode_without_prefix():
    S, B, H = 150, 1, 2
    ids = np.zeros(S, np.int32)
    say("case: FP8 decode with P = 0")
    plan = bca.Plan(ids)
    qb, kb, vb = W.qkv(12, B, S, H, scaled=False)
    cache = bca.KVCache.empty(plan, B, H, bca.KVCache.FP8_KV, device=DEV)
    o = bca.prefill_ex(plan, to_dev(qb), to_dev(kb), to_dev(vb), cache)
    od = bca.decode_ex(plan, to_dev(qb), None, to_dev(kb), to_dev(vb))
    torch.cuda.synchronize()
    ref = O.attention(f32(qb), f32(kb), f32(vb), ids)
    check(o.cpu().numpy(), ref, "prefill")
    check(od.cpu().numpy(), ref, "decode")


@pytest.mark.parametrize("fname,fmt", FORMATS)
def test_fp8_decode_tile_mix(fname, fmt):
    """A target height (N = 3,356, B = 2, H = 32) whose FP8 cached step runs 12-wave workgroups
    in 384-, 256- and 128-row tiles in one launch: sampled rows of three heads against the
    oracle, and two heads as strided views (a grid for the 4-wave decode) bitwise equal."""
    ids = W.block_ids_from_segments([("text", 45), ("image", 260), ("image", 3356)])
    B, H = 2, 32
    plan = bca.Plan(ids)
    P, N = plan.info.prefix_len, plan.info.target_len
    assert N == 3356
    assert bca.decode_layout(N, B * H, 1, fmt)[:4] == (12, 7, 2, 2)
    say(f"case: FP8 tile mix {fname} P={P} N={N}")
    qb, kb, vb = W.qkv(21, B, len(ids), H, scaled=False)
    cache = poison_cache(plan, B, H, fmt)
    bca.prefill_ex(plan, to_dev(qb), to_dev(kb), to_dev(vb), cache)
    qt, kt, vt = W.qkv(22, B, N, H, scaled=False)
    od = bca.decode_ex(plan, to_dev(qt), cache, to_dev(kt), to_dev(vt))
    torch.cuda.synchronize()
    heads = [0, 13, 31]
    rows = np.unique(np.concatenate([np.arange(0, N, 37), [383, 384, 2687, 2688, 3199, 3200,
                                                           3327, 3328, N - 1]]))
    got = od[:, torch.from_numpy(rows).to(DEV)][:, :, heads].cpu().numpy()
    oc = oracle_cache(kb, vb, ids, fmt, heads=heads)
    ref = O.decode_cached(f32(qt[:, :, heads]), oc, f32(kt[:, :, heads]), f32(vt[:, :, heads]),
                          rows=rows)
    check(got, ref, "tile-mix decode over FP8 cache vs oracle")
    two = slice(5, 7)
    assert bca.decode_layout(N, B * 2, 1, fmt)[0] == 4
    sub = bca.KVCache(fmt, cache.k[:, :, two], cache.v[:, :, two],
                      None if cache.k_scale is None else cache.k_scale[:, :, two],
                      None if cache.v_scale is None else cache.v_scale[:, :, two])
    od2 = bca.decode_ex(plan, to_dev(qt)[:, :, two], sub, to_dev(kt)[:, :, two],
                        to_dev(vt)[:, :, two])
    torch.cuda.synchronize()
    assert torch.equal(od[:, :, two], od2)
