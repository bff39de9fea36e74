"""GPU tests of the prefill that hands its target rows to the cached step's kernels (two
launches, bca_prefill_layout out[0] = 2): outputs and caches against the one-launch prefill and
the CPU oracle.

A row's result does not depend on the launch that computes it, so batch item 0 of a B = 2
prefill (one launch: its grid fills two rounds) must equal the B = 1 prefill of the same rows
(two launches) bit for bit.  The text-to-image 1024^2 prefill at B = 1 (every row and head
against the oracle in test_gpu_parity_full.py) takes the two launches too.
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


CASES = [
    ("t2i 1024^2", [("text", 256), ("image", 4096)]),
    ("two prefix tiles, the first partial", [("text", 77), ("image", 640), ("text", 9),
                                             ("image", 3000)]),
    ("prefix under one tile", [("text", 5), ("image", 3200)]),
]


@pytest.mark.parametrize("name,segs", CASES)
def test_two_launch_prefill_equals_one_launch(name, segs):
    ids = W.block_ids_from_segments(segs)
    S, H = len(ids), 32
    plan = bca.Plan(ids)
    P, N = plan.info.prefix_len, plan.info.target_len
    one, two = bca.prefill_layout(plan, 2, H), bca.prefill_layout(plan, 1, H)
    say(f"case: {name} S={S} P={P} N={N} layout B=1 {two} B=2 {one}")
    assert two[0] == 2 and one[0] == 1
    qb, kb, vb = W.qkv(31, 2, S, H, scaled=False)
    q, k, v = to_dev(qb), to_dev(kb), to_dev(vb)
    kc2 = torch.full((2, P, H, 128), float("nan"), dtype=torch.bfloat16, device=DEV)
    vc2 = torch.full_like(kc2, float("nan"))
    o2 = bca.prefill(plan, q, k, v, k_cache=kc2, v_cache=vc2)
    kc1 = torch.full((1, P, H, 128), float("nan"), dtype=torch.bfloat16, device=DEV)
    vc1 = torch.full_like(kc1, float("nan"))
    o1 = bca.prefill(plan, q[:1].contiguous(), k[:1].contiguous(), v[:1].contiguous(),
                     k_cache=kc1, v_cache=vc1)
    torch.cuda.synchronize()
    assert torch.equal(o1[0], o2[0]), "two launches differ from one"
    for c in (kc1, vc1, kc2[:1], vc2[:1]):
        assert not torch.isnan(c.float()).any()
    assert torch.equal(kc1.view(torch.int16).cpu(), torch.from_numpy(kb[:1, :P].view(np.int16)))
    assert torch.equal(vc1.view(torch.int16).cpu(), torch.from_numpy(vb[:1, :P].view(np.int16)))
    heads = [0, 31]
    rows = np.unique(np.r_[np.arange(0, S, 29), P - 1, P, S - 1])
    ref = O.attention(f32(qb[:1, :, heads]), f32(kb[:1, :, heads]), f32(vb[:1, :, heads]), ids,
                      rows=rows)
    got = o1[:, torch.from_numpy(rows).to(DEV)][:, :, heads].cpu().numpy()
    check(got, ref, "two-launch prefill vs oracle (sampled rows)")


@pytest.mark.parametrize("fmt", [1, 2])
def test_two_launch_prefill_writes_the_fp8_cache(fmt):
    """bca_prefill_ex over an FP8 cache through the two launches: the same output as the bf16
    prefill, codes and scales bit-exact with the oracle's quantiser."""
    lay = W.T2I_1024
    ids = lay.block_ids()
    S, H = lay.seq_len, lay.heads
    plan = bca.Plan(ids)
    assert bca.prefill_layout(plan, 1, H)[0] == 2
    P = plan.info.prefix_len
    say(f"case: t2i FP8 cache format {fmt}")
    qb, kb, vb = W.qkv(W.SEEDS["t2i_1024"], 1, S, H, scaled=False)
    q, k, v = to_dev(qb), to_dev(kb), to_dev(vb)
    cache = bca.KVCache.empty(plan, 1, H, fmt, device=DEV)
    o = bca.prefill_ex(plan, q, k, v, cache)
    o_plain = bca.prefill(plan, q, k, v)
    torch.cuda.synchronize()
    assert torch.equal(o, o_plain)
    for t, sc, src, quant in ((cache.k, cache.k_scale, kb, cache.k_quantized),
                              (cache.v, cache.v_scale, vb, cache.v_quantized)):
        if not quant:
            assert torch.equal(t.view(torch.int16).cpu(), torch.from_numpy(src[:, :P].view(np.int16)))
            continue
        codes, scales = O.quantize_fp8_rows(f32(src[:, :P]))
        assert np.array_equal(t.cpu().numpy(), codes)
        assert np.array_equal(sc.cpu().numpy().view(np.uint32), scales.view(np.uint32))
