"""GPU tests of the prefix-cache expansion (bca_cache_dequantize).

* Codes and scales made by the oracle's quantiser (not by the HIP path) are expanded on the GPU;
  every value must be the exact product E4M3(code) * scale rounded to fp32, then to bf16 (RNE),
  bit for bit, and within half a bf16 ulp (plus an fp32 one) of the exact product.  Rows of zeros
  (scale 1) and rows of tiny values (floored scale) are included; a bf16 tensor is copied.
* Decoding over the expanded cache with the bf16 decode matches the oracle's decode over the
  oracle's FP8 cache, and is bitwise the decode over the FP8 cache itself (the FP8 decode turns
  its codes into the same bf16 tiles the bf16 decode loads, and walks them the same way), on a
  random layout and on the two-reference editing shape at full size (P = 8,304, N = 4,096,
  H = 32).
* Strided (non-contiguous) inputs and outputs.
"""
import os
from concurrent.futures import ThreadPoolExecutor

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


def bits_of(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def oracle_cache(seed, B, P, H, fmt):
    """K, V drawn with a spread of row magnitudes, zero rows and tiny rows; quantised by the
    oracle.  Returns (k bits, v bits, oracle cache dict)."""
    rng = np.random.default_rng(seed)
    shape = (B, P, H, 128)
    mag = np.exp(rng.uniform(-6, 6, size=shape[:3] + (1,))).astype(np.float32)
    k = rng.standard_normal(shape, dtype=np.float32) * mag
    v = rng.standard_normal(shape, dtype=np.float32) * mag[:, ::-1]
    k[:, 3], v[:, 5] = 0.0, 0.0                              # all-zero rows: scale 1
    v[:, 7] *= np.float32(2.0 ** -120)                       # tiny rows: floored scale
    kb, vb = W.f32_to_bf16_bits(k), W.f32_to_bf16_bits(v)
    oc = {"format": fmt, "k": f32(kb), "v": f32(vb)}
    if fmt != O.CACHE_BF16:
        oc["v"] = O.quantize_fp8_rows(f32(vb))
    if fmt == O.CACHE_FP8_KV:
        oc["k"] = O.quantize_fp8_rows(f32(kb))
    return kb, vb, oc


def upload(oc, kb, vb):
    fmt = oc["format"]

    def tens(t, bits):
        if isinstance(t, tuple):
            codes, scales = t
            return (torch.from_numpy(np.ascontiguousarray(codes)).to(DEV),
                    torch.from_numpy(np.ascontiguousarray(scales)).to(DEV))
        return to_dev(bits), None

    k, ks = tens(oc["k"], kb)
    v, vs = tens(oc["v"], vb)
    return bca.KVCache(fmt, k, v, ks, vs)


def expected_bits(t, bits):
    """The expansion's value: the exact product rounded to fp32, then to bf16 (a bf16 tensor:
    its own bits)."""
    if not isinstance(t, tuple):
        return bits
    exact = O.dequantize_fp8_rows(*t)                        # float64, exact
    return W.f32_to_bf16_bits(exact.astype(np.float32)), exact


@pytest.mark.parametrize("fmt", [bca.KVCache.BF16, bca.KVCache.FP8_V, bca.KVCache.FP8_KV])
def test_expansion_bit_exact_against_oracle_codes(fmt):
    B, P, H = 2, 333, 3
    kb, vb, oc = oracle_cache(71 + fmt, B, P, H, fmt)
    cache = upload(oc, kb, vb)
    say(f"case: expansion fmt={fmt} B={B} P={P} H={H}")
    out = bca.dequantize_cache(cache)
    torch.cuda.synchronize()
    for name, t, bits in (("k", oc["k"], kb), ("v", oc["v"], vb)):
        got = bits_of(getattr(out, name))
        e = expected_bits(t, bits)
        if isinstance(e, tuple):
            want, exact = e
            assert np.array_equal(got, want), name
            g = f32(got).astype(np.float64)
            ulp32 = np.spacing(np.abs(exact).astype(np.float32)).astype(np.float64)
            bound = 2.0 ** 15 * ulp32 + ulp32
            # half a bf16 ulp of the value (2^16 fp32 ulps / 2) plus one fp32 ulp
            assert (np.abs(g - exact) <= bound).all(), name
        else:
            assert np.array_equal(got, e), name


def test_expansion_strided_views():
    B, P, H = 1, 200, 4
    kb, vb, oc = oracle_cache(75, B, P, H, bca.KVCache.FP8_KV)
    (kc, ks), (vc, vs) = oc["k"], oc["v"]
    # codes stored inside wider buffers: [B, P, H, 256] and scales [B, P, H, 2], sliced
    kbig = torch.zeros((B, P, H, 256), dtype=torch.uint8, device=DEV)
    kbig[..., 64:192] = torch.from_numpy(kc).to(DEV)
    vbig = torch.zeros((B, P, H, 256), dtype=torch.uint8, device=DEV)
    vbig[..., :128] = torch.from_numpy(vc).to(DEV)
    ksbig = torch.zeros((B, P, H, 2), dtype=torch.float32, device=DEV)
    ksbig[..., 1] = torch.from_numpy(ks).to(DEV)
    vsbig = torch.zeros((B, P, H, 2), dtype=torch.float32, device=DEV)
    vsbig[..., 0] = torch.from_numpy(vs).to(DEV)
    cache = bca.KVCache(bca.KVCache.FP8_KV, kbig[..., 64:192], vbig[..., :128], ksbig[..., 1],
                        vsbig[..., 0])
    obig = torch.full((B, P, 2 * H, 128), 3.0, dtype=torch.bfloat16, device=DEV)
    out = bca.KVCache(bca.KVCache.BF16, obig[:, :, :H], obig[:, :, H:])
    say("case: expansion strided")
    bca.dequantize_cache(cache, out)
    torch.cuda.synchronize()
    for name, t in (("k", oc["k"]), ("v", oc["v"])):
        want, _ = expected_bits(t, None)
        assert np.array_equal(bits_of(getattr(out, name)), want), name


def _fp8_decode_pair(ids, B, H, fmt, seed):
    plan = bca.Plan(ids)
    P = plan.info.prefix_len
    qb, kb, vb = W.qkv(seed, B, len(ids), H, scaled=False)
    cache = bca.KVCache.empty(plan, B, H, fmt, device=DEV)
    bca.prefill_ex(plan, to_dev(qb), to_dev(kb), to_dev(vb), cache)
    q, k, v = to_dev(qb[:, P:]), to_dev(kb[:, P:]), to_dev(vb[:, P:])
    fused = bca.decode_ex(plan, q, cache, k, v)
    wide = bca.dequantize_cache(cache)
    expanded = bca.decode_ex(plan, q, wide, k, v)
    torch.cuda.synchronize()
    return plan, (qb, kb, vb), fused, expanded


def check(got, ref, what):
    err = np.abs(np.asarray(got, np.float64) - np.asarray(ref, np.float64))
    say(f"  {what}: max|err|={err.max():.3e} mean|err|={err.mean():.3e}")
    assert np.isfinite(got).all() and err.max() <= MAX_TOL and err.mean() <= MEAN_TOL, what


@pytest.mark.parametrize("fmt", [bca.KVCache.FP8_V, bca.KVCache.FP8_KV])
def test_decode_over_expansion_matches_the_fp8_decode(fmt):
    rng = np.random.default_rng(77)
    ids = W.random_layout(rng, 1100, max_seg=250)
    ids[-200:] = 10 ** 6
    B, H = 2, 2
    say(f"case: decode over expansion fmt={fmt}")
    plan, (qb, kb, vb), fused, expanded = _fp8_decode_pair(ids, B, H, fmt, 77)
    P = plan.info.prefix_len
    oc = O.prefix_cache_fp8(f32(kb), f32(vb), ids, fmt)
    ref = O.decode_cached(f32(qb[:, P:]), oc, f32(kb[:, P:]), f32(vb[:, P:]))
    check(expanded.cpu().numpy(), ref, "expanded, bf16 decode vs oracle")
    assert np.array_equal(expanded.cpu().numpy(), fused.cpu().numpy()), "expanded vs FP8 decode"


@pytest.mark.parametrize("fmt", [bca.KVCache.FP8_V, bca.KVCache.FP8_KV])
def test_decode_over_expansion_full_size(fmt):
    lay = W.EDIT_2REF
    say(f"case: decode over expansion, 2-ref edit full size, fmt={fmt}")
    ids = lay.block_ids()
    plan, (qb, kb, vb), fused, expanded = _fp8_decode_pair(ids, 1, lay.heads, fmt,
                                                           W.SEEDS["edit_2ref"])
    P, N, H = plan.info.prefix_len, plan.info.target_len, lay.heads
    assert (P, N) == (8304, 4096)
    assert np.array_equal(expanded.cpu().numpy(), fused.cpu().numpy()), \
        "expanded vs the FP8 decode, full size"
    # and both against the oracle's decode over the oracle's own FP8 cache, every row and head
    # (one thread per head: NumPy releases the interpreter lock in its products)
    oc = O.prefix_cache_fp8(f32(kb), f32(vb), ids, fmt)
    ockv = O.cache_values(oc)
    qf, kf, vf = f32(qb[:, P:]), f32(kb[:, P:]), f32(vb[:, P:])
    with ThreadPoolExecutor(max(1, min(16, os.cpu_count() or 1))) as ex:
        parts = list(ex.map(lambda h: O.decode(qf, *ockv, kf, vf, heads=[h]), range(H)))
    ref = np.concatenate(parts, axis=2)
    check(expanded.cpu().numpy(), ref, "expanded, bf16 decode vs oracle, full size")
    check(fused.cpu().numpy(), ref, "FP8 decode vs oracle, full size")
