"""Plain, slow, float64 CPU oracle of block-causal attention (TEST INFRASTRUCTURE).

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline`` leg may import
this module.  It materialises the visibility mask from its definition and runs dense softmax
attention in float64; nothing here is blocked, fused or reordered beyond computing one (batch,
head) pair and one chunk of query rows at a time.

Sources (web pages, cited by title and section):

* [QI21-guide] "Qwen-Image 2.1: Block-Causal Attention, Prefix KV Cache, and Turbo" (flozi.net
  guide, English; the German edition has the same sections).  Sections used: "One stream for
  text, reference images, and the target", "Block-causal attention is the cache-enabling
  boundary", "Timestep-zero conditioning makes the prefix invariant", "The prefix cache is a
  compute-for-memory trade", "Two exact attention paths, with different operating requirements".
* [QI21-article] the 10100.com article on Qwen-Image 2.1 inference (Chinese): its Block-Causal
  mask part (the rule written as a boolean expression), its piecewise-attention part (the
  bottom-right aligned causal mask for a text segment whose Q length is shorter than its K
  length) and its prefix-KV-cache part (prefill on step 1, mask-free decode afterwards).

Parity pins (tests/test_oracle_pins.py): every function below is pinned by a check that does not
reuse its own formula -- brute force of the rule as stated in words, the per-segment
construction, the pages' worked 3x8 example, closed forms (Q = 0), reductions to
``torch.nn.functional.scaled_dot_product_attention`` (unmasked, causal, piecewise segment calls),
prefix invariance, decode == prefill rows, and the pages' cache-size figures.  The FP8 cache
functions (tests/test_oracle_fp8_pins.py) are pinned to the E4M3 definition (closed-form codes,
brute-force nearest value over all 256 codes, tie midpoints), the half-ulp error bound, exact
round trips and the pages' "V-only saves about a quarter".  The batch-of-sequences functions
(tests/test_oracle_varlen_pins.py) are pinned to a dense construction of the rule over the whole
row axis, and the batched cached step to the prefill rows of each sequence.  No function here is
"parity unpinned".
"""
from __future__ import annotations

from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

TEXT = -1
ROW_CHUNK = 1024  # query rows per dense block; bounds memory at S = 32,912


class OracleInputError(ValueError):
    """Raised for block-id vectors the rule does not define."""


# ----------------------------------------------------------------------------------------------
# Block ids and runs
# ----------------------------------------------------------------------------------------------
def validate_block_ids(ids: Sequence[int]) -> np.ndarray:
    """Check a block-id vector: -1 for text, k >= 0 for image block k.

    [QI21-guide, "Block-causal attention is the cache-enabling boundary"]: every position gets an
    identifier, -1 for text, a unique non-negative identifier per reference image and another
    one for the target; adjacent images keep distinct identifiers.  Reading: an image id must
    occupy exactly one contiguous run (a reused id would let an earlier run see a later one, which
    the same section rules out), so reuse is rejected rather than honoured.
    """
    a = np.asarray(ids)
    if a.ndim != 1 or a.size < 1:
        raise OracleInputError("block ids must be a non-empty 1-D vector")
    a = a.astype(np.int64)
    if (a < TEXT).any():
        raise OracleInputError("block ids must be >= -1")
    seen = set()
    for start, end, bid in runs(a, _validated=True):
        if bid >= 0:
            if bid in seen:
                raise OracleInputError(f"image block id {bid} occupies more than one run")
            seen.add(bid)
    return a


def runs(ids: Sequence[int], _validated: bool = False) -> List[Tuple[int, int, int]]:
    """Maximal runs of equal id as (start, end, id), end exclusive."""
    a = np.asarray(ids).astype(np.int64)
    out: List[Tuple[int, int, int]] = []
    start = 0
    for i in range(1, a.size + 1):
        if i == a.size or a[i] != a[start]:
            out.append((start, i, int(a[start])))
            start = i
    return out


def prefix_split(ids: Sequence[int]) -> Tuple[int, int, bool]:
    """(P, N, decode_ok): the prefix is everything before the last block.

    [QI21-guide, "Timestep-zero conditioning makes the prefix invariant"]: the cache holds the
    text and reference positions, i.e. everything before the target, which is the final block;
    N target queries score P + N keys.  Cached decode needs that final block to be an image block
    ([QI21-article], prefix-KV-cache part: the target is the last complete image block, so its rows
    need no mask).
    """
    a = validate_block_ids(ids)
    last = runs(a)[-1]
    P = last[0]
    return P, a.size - P, last[2] >= 0


# ----------------------------------------------------------------------------------------------
# The mask, from its definition
# ----------------------------------------------------------------------------------------------
def visibility_mask(ids: Sequence[int], rows: Optional[np.ndarray] = None) -> np.ndarray:
    """M[i, j] = (i >= j) or (i and j are in the same image block).

    [QI21-article], Block-Causal mask part: a query sees a key when the key is not later than the
    query, or when both belong to one image block.  Text is -1 and is strictly causal ([QI21-guide], "Block-causal attention
    is the cache-enabling boundary"), so "same image block" requires a non-negative id.
    Returns bool [len(rows), S] (all rows when ``rows`` is None).
    """
    a = validate_block_ids(ids)
    S = a.size
    r = np.arange(S) if rows is None else np.asarray(rows, dtype=np.int64)
    i = r[:, None]
    j = np.arange(S)[None, :]
    same_image = (a[r][:, None] >= 0) & (a[r][:, None] == a[None, :])
    return (i >= j) | same_image


# ----------------------------------------------------------------------------------------------
# Attention
# ----------------------------------------------------------------------------------------------
def _softmax_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float,
                       mask: Optional[np.ndarray]) -> np.ndarray:
    """softmax(scale * q k^T, masked) v for one head, float64 throughout."""
    s = (q @ k.T) * scale
    if mask is not None:
        if not mask.any(axis=1).all():
            raise AssertionError("a query row with no visible key")
        s = np.where(mask, s, -np.inf)
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    p = e / e.sum(axis=1, keepdims=True)
    return p @ v


def default_scale(head_dim: int) -> float:
    """Softmax scale when none is given: 1/sqrt(D), the default of the exact attention calls the
    pages' default processor issues ([QI21-guide], "Two exact attention paths ...").  Reading:
    the pages never state the scale."""
    return 1.0 / np.sqrt(head_dim)


def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, ids: Sequence[int],
              scale: Optional[float] = None, rows: Optional[Sequence[int]] = None,
              batches: Optional[Sequence[int]] = None,
              heads: Optional[Sequence[int]] = None) -> np.ndarray:
    """Block-causal prefill attention, float64, for [B, S, H, D] inputs.

    For every (b, h): s = scale * Q K^T, s[i, j] = -inf where M[i, j] is False, row softmax,
    O = p V ([QI21-guide], "Block-causal attention is the cache-enabling boundary").  Returns
    float64 [len(batches), len(rows), len(heads), D]; callers round to float32 if they want the
    stored precision.  ``rows``/``batches``/``heads`` select a subset (default: all).
    """
    a = validate_block_ids(ids)
    B, S, H, D = q.shape
    if a.size != S or k.shape != q.shape or v.shape != q.shape:
        raise OracleInputError("shape mismatch")
    sc = default_scale(D) if not scale else float(scale)
    rsel = np.arange(S) if rows is None else np.asarray(rows, dtype=np.int64)
    bsel = range(B) if batches is None else list(batches)
    hsel = range(H) if heads is None else list(heads)
    out = np.empty((len(bsel), rsel.size, len(hsel), D), dtype=np.float64)
    for c0 in range(0, rsel.size, ROW_CHUNK):
        rr = rsel[c0:c0 + ROW_CHUNK]
        m = visibility_mask(a, rr)
        for bi, b in enumerate(bsel):
            for hi_, h in enumerate(hsel):
                qq = q[b, rr, h, :].astype(np.float64)
                kk = k[b, :, h, :].astype(np.float64)
                vv = v[b, :, h, :].astype(np.float64)
                out[bi, c0:c0 + rr.size, hi_, :] = _softmax_attention(qq, kk, vv, sc, m)
    return out


def prefix_cache(k: np.ndarray, v: np.ndarray, ids: Sequence[int]) -> Tuple[np.ndarray, np.ndarray]:
    """The per-layer prefix K/V: copies (not views) of positions [0, P).

    [QI21-guide], "Timestep-zero conditioning makes the prefix invariant": the extract step stores
    the prefix K/V and the implementation clones the prefix slices.
    """
    P, _, _ = prefix_split(ids)
    return k[:, :P].copy(), v[:, :P].copy()


def decode(q_t: np.ndarray, k_cache: np.ndarray, v_cache: np.ndarray, k_t: np.ndarray,
           v_t: np.ndarray, scale: Optional[float] = None, rows: Optional[Sequence[int]] = None,
           batches: Optional[Sequence[int]] = None,
           heads: Optional[Sequence[int]] = None) -> np.ndarray:
    """Cached step: target queries attend, with no mask, to [cached prefix K/V ; target K/V].

    [QI21-article], prefix-KV-cache part: Query = current target latents, Key/Value = cached
    prefix K/V + current target K/V, one full attention with no mask; [QI21-guide], "Two exact
    attention paths ...": target rows have full access to [cached prefix, target].
    Returns float64 [len(batches), len(rows), len(heads), D] (default: all of them).
    """
    B, N, H, D = q_t.shape
    P = k_cache.shape[1]
    if k_t.shape != q_t.shape or v_t.shape != q_t.shape or v_cache.shape != k_cache.shape:
        raise OracleInputError("shape mismatch")
    if k_cache.shape[0] != B or k_cache.shape[2] != H or k_cache.shape[3] != D:
        raise OracleInputError("cache shape mismatch")
    sc = default_scale(D) if not scale else float(scale)
    rsel = np.arange(N) if rows is None else np.asarray(rows, dtype=np.int64)
    bsel = range(B) if batches is None else list(batches)
    hsel = range(H) if heads is None else list(heads)
    out = np.empty((len(bsel), rsel.size, len(hsel), D), dtype=np.float64)
    for bi, b in enumerate(bsel):
        for hi_, h in enumerate(hsel):
            kk = np.concatenate([k_cache[b, :, h, :], k_t[b, :, h, :]]).astype(np.float64)
            vv = np.concatenate([v_cache[b, :, h, :], v_t[b, :, h, :]]).astype(np.float64)
            assert kk.shape[0] == P + N
            for c0 in range(0, rsel.size, ROW_CHUNK):
                rr = rsel[c0:c0 + ROW_CHUNK]
                qq = q_t[b, rr, h, :].astype(np.float64)
                out[bi, c0:c0 + rr.size, hi_, :] = _softmax_attention(qq, kk, vv, sc, None)
    return out


# ----------------------------------------------------------------------------------------------
# Plan derived from the mask
# ----------------------------------------------------------------------------------------------
def row_key_limits(ids: Sequence[int]) -> np.ndarray:
    """hi[i] = 1 + (last visible key of row i), read off the materialised mask.

    Also checks that every mask row is a prefix: M[i, :hi[i]] all True and M[i, hi[i]:] all
    False.  (Not stated on the pages; it follows from the rule, and the check makes the mask's
    shape explicit rather than assumed.)
    """
    a = validate_block_ids(ids)
    S = a.size
    hi = np.empty(S, dtype=np.int64)
    for c0 in range(0, S, ROW_CHUNK):
        rr = np.arange(c0, min(S, c0 + ROW_CHUNK))
        m = visibility_mask(a, rr)
        last = S - 1 - np.argmax(m[:, ::-1], axis=1)
        hi[rr] = last + 1
        prefix = np.arange(S)[None, :] < hi[rr][:, None]
        if not np.array_equal(m, prefix):
            raise AssertionError("a mask row is not a prefix of the keys")
    return hi


def plan_from_mask(ids: Sequence[int], block_m: int) -> Dict[str, np.ndarray]:
    """Per-query-tile key ranges derived from the mask, for bit-exact comparison with a planner.

    The pages fix no partition of the queries into tiles; the reading taken here (and by the
    planner) is that the nt = ceil(S / block_m) tiles end at the sequence's end, so only the
    first one may be partial: tile t holds rows [max(0, S - (nt-t)*block_m), S - (nt-1-t)*block_m)
    (``tile_first`` gives S - (nt-t)*block_m, negative for a partial first tile).  Then
    kv_full[t] = min hi over its rows (every key below it is visible to every row of the tile),
    kv_end[t] = max hi (no row sees a key at or beyond it).  ``order`` lists the tiles by kv_end
    descending, ties by tile index ascending.  ``segments`` are the maximal equal-id runs
    (start, end, id).
    """
    a = validate_block_ids(ids)
    S = a.size
    hi = row_key_limits(a)
    nt = -(-S // block_m)
    kv_full = np.empty(nt, dtype=np.int64)
    kv_end = np.empty(nt, dtype=np.int64)
    tile_first = np.empty(nt, dtype=np.int64)
    for t in range(nt):
        first = S - (nt - t) * block_m
        seg = hi[max(0, first):first + block_m]
        tile_first[t] = first
        kv_full[t] = seg.min()
        kv_end[t] = seg.max()
    order = np.array(sorted(range(nt), key=lambda t: (-kv_end[t], t)), dtype=np.int64)
    P, N, ok = prefix_split(a)
    return {
        "segments": np.array(runs(a), dtype=np.int64).reshape(-1, 3),
        "row_limit": hi,
        "kv_full": kv_full,
        "kv_end": kv_end,
        "tile_first": tile_first,
        "order": order,
        "prefix_len": np.int64(P),
        "target_len": np.int64(N),
        "decode_ok": np.int64(1 if ok else 0),
        "useful_pairs": np.int64(hi.sum()),
    }


def prefix_cache_bytes(layers: int, batch: int, prefix_len: int, heads: int, head_dim: int,
                       bytes_per_scalar: int) -> int:
    """Logical prefix-K/V payload: two tensors (K and V) of [batch, prefix, heads, head_dim] per
    layer ([QI21-guide], "The prefix cache is a compute-for-memory trade")."""
    return 2 * layers * batch * prefix_len * heads * head_dim * bytes_per_scalar


# ----------------------------------------------------------------------------------------------
# FP8 prefix cache
# ----------------------------------------------------------------------------------------------
# [QI21-article], FP8 part: the prefix K/V cache can be stored as FP8 E4M3 with one FP32 scale per
# token and per attention head; quantising only V saves about 25% of the cache and is the safer
# trade (K carries RoPE and drives the attention weights).  Readings: E4M3 is the OCP "E4M3FN"
# encoding (1 sign, 4 exponent bits with bias 7, 3 mantissa bits, subnormals, no infinities,
# S.1111.111 = NaN, largest finite 448); the scale of a (token, head) row is the smallest power of
# two 2^k with amax(|x|) <= 448 * 2^k, k >= -126 (the smallest normal fp32 number; 1 for an
# all-zero row), so the row's largest value lands in E4M3's top binade; a row is quantised as
# x * 2^-k (exact in fp32) rounded to the nearest E4M3 value, ties to the even code (|x| * 2^-k
# never exceeds 448); a stored value is E4M3(code) * 2^k, exact.

E4M3_MAX = 448.0
SCALE_FLOOR = 2.0 ** -126  # smallest normal fp32 number
CACHE_BF16, CACHE_FP8_V, CACHE_FP8_KV = 0, 1, 2


def e4m3_value_table() -> np.ndarray:
    """float64 value of each of the 256 E4M3 codes (NaN for the two NaN codes)."""
    vals = np.empty(256, dtype=np.float64)
    for code in range(256):
        sign = -1.0 if code & 0x80 else 1.0
        e = (code >> 3) & 0xF
        m = code & 0x7
        if e == 0xF and m == 0x7:
            vals[code] = np.nan
        elif e == 0:
            vals[code] = sign * (m / 8.0) * 2.0 ** (1 - 7)
        else:
            vals[code] = sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return vals


_E4M3 = e4m3_value_table()
_E4M3_POS = _E4M3[:0x7F]  # codes 0x00..0x7E: 0 and the 126 positive finite values, ascending


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    return _E4M3[np.asarray(codes, dtype=np.uint8)]


def e4m3_encode(x: np.ndarray) -> np.ndarray:
    """Nearest finite E4M3 code, ties to the even code; |x| above 448 saturates; NaN -> 0x7F."""
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    hi = np.clip(np.searchsorted(_E4M3_POS, a, side="left"), 0, 0x7E)
    lo = np.clip(hi - 1, 0, 0x7E)
    dlo = np.abs(a - _E4M3_POS[lo])
    dhi = np.abs(_E4M3_POS[hi] - a)
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    code = np.where(a > E4M3_MAX, np.uint8(0x7E), code)
    code = np.where(np.signbit(x), code | np.uint8(0x80), code).astype(np.uint8)
    return np.where(np.isnan(x), np.uint8(0x7F), code).astype(np.uint8)


def fp8_row_scale(amax: np.ndarray) -> np.ndarray:
    """The scale of rows with these amax values: the smallest power of two 2^k with
    amax <= 448 * 2^k, at least 2^-126; 1 for amax = 0.  float32."""
    a = np.asarray(amax, dtype=np.float64)
    k = np.zeros(a.shape, dtype=np.int64)
    pos = a > 0
    k[pos] = np.ceil(np.log2(a[pos] / E4M3_MAX)).astype(np.int64)
    # log2 may land one off next to a power of two: settle k by exact comparisons
    for _ in range(2):
        k = np.where(pos & (a > E4M3_MAX * np.exp2(k.astype(np.float64))), k + 1, k)
        k = np.where(pos & (a <= E4M3_MAX * np.exp2((k - 1).astype(np.float64))), k - 1, k)
    k = np.where(pos, np.maximum(k, int(np.log2(SCALE_FLOOR))), 0)
    return np.exp2(k.astype(np.float64)).astype(np.float32)


def quantize_fp8_rows(x: np.ndarray):
    """Per-row (last axis) FP8 quantisation with fp32 scales, as the method fixes them.

    Returns (codes uint8 like x, scales float32 of x.shape[:-1])."""
    xf = np.asarray(x, dtype=np.float32)
    amax = np.max(np.abs(xf), axis=-1)
    # Reading: one power-of-two scale per row, the smallest that keeps the row within E4M3's
    # range (its largest value then uses E4M3's top binade, so no relative precision is lost),
    # floored at the smallest normal fp32 number; x * 2^-k is exact.
    scale = fp8_row_scale(amax)
    inv = (np.float32(1.0) / scale).astype(np.float32)
    q = (xf * inv[..., None]).astype(np.float32)
    return e4m3_encode(q), scale


def dequantize_fp8_rows(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """code value * scale, exact in float64 (and in bf16 down to bf16's smallest normal)."""
    return e4m3_decode(codes) * np.asarray(scales, dtype=np.float64)[..., None]


def prefix_cache_fp8(k: np.ndarray, v: np.ndarray, ids: Sequence[int], fmt: int) -> Dict:
    """The prefix cache in a given format: V quantised for CACHE_FP8_V, K and V for
    CACHE_FP8_KV, nothing for CACHE_BF16.  Quantised tensors are (codes, scales)."""
    kc, vc = prefix_cache(k, v, ids)
    out = {"format": fmt, "k": kc, "v": vc}
    if fmt in (CACHE_FP8_V, CACHE_FP8_KV):
        out["v"] = quantize_fp8_rows(vc)
    if fmt == CACHE_FP8_KV:
        out["k"] = quantize_fp8_rows(kc)
    return out


def cache_values(cache: Dict):
    """float64 K and V of a prefix cache as the decode sees them."""
    def val(t):
        return dequantize_fp8_rows(*t) if isinstance(t, tuple) else np.asarray(t, np.float64)
    return val(cache["k"]), val(cache["v"])


def decode_cached(q_t, cache: Dict, k_t, v_t, scale: Optional[float] = None, **sel) -> np.ndarray:
    """Cached step over a prefix cache in any format: dequantise, then the plain decode."""
    kc, vc = cache_values(cache)
    return decode(q_t, kc, vc, k_t, v_t, scale=scale, **sel)


def prefix_cache_bytes_fp8(layers: int, batch: int, prefix_len: int, heads: int, head_dim: int,
                           fmt: int) -> int:
    """Payload of the prefix cache in a format: 2 bytes per bf16 scalar, 1 per FP8 code and 4
    per (token, head) scale of each quantised tensor."""
    per_tensor_bf16 = prefix_len * heads * head_dim * 2
    per_tensor_fp8 = prefix_len * heads * head_dim + prefix_len * heads * 4
    n_fp8 = {CACHE_BF16: 0, CACHE_FP8_V: 1, CACHE_FP8_KV: 2}[fmt]
    return layers * batch * ((2 - n_fp8) * per_tensor_bf16 + n_fp8 * per_tensor_fp8)


# ----------------------------------------------------------------------------------------------
# Q/K prologue: per-head RMS normalisation, then three-axis RoPE
# ----------------------------------------------------------------------------------------------
# [QI21-guide], "One stream for text, reference images, and the target": Q and K are normalised
# per head (RMS over the 128 values of a head) before RoPE.  "Three-axis RoPE preserves image
# geometry": the 128 dims of a head are split (16, 56, 56) over frame, height and width, base
# 10,000; text positions advance one shared coordinate on all three axes; an image block keeps
# the frame coordinate reached by the preceding text while its height and width coordinates form
# a grid centred on zero; RoPE touches Q and K, not V.  Readings (the pages are silent on them):
#   * RMS norm: y = x / sqrt(mean(x^2) + eps) * w with a learned weight w[128] shared by all
#     heads; eps = 1e-6.
#   * rotation pairs are adjacent dims (2i, 2i + 1) (the complex-number form); inside an axis
#     section of width d_a, pair k turns by pos_axis * base^(-2k / d_a).
#   * the shared counter c starts at 0; a text token gets (c, c, c) and advances c by one; an
#     image block of H x W latents (row-major) gets (c, h - H//2, w - W//2) and then advances c by
#     one, so adjacent blocks never share a frame coordinate.
ROPE_SECTIONS = (16, 56, 56)
ROPE_BASE = 10000.0
RMS_EPS = 1e-6


def rope_positions(ids: Sequence[int], image_hw: Optional[Sequence[Tuple[int, int]]] = None
                   ) -> np.ndarray:
    """int64 [S, 3] (frame, height, width) coordinates of every position.  image_hw lists
    (H, W) of each image block in sequence order (default: square blocks)."""
    ids = validate_block_ids(ids)
    S = len(ids)
    pos = np.zeros((S, 3), dtype=np.int64)
    c = 0
    img = 0
    for a, e, bid in runs(ids, _validated=True):
        if bid < 0:
            for i in range(a, e):
                pos[i] = (c, c, c)
                c += 1
            continue
        n = e - a
        if image_hw is None:
            H = int(round(np.sqrt(n)))
            W = H
        else:
            H, W = image_hw[img]
        if H * W != n:
            raise ValueError(f"image block of {n} positions is not {H} x {W}")
        img += 1
        for t in range(n):
            h, w = divmod(t, W)
            pos[a + t] = (c, h - H // 2, w - W // 2)
        c += 1
    return pos


def rope_angles(pos: np.ndarray, base: float = ROPE_BASE,
                sections: Sequence[int] = ROPE_SECTIONS) -> np.ndarray:
    """float64 [S, 64] rotation angle of each adjacent pair of a head's 128 dims."""
    pos = np.asarray(pos, dtype=np.float64)
    cols = []
    for axis, d in enumerate(sections):
        k = np.arange(d // 2, dtype=np.float64)
        inv = base ** (-2.0 * k / d)
        cols.append(pos[:, axis:axis + 1] * inv[None, :])
    return np.concatenate(cols, axis=1)


def rms_norm(x: np.ndarray, w: np.ndarray, eps: float = RMS_EPS) -> np.ndarray:
    """Per-head RMS normalisation over the last axis, in float64."""
    x = np.asarray(x, dtype=np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * np.asarray(w, dtype=np.float64)


def apply_rope(x: np.ndarray, angles: np.ndarray) -> np.ndarray:
    """Rotate adjacent pairs of x [B, S, H, D] by angles [S, D/2], in float64."""
    x = np.asarray(x, dtype=np.float64)
    a = np.asarray(angles, dtype=np.float64)[None, :, None, :]
    x0, x1 = x[..., 0::2], x[..., 1::2]
    c, s = np.cos(a), np.sin(a)
    out = np.empty_like(x)
    out[..., 0::2] = x0 * c - x1 * s
    out[..., 1::2] = x0 * s + x1 * c
    return out


def qk_prologue(q: np.ndarray, k: np.ndarray, wq: np.ndarray, wk: np.ndarray, pos: np.ndarray,
                eps: float = RMS_EPS, base: float = ROPE_BASE) -> Tuple[np.ndarray, np.ndarray]:
    """(RoPE(RMSNorm(q) * wq), RoPE(RMSNorm(k) * wk)) in float64; pos is [S, 3]."""
    ang = rope_angles(pos, base)
    return apply_rope(rms_norm(q, wq, eps), ang), apply_rope(rms_norm(k, wk, eps), ang)


# ----------------------------------------------------------------------------------------------
# Batches of sequences with different lengths and layouts (varlen)
# ----------------------------------------------------------------------------------------------
# [QI21-guide], "Block-causal attention is the cache-enabling boundary" (padded keys are ignored)
# and [infra], "NEO-Unify 多模态 Prefill 的注意力" (batches of prompts up to 64k positions with few
# image tokens): every sequence of a batch is attended on its own, under its own block-id layout;
# rows of one sequence never see keys of another or padding.  Sequences sit along one row axis of
# [rows, H, D] tensors, sequence b at rows [row_start[b], row_start[b] + len_b).
def attention_varlen(q: np.ndarray, k: np.ndarray, v: np.ndarray, ids_list: Sequence[Sequence[int]],
                     row_start: Sequence[int], scale: Optional[float] = None,
                     rows_of: Optional[Dict[int, np.ndarray]] = None,
                     heads: Optional[Sequence[int]] = None) -> Dict[int, np.ndarray]:
    """{b: float64 [len_b or len(rows_of[b]), H', D]} for each sequence b; q, k, v are [R, H, D].
    rows_of[b] (optional) selects local query rows of sequence b, heads a subset of heads."""
    out = {}
    for b, ids in enumerate(ids_list):
        a = int(row_start[b])
        n = len(ids)
        sl = slice(a, a + n)
        rows = None if rows_of is None else rows_of.get(b)
        out[b] = attention(q[None, sl], k[None, sl], v[None, sl], ids, scale=scale, rows=rows,
                           heads=heads)[0]
    return out


def packed_row_starts(lengths: Sequence[int]) -> np.ndarray:
    """Row of each sequence when the batch is packed without gaps."""
    return np.concatenate([[0], np.cumsum(np.asarray(lengths, dtype=np.int64))[:-1]])


# ----------------------------------------------------------------------------------------------
# [QI21-guide], "The prefix cache is a compute-for-memory trade": one prefix cache per CFG branch
# (the cond and uncond prompts differ, so their prefixes differ in length).  For a batch of
# sequences, sequence b's prefix is everything before its last block (prefix_split), and the
# batch's caches are laid end to end along one row axis: sequence b's P_b rows start at
# c_b = P_0 + ... + P_{b-1}.  Its cached step takes its N_b target rows, which start at
# t_b = N_0 + ... + N_{b-1} along the row axis of the target tensors.
def varlen_offsets(ids_list: Sequence[Sequence[int]]) -> Dict[str, np.ndarray]:
    """Per sequence: P (prefix), N (target), c (first cache row), t (first target row)."""
    P = np.array([prefix_split(ids)[0] for ids in ids_list], dtype=np.int64)
    N = np.array([len(ids) for ids in ids_list], dtype=np.int64) - P
    return {"P": P, "N": N, "c": packed_row_starts(P), "t": packed_row_starts(N)}


def prefix_cache_varlen(k: np.ndarray, v: np.ndarray, ids_list: Sequence[Sequence[int]],
                        row_start: Sequence[int]) -> Tuple[np.ndarray, np.ndarray]:
    """Copies of every sequence's prefix K/V rows, laid end to end: [sum P_b, H, D] each."""
    off = varlen_offsets(ids_list)
    kc = [k[int(row_start[b]):int(row_start[b]) + int(off["P"][b])] for b in range(len(ids_list))]
    vc = [v[int(row_start[b]):int(row_start[b]) + int(off["P"][b])] for b in range(len(ids_list))]
    return np.concatenate(kc).copy(), np.concatenate(vc).copy()


def decode_varlen(q_t: np.ndarray, k_cache: np.ndarray, v_cache: np.ndarray, k_t: np.ndarray,
                  v_t: np.ndarray, ids_list: Sequence[Sequence[int]],
                  scale: Optional[float] = None, rows_of: Optional[Dict[int, np.ndarray]] = None,
                  heads: Optional[Sequence[int]] = None) -> Dict[int, np.ndarray]:
    """Cached step of every sequence of a batch: sequence b's target queries attend with no mask
    to [its cache rows ; its target keys] (decode, per sequence).  q_t, k_t, v_t are
    [sum N_b, H, D], the caches [sum P_b, H, D].  Returns {b: float64 [N_b or len(rows_of[b]),
    H', D]}."""
    off = varlen_offsets(ids_list)
    if k_cache.shape[0] != off["P"].sum() or q_t.shape[0] != off["N"].sum():
        raise OracleInputError("cache or target rows do not match the batch's P_b and N_b")
    out = {}
    for b in range(len(ids_list)):
        c, P = int(off["c"][b]), int(off["P"][b])
        t, N = int(off["t"][b]), int(off["N"][b])
        rows = None if rows_of is None else rows_of.get(b)
        out[b] = decode(q_t[None, t:t + N], k_cache[None, c:c + P], v_cache[None, c:c + P],
                        k_t[None, t:t + N], v_t[None, t:t + N], scale=scale, rows=rows,
                        heads=heads)[0]
    return out
