"""Seeded synthetic inputs for block-causal attention: sequence layouts and Q/K/V draws.

This module is shared by the tests, the benchmark and the smoke check. It holds no part of
the attention arithmetic: it only describes sequence layouts (which positions are text and
which belong to which image block) and draws random bf16 tensors, so that the CPU oracle and
the HIP path are fed the very same bits.

Layouts follow the sequence assembly of the Qwen-Image 2.1 pages ("One stream for text,
reference images, and the target": text positions, then reference-image latents, then the
target latents, all in one sequence).  A 1024x1024 image at VAE scale 16 gives 64x64 = 4,096
latent positions, a 2048x2048 image 128x128 = 16,384.  Text positions carry block id -1; each
image block gets its own non-negative id, numbered 0, 1, 2, ... in sequence order.

Input recipe: numpy ``default_rng(seed)`` (PCG64), ``standard_normal`` float32 draws of shape
[B, S, H, D] for Q, then K, then V, multiplied by 1/sqrt(128) for the "scaled" distribution
(the "sharp" distribution skips the factor), rounded to bf16 with round-to-nearest-even.
"""
from __future__ import annotations

import dataclasses
from typing import List, Sequence, Tuple

import numpy as np

HEAD_DIM = 128


@dataclasses.dataclass(frozen=True)
class Layout:
    """A sequence layout: an ordered list of ("text"|"image", length) segments."""

    name: str
    segments: Tuple[Tuple[str, int], ...]
    batch: int
    heads: int

    @property
    def seq_len(self) -> int:
        return sum(n for _, n in self.segments)

    def block_ids(self) -> np.ndarray:
        return block_ids_from_segments(self.segments)


def block_ids_from_segments(segments: Sequence[Tuple[str, int]]) -> np.ndarray:
    """-1 for every text position, a fresh id 0, 1, 2, ... for each image segment."""
    out: List[int] = []
    next_id = 0
    for kind, n in segments:
        if kind == "text":
            out.extend([-1] * n)
        elif kind == "image":
            out.extend([next_id] * n)
            next_id += 1
        else:
            raise ValueError(f"unknown segment kind {kind!r}")
    return np.asarray(out, dtype=np.int32)


def _two_ref_edit() -> Tuple[Tuple[str, int], ...]:
    return (("text", 48), ("image", 4096), ("text", 40), ("image", 4096), ("text", 24),
            ("image", 4096))


def _four_ref_long() -> Tuple[Tuple[str, int], ...]:
    segs: List[Tuple[str, int]] = [("text", 96), ("image", 4096)]
    for _ in range(3):
        segs += [("text", 16), ("image", 4096)]
    segs.append(("image", 16384))
    return tuple(segs)


# The five workloads.  Segment lists are taken as written; the sequence lengths follow from them.
TINY = Layout("tiny: [text 12][ref 64][text 6][target 64], H=2",
              (("text", 12), ("image", 64), ("text", 6), ("image", 64)), batch=1, heads=2)
T2I_1024 = Layout("text-to-image 1024^2: [text 256][target 4096]",
                  (("text", 256), ("image", 4096)), batch=1, heads=32)
EDIT_2REF = Layout("2-ref 1024^2 edit: [t48][ref 4096][t40][ref 4096][t24][target 4096]",
                   _two_ref_edit(), batch=1, heads=32)
EDIT_2REF_CFG = Layout("2-ref 1024^2 edit under CFG (B=2)", _two_ref_edit(), batch=2, heads=32)
LONG_4REF = Layout("4-ref 1024^2 + 2048^2 target: [t96][ref]([t16][ref])x3[target 16384]",
                   _four_ref_long(), batch=1, heads=32)

# A small target under the same two references (512^2 target: 32 x 32 = 1,024 latents): the
# cached step then has too few query tiles to fill the GPU, the case split-KV decode is for.
EDIT_2REF_T512 = Layout("2-ref 1024^2 edit, 512^2 target: [t48][ref 4096][t40][ref 4096][t24]"
                        "[target 1024]", _two_ref_edit()[:-1] + (("image", 1024),), batch=1,
                        heads=32)

# Classifier-free guidance with prompts of different lengths: the cond branch is the 2-ref edit
# above; the uncond branch keeps the references and the target but has a shorter first text
# segment (8 positions in place of 48, standing for a short negative prompt).  Each branch keeps
# its own prefix cache.
EDIT_2REF_UNCOND = Layout("2-ref 1024^2 edit, uncond branch: [t8][ref 4096][t40][ref 4096][t24]"
                          "[target 4096]", (("text", 8),) + _two_ref_edit()[1:], batch=1, heads=32)
CFG_VARLEN = (EDIT_2REF, EDIT_2REF_UNCOND)

WORKLOADS = {"tiny": TINY, "t2i_1024": T2I_1024, "edit_2ref": EDIT_2REF,
             "edit_2ref_cfg": EDIT_2REF_CFG, "long_4ref": LONG_4REF,
             "edit_2ref_t512": EDIT_2REF_T512}
SEEDS = {"tiny": 1001, "t2i_1024": 2001, "edit_2ref": 3001, "edit_2ref_cfg": 4000,
         "long_4ref": 5001, "edit_2ref_t512": 6001, "cfg_varlen": 7001}
DECODE_STEPS = 49  # 50 denoising steps: one prefill, then 49 cached steps


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 (round to nearest, ties to even); returns the uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(
        np.float32)


def draw_bf16(rng: np.random.Generator, shape, scaled: bool = True) -> np.ndarray:
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if scaled:
        x *= np.float32(1.0 / np.sqrt(HEAD_DIM))
    return f32_to_bf16_bits(x)


def qkv(seed: int, batch: int, seq: int, heads: int, scaled: bool = True):
    """Q, K, V as uint16 bf16 bit arrays [B, S, H, 128], drawn in that order from one stream."""
    rng = np.random.default_rng(seed)
    shape = (batch, seq, heads, HEAD_DIM)
    q = draw_bf16(rng, shape, scaled)
    k = draw_bf16(rng, shape, scaled)
    v = draw_bf16(rng, shape, scaled)
    return q, k, v


def decode_step_qkv(step: int, batch: int, target_len: int, heads: int, base_seed: int = 4000,
                    scaled: bool = True):
    """Fresh target Q/K/V for cached step ``step`` (1-based) of a generation."""
    return qkv(base_seed + step, batch, target_len, heads, scaled)


def random_layout(rng: np.random.Generator, seq: int, p_text: float = 0.5,
                  max_seg: int = 40) -> np.ndarray:
    """A random run layout of length ``seq`` (text runs and image blocks with distinct ids)."""
    segs: List[Tuple[str, int]] = []
    left = seq
    while left > 0:
        n = int(min(left, rng.integers(1, max_seg + 1)))
        segs.append(("text" if rng.random() < p_text else "image", n))
        left -= n
    return block_ids_from_segments(segs)


def prologue_inputs(seed: int, batch: int, seq: int, heads: int, head_dim: int = 128):
    """Raw (pre-norm) Q and K as bf16 bits [B, S, H, D] with a spread of per-row scales, and
    RMS-norm weights w_q, w_k float32 [D] near 1 (synthetic stand-ins for learned weights)."""
    rng = np.random.default_rng(seed)
    shape = (batch, seq, heads, head_dim)
    row_scale = np.exp(rng.uniform(-2.0, 2.0, size=shape[:3] + (1,))).astype(np.float32)
    q = rng.standard_normal(shape, dtype=np.float32) * row_scale
    k = rng.standard_normal(shape, dtype=np.float32) * row_scale[:, :, ::-1]
    wq = (1.0 + 0.1 * rng.standard_normal(head_dim)).astype(np.float32)
    wk = (1.0 + 0.1 * rng.standard_normal(head_dim)).astype(np.float32)
    return f32_to_bf16_bits(q), f32_to_bf16_bits(k), wq, wk


def neo_like_batch(seed: int, batch: int, max_seq_len: int, image_tokens: int):
    """A batch shaped like a row of the NEO-Unify mixed-mask prefill table (batch, max_seq_len,
    image_token_num): mostly text; the first sequence has max_seq_len positions and the others a
    length drawn from [max_seq_len / 2, max_seq_len]; image_tokens image positions in total, in
    spans of 16..64 tokens placed at random inside the text.  Returns (ids_list, lengths)."""
    rng = np.random.default_rng(seed)
    lengths = [max_seq_len] + [int(rng.integers(max_seq_len // 2, max_seq_len + 1))
                               for _ in range(batch - 1)]
    spans: List[List[int]] = [[] for _ in range(batch)]
    left = image_tokens
    while left > 0:
        n = int(min(left, rng.integers(16, 65)))
        spans[int(rng.integers(0, batch))].append(n)
        left -= n
    ids_list = []
    for b, L in enumerate(lengths):
        segs: List[Tuple[str, int]] = []
        imgs = spans[b]
        text = L - sum(imgs)
        cuts = np.sort(rng.integers(0, text + 1, size=len(imgs)))
        prev = 0
        for c, n in zip(cuts, imgs):
            if c > prev:
                segs.append(("text", int(c - prev)))
            segs.append(("image", n))
            prev = int(c)
        if text > prev:
            segs.append(("text", text - prev))
        ids_list.append(block_ids_from_segments(segs))
    return ids_list, lengths
