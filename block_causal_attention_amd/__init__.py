"""Block-causal attention for AMD MI355X: thin Python binding over libbca.so.

The binding only marshals arguments: every step of the computation runs in the library's HIP
kernels.  PyTorch supplies device memory and the current stream.

    plan = Plan(block_ids)                        # -1 text, k >= 0 image block k
    o = prefill(plan, q, k, v, k_cache=kc, v_cache=vc)  # bf16 [B,S,H,128] -> fp32, fills cache
    o_t = decode(plan, q_t, kc, vc, k_t, v_t)     # bf16 target [B,N,H,128] -> fp32

    cache = KVCache.empty(plan, B, H, KVCache.FP8_V)    # FP8 prefix cache (bca_kv_cache)
    o = prefill_ex(plan, q, k, v, cache)
    o_t = decode_ex(plan, q_t, cache, k_t, v_t)

    table = torch.from_numpy(rope_table(rope_positions(block_ids))).cuda()   # once per layout
    qk_prologue(q, k, wq, wk, table, q_out=q, k_out=k)   # per-head RMS norm + 3-axis RoPE
"""
from __future__ import annotations

import ctypes
from typing import Dict, Optional

import numpy as np

from . import _lib
from ._lib import BcaKvCache, BcaPlanInfo, BcaTensor

__all__ = ["Plan", "prefill", "decode", "prefill_ex", "decode_ex", "KVCache", "BcaError",
           "plan_info", "rope_positions", "rope_table", "qk_prologue", "prefill_varlen",
           "decode_split", "split_workspace", "dequantize_cache", "decode_split_noalloc",
           "decode_varlen", "decode_layout", "prefill_layout"]


class BcaError(RuntimeError):
    """A non-OK status from libbca, with the library's error text."""

    def __init__(self, status: int, msg: str):
        self.status = status
        lib = _lib.load()
        name = lib.bca_status_str(status).decode()
        super().__init__(f"{name}: {msg}")


def _check(status: int) -> None:
    if status != _lib.BCA_OK:
        raise BcaError(status, _lib.load().bca_last_error().decode())


def _ids32(block_ids) -> np.ndarray:
    """A block-id vector as contiguous int32, rejecting values outside the int32 range."""
    if hasattr(block_ids, "detach"):
        block_ids = block_ids.detach().cpu().numpy()
    a = np.asarray(block_ids)
    if a.dtype.kind == "i" and a.dtype.itemsize <= 4 or a.dtype.kind == "u" and a.dtype.itemsize < 4:
        return np.ascontiguousarray(a, dtype=np.int32)
    a = np.asarray(a, dtype=np.int64)
    if a.size and (a.min() < -(2**31) or a.max() >= 2**31):
        raise BcaError(_lib.BCA_ERR_BLOCK_IDS, "block id out of int32 range")
    return np.ascontiguousarray(a, dtype=np.int32)


class Plan:
    """Launch plan built from a per-position block-id vector (see include/bca.h, bca_plan)."""

    def __init__(self, block_ids, host_only: bool = False):
        lib = _lib.load()
        ids32 = _ids32(block_ids)
        if ids32.ndim != 1:
            raise ValueError("block ids must be 1-D")
        self._h = ctypes.c_void_p()
        flags = _lib.BCA_PLAN_HOST_ONLY if host_only else 0
        ptr = ids32.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)) if ids32.size else None
        _check(lib.bca_plan(ptr, ids32.size, flags, ctypes.byref(self._h)))
        self.info = plan_info(self)

    @classmethod
    def varlen(cls, ids_list, row_start=None, host_only: bool = False) -> "Plan":
        """Plan for a batch of sequences with their own layouts (bca_plan_varlen): sequence b
        at rows [row_start[b], row_start[b] + len_b) (default: packed)."""
        lib = _lib.load()
        seqs = [_ids32(i) for i in ids_list]
        if not seqs or any(x.ndim != 1 for x in seqs):
            raise ValueError("ids_list must be a non-empty list of 1-D id vectors")
        flat = np.ascontiguousarray(np.concatenate(seqs))
        lens = np.ascontiguousarray(np.array([x.size for x in seqs], dtype=np.int64))
        starts = None
        if row_start is not None:
            starts = np.ascontiguousarray(np.asarray(row_start, dtype=np.int64))
            if starts.shape != lens.shape:
                raise ValueError("row_start needs one entry per sequence")
        self = cls.__new__(cls)
        self._h = ctypes.c_void_p()
        flags = _lib.BCA_PLAN_HOST_ONLY if host_only else 0
        i64 = lambda a: None if a is None else a.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))
        ptr = flat.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)) if flat.size else None
        _check(lib.bca_plan_varlen(ptr, i64(lens), i64(starts), lens.size, flags,
                                   ctypes.byref(self._h)))
        self.info = plan_info(self)
        return self

    @property
    def handle(self) -> ctypes.c_void_p:
        if not self._h:
            raise ValueError("plan already freed")
        return self._h

    def export(self) -> Dict[str, np.ndarray]:
        i = self.info
        seg = np.empty(3 * i.n_segments, np.int32)
        rl = np.empty(i.seq_len, np.int32)
        kf = np.empty(i.n_qtiles, np.int32)
        ke = np.empty(i.n_qtiles, np.int32)
        od = np.empty(i.n_qtiles, np.int32)
        p = lambda a: a.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
        _check(_lib.load().bca_plan_export(self.handle, p(seg), p(rl), p(kf), p(ke), p(od)))
        return {"segments": seg.reshape(-1, 3), "row_limit": rl, "kv_full": kf, "kv_end": ke,
                "order": od}

    def sequences(self) -> np.ndarray:
        """int64 [n_sequences, 6] (bca_plan_sequences): per sequence its first tensor row,
        length, prefix P_b, target N_b, first cache row c_b and first target row t_b."""
        out = np.empty((self.info.n_sequences, 6), np.int64)
        _check(_lib.load().bca_plan_sequences(
            self.handle, out.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))))
        return out

    def free(self) -> None:
        if self._h:
            _lib.load().bca_plan_free(self._h)
            self._h = ctypes.c_void_p()

    def __del__(self):
        try:
            self.free()
        except Exception:
            pass


def plan_info(plan: Plan) -> BcaPlanInfo:
    info = BcaPlanInfo()
    _check(_lib.load().bca_plan_get_info(plan.handle, ctypes.byref(info)))
    return info


def _desc(t, name: str, dtype) -> BcaTensor:
    """bca_tensor of a 4-D [B, S, H, D] torch tensor with D contiguous."""
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.dim() != 4:
        raise ValueError(f"{name} must be 4-D [B, S, H, D]")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    sb, ss, sh, sd = t.stride()
    if sd != 1 and t.shape[3] > 1:
        raise ValueError(f"{name}: the last dimension must be contiguous")
    return BcaTensor(t.data_ptr(), sb, ss, sh)


def _scale_desc(t, name: str) -> BcaTensor:
    """bca_tensor of a 3-D fp32 [B, P, H] scale tensor."""
    import torch

    if t.dtype != torch.float32 or t.dim() != 3 or not t.is_cuda:
        raise ValueError(f"{name} must be a float32 device tensor [B, P, H]")
    sb, ss, sh = t.stride()
    return BcaTensor(t.data_ptr(), sb, ss, sh)


class KVCache:
    """A prefix K/V cache in one of the storage formats of bca.h (bca_kv_cache).

    BF16: k, v bf16 [B, P, H, D].  FP8_V: k bf16, v uint8 E4M3 codes [B, P, H, D] and v_scale
    fp32 [B, P, H].  FP8_KV: k and v codes with k_scale and v_scale."""

    BF16 = _lib.BCA_CACHE_BF16
    FP8_V = _lib.BCA_CACHE_FP8_V
    FP8_KV = _lib.BCA_CACHE_FP8_KV

    def __init__(self, fmt: int, k, v, k_scale=None, v_scale=None):
        if fmt not in (self.BF16, self.FP8_V, self.FP8_KV):
            raise ValueError(f"unknown cache format {fmt}")
        self.format, self.k, self.v, self.k_scale, self.v_scale = fmt, k, v, k_scale, v_scale

    @property
    def k_quantized(self) -> bool:
        return self.format == self.FP8_KV

    @property
    def v_quantized(self) -> bool:
        return self.format != self.BF16

    @classmethod
    def empty(cls, plan: "Plan", batch: int, heads: int, fmt: int = 0, head_dim: int = 128,
              device="cuda") -> "KVCache":
        import torch

        P = plan.info.prefix_len
        shape = (batch, P, heads, head_dim)
        kq, vq = fmt == cls.FP8_KV, fmt != cls.BF16
        k = torch.empty(shape, dtype=torch.uint8 if kq else torch.bfloat16, device=device)
        v = torch.empty(shape, dtype=torch.uint8 if vq else torch.bfloat16, device=device)
        ks = torch.empty((batch, P, heads), dtype=torch.float32, device=device) if kq else None
        vs = torch.empty((batch, P, heads), dtype=torch.float32, device=device) if vq else None
        return cls(fmt, k, v, ks, vs)

    def nbytes(self) -> int:
        return sum(t.numel() * t.element_size()
                   for t in (self.k, self.v, self.k_scale, self.v_scale) if t is not None)

    def _struct(self, B: int, P: int, H: int, D: int) -> BcaKvCache:
        import torch

        c = BcaKvCache()
        c.format = self.format
        for name, t, q in (("k", self.k, self.k_quantized), ("v", self.v, self.v_quantized)):
            if t is None or tuple(t.shape) != (B, P, H, D):
                raise ValueError(f"cache.{name} must be [B, P={P}, H, D]")
            setattr(c, name, _desc(t, f"cache.{name}", torch.uint8 if q else torch.bfloat16))
        for name, t, q in (("k_scale", self.k_scale, self.k_quantized),
                           ("v_scale", self.v_scale, self.v_quantized)):
            if q:
                if t is None or tuple(t.shape) != (B, P, H):
                    raise ValueError(f"cache.{name} must be [B, P={P}, H]")
                setattr(c, name, _scale_desc(t, f"cache.{name}"))
        return c


def _scale(scale: Optional[float]) -> float:
    return 0.0 if scale is None else float(scale)


def prefill(plan: Plan, q, k, v, *, scale: Optional[float] = None, out=None, k_cache=None,
            v_cache=None):
    """Block-causal prefill (bca_prefill).  Returns the fp32 output [B, S, H, D]."""
    import torch

    B, S, H, D = q.shape
    if tuple(k.shape) != (B, S, H, D) or tuple(v.shape) != (B, S, H, D):
        raise ValueError("q, k, v must share the shape [B, S, H, D]")
    if S != plan.info.seq_len:
        raise ValueError(f"sequence length {S} != plan's {plan.info.seq_len}")
    if out is None:
        out = torch.empty((B, S, H, D), dtype=torch.float32, device=q.device)
    if tuple(out.shape) != (B, S, H, D):
        raise ValueError("out has the wrong shape")
    P = plan.info.prefix_len
    kc = vc = None
    if (k_cache is None) != (v_cache is None):
        raise ValueError("k_cache and v_cache go together")
    if k_cache is not None:
        for c in (k_cache, v_cache):
            if tuple(c.shape) != (B, P, H, D):
                raise ValueError(f"cache must be [B, P={P}, H, D]")
        kc = ctypes.byref(_desc(k_cache, "k_cache", torch.bfloat16))
        vc = ctypes.byref(_desc(v_cache, "v_cache", torch.bfloat16))
    stream = torch.cuda.current_stream(q.device).cuda_stream
    with torch.cuda.device(q.device):
        _check(_lib.load().bca_prefill(
            plan.handle, B, H, D, _scale(scale),
            ctypes.byref(_desc(q, "q", torch.bfloat16)), ctypes.byref(_desc(k, "k", torch.bfloat16)),
            ctypes.byref(_desc(v, "v", torch.bfloat16)), ctypes.byref(_desc(out, "out", torch.float32)),
            kc, vc, ctypes.c_void_p(stream)))
    return out


def decode(plan: Plan, q, k_cache, v_cache, k, v, *, scale: Optional[float] = None, out=None):
    """Prefix-cached decode (bca_decode).  q/k/v are the target's [B, N, H, D]; returns fp32."""
    import torch

    B, N, H, D = q.shape
    P = plan.info.prefix_len
    if N != plan.info.target_len:
        raise ValueError(f"target length {N} != plan's {plan.info.target_len}")
    checks = [("k", k, N), ("v", v, N)]
    if P > 0 or k_cache is not None or v_cache is not None:
        checks += [("k_cache", k_cache, P), ("v_cache", v_cache, P)]
    for name, t, n in checks:
        if t is None or tuple(t.shape) != (B, n, H, D):
            raise ValueError(f"{name} must be [B, {n}, H, D]")
    if out is None:
        out = torch.empty((B, N, H, D), dtype=torch.float32, device=q.device)
    if tuple(out.shape) != (B, N, H, D):
        raise ValueError("out has the wrong shape")
    kc = ctypes.byref(_desc(k_cache, "k_cache", torch.bfloat16)) if P > 0 else None
    vc = ctypes.byref(_desc(v_cache, "v_cache", torch.bfloat16)) if P > 0 else None
    stream = torch.cuda.current_stream(q.device).cuda_stream
    with torch.cuda.device(q.device):
        _check(_lib.load().bca_decode(
            plan.handle, B, H, D, _scale(scale), ctypes.byref(_desc(q, "q", torch.bfloat16)),
            kc, vc, ctypes.byref(_desc(k, "k", torch.bfloat16)),
            ctypes.byref(_desc(v, "v", torch.bfloat16)),
            ctypes.byref(_desc(out, "out", torch.float32)), ctypes.c_void_p(stream)))
    return out


def prefill_ex(plan: Plan, q, k, v, cache: Optional[KVCache] = None, *,
               scale: Optional[float] = None, out=None):
    """Block-causal prefill storing the prefix cache in any format (bca_prefill_ex)."""
    import torch

    B, S, H, D = q.shape
    if tuple(k.shape) != (B, S, H, D) or tuple(v.shape) != (B, S, H, D):
        raise ValueError("q, k, v must share the shape [B, S, H, D]")
    if S != plan.info.seq_len:
        raise ValueError(f"sequence length {S} != plan's {plan.info.seq_len}")
    if out is None:
        out = torch.empty((B, S, H, D), dtype=torch.float32, device=q.device)
    if tuple(out.shape) != (B, S, H, D):
        raise ValueError("out has the wrong shape")
    P = plan.info.prefix_len
    c = None
    if cache is not None and P > 0:
        c = ctypes.byref(cache._struct(B, P, H, D))
    stream = torch.cuda.current_stream(q.device).cuda_stream
    with torch.cuda.device(q.device):
        _check(_lib.load().bca_prefill_ex(
            plan.handle, B, H, D, _scale(scale),
            ctypes.byref(_desc(q, "q", torch.bfloat16)), ctypes.byref(_desc(k, "k", torch.bfloat16)),
            ctypes.byref(_desc(v, "v", torch.bfloat16)),
            ctypes.byref(_desc(out, "out", torch.float32)), c, ctypes.c_void_p(stream)))
    return out


def decode_ex(plan: Plan, q, cache: Optional[KVCache], k, v, *, scale: Optional[float] = None,
              out=None):
    """Prefix-cached decode over a cache of any format (bca_decode_ex); returns fp32."""
    import torch

    B, N, H, D = q.shape
    P = plan.info.prefix_len
    if N != plan.info.target_len:
        raise ValueError(f"target length {N} != plan's {plan.info.target_len}")
    for name, t in (("k", k), ("v", v)):
        if tuple(t.shape) != (B, N, H, D):
            raise ValueError(f"{name} must be [B, {N}, H, D]")
    if P > 0 and cache is None:
        raise ValueError("the prefix is not empty: a cache is required")
    if out is None:
        out = torch.empty((B, N, H, D), dtype=torch.float32, device=q.device)
    if tuple(out.shape) != (B, N, H, D):
        raise ValueError("out has the wrong shape")
    c = ctypes.byref(cache._struct(B, P, H, D)) if P > 0 else None
    stream = torch.cuda.current_stream(q.device).cuda_stream
    with torch.cuda.device(q.device):
        _check(_lib.load().bca_decode_ex(
            plan.handle, B, H, D, _scale(scale), ctypes.byref(_desc(q, "q", torch.bfloat16)), c,
            ctypes.byref(_desc(k, "k", torch.bfloat16)),
            ctypes.byref(_desc(v, "v", torch.bfloat16)),
            ctypes.byref(_desc(out, "out", torch.float32)), ctypes.c_void_p(stream)))
    return out


def rope_positions(block_ids, image_hw=None) -> np.ndarray:
    """(frame, height, width) of every position (bca_rope_positions): int32 [S, 3].  image_hw:
    None (square image blocks) or a list of (H, W) per image block in sequence order."""
    lib = _lib.load()
    if hasattr(block_ids, "detach"):
        block_ids = block_ids.detach().cpu().numpy()
    ids = np.ascontiguousarray(np.asarray(block_ids, dtype=np.int64))
    if ids.ndim != 1 or ids.size == 0:
        raise ValueError("block ids must be a non-empty 1-D sequence")
    ids32 = ids.astype(np.int32)
    out = np.empty((ids32.size, 3), np.int32)
    p = lambda a: a.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
    hw = None
    n_img = 0
    if image_hw is not None:
        hw = np.ascontiguousarray(np.asarray(image_hw, dtype=np.int32).reshape(-1, 2))
        n_img = hw.shape[0]
    _check(lib.bca_rope_positions(p(ids32), ids32.size, None if hw is None else p(hw), n_img,
                                  p(out)))
    return out


def rope_table(pos, base: float = 10000.0) -> np.ndarray:
    """{cos, sin} of every rotation pair at every position (bca_rope_table): float32
    [S, 64, 2]."""
    pos = np.ascontiguousarray(np.asarray(pos, dtype=np.int32).reshape(-1, 3))
    out = np.empty((pos.shape[0], 64, 2), np.float32)
    _check(_lib.load().bca_rope_table(pos.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                                      pos.shape[0], float(base),
                                      out.ctypes.data_as(ctypes.POINTER(ctypes.c_float))))
    return out


def qk_prologue(q, k, q_weight, k_weight, table, *, eps: float = 1e-6, q_out=None, k_out=None):
    """Per-head RMS norm then three-axis RoPE of q and k (bca_qk_prologue).  q, k: bf16
    [B, S, H, 128]; weights: fp32 [128]; table: fp32 [S, 64, 2] on the device.  Returns
    (q_out, k_out); pass q_out=q, k_out=k to work in place."""
    import torch

    B, S, H, D = q.shape
    if tuple(k.shape) != (B, S, H, D):
        raise ValueError("q and k must share the shape [B, S, H, D]")
    for name, t, shape in (("q_weight", q_weight, (D,)), ("k_weight", k_weight, (D,)),
                           ("table", table, (S, 64, 2))):
        if (t.dtype != torch.float32 or tuple(t.shape) != shape or not t.is_cuda
                or not t.is_contiguous()):
            raise ValueError(f"{name} must be a contiguous float32 device tensor {shape}")
    q_out = torch.empty_like(q) if q_out is None else q_out
    k_out = torch.empty_like(k) if k_out is None else k_out
    for name, t in (("q_out", q_out), ("k_out", k_out)):
        if tuple(t.shape) != (B, S, H, D):
            raise ValueError(f"{name} has the wrong shape")
    stream = torch.cuda.current_stream(q.device).cuda_stream
    vp = lambda t: ctypes.c_void_p(t.data_ptr())
    with torch.cuda.device(q.device):
        _check(_lib.load().bca_qk_prologue(
            B, S, H, D, float(eps), ctypes.byref(_desc(q, "q", torch.bfloat16)),
            ctypes.byref(_desc(k, "k", torch.bfloat16)),
            ctypes.byref(_desc(q_out, "q_out", torch.bfloat16)),
            ctypes.byref(_desc(k_out, "k_out", torch.bfloat16)), vp(q_weight), vp(k_weight),
            vp(table), ctypes.c_void_p(stream)))
    return q_out, k_out


def _desc3(t, name: str, dtype) -> BcaTensor:
    """bca_tensor of a 3-D [rows, H, D] torch tensor with D contiguous (stride_b unused)."""
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.dim() != 3 or not t.is_cuda:
        raise ValueError(f"{name} must be a 3-D [rows, H, D] device tensor")
    ss, sh, sd = t.stride()
    if sd != 1 and t.shape[2] > 1:
        raise ValueError(f"{name}: the last dimension must be contiguous")
    return BcaTensor(t.data_ptr(), 0, ss, sh)


def prefill_varlen(plan: Plan, q, k, v, *, k_cache=None, v_cache=None,
                   scale: Optional[float] = None, out=None):
    """Block-causal prefill of every sequence of a varlen plan (bca_prefill_varlen).  q, k, v:
    bf16 [rows, H, D]; returns fp32 [rows, H, D] (rows outside the sequences left untouched:
    zero when `out` is not given).  k_cache, v_cache (optional, both or neither): bf16
    [plan.info.prefix_len, H, D], receiving every sequence's prefix rows, packed."""
    import torch

    R, H, D = q.shape
    if tuple(k.shape) != (R, H, D) or tuple(v.shape) != (R, H, D):
        raise ValueError("q, k, v must share the shape [rows, H, D]")
    if R < plan.info.rows:
        raise ValueError(f"the plan spans {plan.info.rows} rows, the tensors {R}")
    if (k_cache is None) != (v_cache is None):
        raise ValueError("give both k_cache and v_cache, or neither")
    P = plan.info.prefix_len
    if k_cache is not None:
        for name, t in (("k_cache", k_cache), ("v_cache", v_cache)):
            if tuple(t.shape) != (P, H, D):
                raise ValueError(f"{name} must be [{P}, H, D]")
    if out is None:
        out = torch.zeros((R, H, D), dtype=torch.float32, device=q.device)
    if tuple(out.shape) != (R, H, D):
        raise ValueError("out has the wrong shape")
    store = k_cache is not None and P > 0
    kc = ctypes.byref(_desc3(k_cache, "k_cache", torch.bfloat16)) if store else None
    vc = ctypes.byref(_desc3(v_cache, "v_cache", torch.bfloat16)) if store else None
    stream = torch.cuda.current_stream(q.device).cuda_stream
    with torch.cuda.device(q.device):
        _check(_lib.load().bca_prefill_varlen(
            plan.handle, H, D, _scale(scale), ctypes.byref(_desc3(q, "q", torch.bfloat16)),
            ctypes.byref(_desc3(k, "k", torch.bfloat16)),
            ctypes.byref(_desc3(v, "v", torch.bfloat16)),
            ctypes.byref(_desc3(out, "out", torch.float32)), kc, vc, ctypes.c_void_p(stream)))
    return out


def decode_varlen(plan: Plan, q, k_cache, v_cache, k, v, *, scale: Optional[float] = None,
                  out=None):
    """Cached step of every sequence of a varlen plan in one launch (bca_decode_varlen).  q, k, v:
    bf16 [plan.info.target_len, H, D] (the sequences' targets, packed); k_cache, v_cache: bf16
    [plan.info.prefix_len, H, D] as prefill_varlen stores them.  Returns fp32 like q."""
    import torch

    N, H, D = q.shape
    P = plan.info.prefix_len
    if N != plan.info.target_len:
        raise ValueError(f"{N} target rows != the plan's {plan.info.target_len}")
    checks = [("k", k, N), ("v", v, N)]
    if P > 0 or k_cache is not None or v_cache is not None:
        checks += [("k_cache", k_cache, P), ("v_cache", v_cache, P)]
    for name, t, n in checks:
        if t is None or tuple(t.shape) != (n, H, D):
            raise ValueError(f"{name} must be [{n}, H, D]")
    if out is None:
        out = torch.empty((N, H, D), dtype=torch.float32, device=q.device)
    if tuple(out.shape) != (N, H, D):
        raise ValueError("out has the wrong shape")
    kc = ctypes.byref(_desc3(k_cache, "k_cache", torch.bfloat16)) if P > 0 else None
    vc = ctypes.byref(_desc3(v_cache, "v_cache", torch.bfloat16)) if P > 0 else None
    stream = torch.cuda.current_stream(q.device).cuda_stream
    with torch.cuda.device(q.device):
        _check(_lib.load().bca_decode_varlen(
            plan.handle, H, D, _scale(scale), ctypes.byref(_desc3(q, "q", torch.bfloat16)),
            kc, vc, ctypes.byref(_desc3(k, "k", torch.bfloat16)),
            ctypes.byref(_desc3(v, "v", torch.bfloat16)),
            ctypes.byref(_desc3(out, "out", torch.float32)), ctypes.c_void_p(stream)))
    return out


def decode_layout(n_q: int, batch_heads: int, n_split: int = 1, cache_fmt: int = 0,
                  cus: int = 0):
    """(waves, tiles of 384, 256 and 128 rows, tail tiles of 256 rows in a second 8-wave launch)
    per (batch, head, key range) of a cached step with n_q query rows per (batch, head),
    batch_heads = B * H, n_split key ranges and a cache of format cache_fmt (KVCache.BF16 / FP8_V /
    FP8_KV), on `cus` compute units (0: the current device's) (bca_decode_layout)."""
    out = (ctypes.c_int32 * 5)()
    _check(_lib.load().bca_decode_layout(n_q, batch_heads, n_split, cache_fmt, cus, out))
    return tuple(out)


def prefill_layout(plan: Plan, batch: int, heads: int, cus: int = 0):
    """(attention launches, query tiles per (batch, head) of the prefill launch, target rows
    handed to the second launch) of a single-sequence prefill on `cus` compute units (0: the
    current device's) (bca_prefill_layout)."""
    out = (ctypes.c_int32 * 3)()
    _check(_lib.load().bca_prefill_layout(plan.handle, batch, heads, cus, out))
    return tuple(out)


def split_workspace(plan: Plan, batch: int, heads: int, n_split: int = 0):
    """(bytes, n_split_used) of a split decode (bca_decode_split_workspace)."""
    nbytes = ctypes.c_int64()
    used = ctypes.c_int32()
    _check(_lib.load().bca_decode_split_workspace(plan.handle, batch, heads, n_split,
                                                  ctypes.byref(nbytes), ctypes.byref(used)))
    return nbytes.value, used.value


def decode_split(plan: Plan, q, cache: Optional[KVCache], k, v, *, n_split: int = 0,
                 workspace=None, scale: Optional[float] = None, out=None):
    """Split-KV cached decode (bca_decode_split).  The workspace (a uint8 device tensor) is
    allocated here when not given."""
    import torch

    B, N, H, D = q.shape
    P = plan.info.prefix_len
    if N != plan.info.target_len:
        raise ValueError(f"target length {N} != plan's {plan.info.target_len}")
    for name, t in (("k", k), ("v", v)):
        if tuple(t.shape) != (B, N, H, D):
            raise ValueError(f"{name} must be [B, {N}, H, D]")
    if P > 0 and cache is None:
        raise ValueError("the prefix is not empty: a cache is required")
    nbytes, _ = split_workspace(plan, B, H, n_split)
    if workspace is None and nbytes:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=q.device)
    if workspace is not None and workspace.numel() * workspace.element_size() < nbytes:
        raise ValueError(f"workspace needs {nbytes} bytes")
    if out is None:
        out = torch.empty((B, N, H, D), dtype=torch.float32, device=q.device)
    c = ctypes.byref(cache._struct(B, P, H, D)) if P > 0 else None
    ws = ctypes.c_void_p(workspace.data_ptr()) if workspace is not None else None
    wsb = workspace.numel() * workspace.element_size() if workspace is not None else 0
    stream = torch.cuda.current_stream(q.device).cuda_stream
    with torch.cuda.device(q.device):
        _check(_lib.load().bca_decode_split(
            plan.handle, B, H, D, _scale(scale), ctypes.byref(_desc(q, "q", torch.bfloat16)), c,
            ctypes.byref(_desc(k, "k", torch.bfloat16)),
            ctypes.byref(_desc(v, "v", torch.bfloat16)),
            ctypes.byref(_desc(out, "out", torch.float32)), n_split, ws, wsb,
            ctypes.c_void_p(stream)))
    return out


def decode_split_noalloc(plan: Plan, q, cache: Optional[KVCache], k, v, *, n_split: int = 0,
                         scale: Optional[float] = None, out=None):
    """Split-KV cached decode whose partial results live in the library's own device scratch
    (bca_decode_split_noalloc): the library allocates nothing.  `out` is allocated here (by
    torch) only when not given."""
    import torch

    B, N, H, D = q.shape
    P = plan.info.prefix_len
    if N != plan.info.target_len:
        raise ValueError(f"target length {N} != plan's {plan.info.target_len}")
    for name, t in (("k", k), ("v", v)):
        if tuple(t.shape) != (B, N, H, D):
            raise ValueError(f"{name} must be [B, {N}, H, D]")
    if P > 0 and cache is None:
        raise ValueError("the prefix is not empty: a cache is required")
    if out is None:
        out = torch.empty((B, N, H, D), dtype=torch.float32, device=q.device)
    c = ctypes.byref(cache._struct(B, P, H, D)) if P > 0 else None
    stream = torch.cuda.current_stream(q.device).cuda_stream
    with torch.cuda.device(q.device):
        _check(_lib.load().bca_decode_split_noalloc(
            plan.handle, B, H, D, _scale(scale), ctypes.byref(_desc(q, "q", torch.bfloat16)), c,
            ctypes.byref(_desc(k, "k", torch.bfloat16)),
            ctypes.byref(_desc(v, "v", torch.bfloat16)),
            ctypes.byref(_desc(out, "out", torch.float32)), n_split, ctypes.c_void_p(stream)))
    return out


def dequantize_cache(cache: KVCache, out: Optional[KVCache] = None) -> KVCache:
    """The cache written back as bf16 (bca_cache_dequantize): values E4M3(code) * scale in fp32,
    rounded to bf16, bitwise what the FP8 decode uses.  `out` (a bf16 KVCache of the same
    shape) is reused when given."""
    import torch

    B, P, H, D = cache.k.shape
    if out is None:
        out = KVCache(KVCache.BF16,
                      torch.empty((B, P, H, D), dtype=torch.bfloat16, device=cache.k.device),
                      torch.empty((B, P, H, D), dtype=torch.bfloat16, device=cache.k.device))
    if out.format != KVCache.BF16:
        raise ValueError("out must be a bf16 cache")
    for name, t in (("out.k", out.k), ("out.v", out.v)):
        if tuple(t.shape) != (B, P, H, D) or t.device != cache.k.device:
            raise ValueError(f"{name} must be [B, P={P}, H, D] on the cache's device")
    if P == 0:
        return out
    c = cache._struct(B, P, H, D)
    stream = torch.cuda.current_stream(cache.k.device).cuda_stream
    with torch.cuda.device(cache.k.device):
        _check(_lib.load().bca_cache_dequantize(
            B, P, H, D, ctypes.byref(c), ctypes.byref(_desc(out.k, "out.k", torch.bfloat16)),
            ctypes.byref(_desc(out.v, "out.v", torch.bfloat16)), ctypes.c_void_p(stream)))
    return out
