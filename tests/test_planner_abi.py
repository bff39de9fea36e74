"""CPU tests of the C-ABI library: symbols, planner parity with the oracle, argument validation.

No compute call runs here: plans are host-only and every launch is expected to be rejected by a
host-side check before anything touches a GPU.
"""
import ctypes
import os
import re
import shutil
import subprocess

import numpy as np
import pytest

import bca_workloads as W
from oracle import bca_oracle as O

bca = pytest.importorskip("block_causal_attention_amd")
from block_causal_attention_amd import _lib  # noqa: E402

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    with open(os.path.join(ROOT, "include", "bca.h")) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(bca_\w+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = _lib.load()
    names = declared_functions()
    assert set(names) == set(_lib.EXPORTED)
    for n in names:
        assert hasattr(lib, n), n


def test_library_exports_only_the_c_abi():
    """Internal C++ functions and kernel stubs stay local to libbca.so."""
    nm = shutil.which("nm")
    if nm is None:
        pytest.skip("nm not available")
    out = subprocess.run([nm, "-D", "--defined-only", _lib.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    names = [line.split()[-1] for line in out.splitlines() if line.strip()]
    assert sorted(names) == sorted(declared_functions())


def plan_host(ids):
    return bca.Plan(np.asarray(ids), host_only=True)


def assert_plan_matches_oracle(ids):
    p = plan_host(ids)
    info = p.info
    got = p.export()
    want = O.plan_from_mask(ids, info.block_m)
    for key in ("segments", "row_limit", "kv_full", "kv_end", "order"):
        assert np.array_equal(got[key].astype(np.int64), want[key]), key
    assert info.prefix_len == want["prefix_len"]
    assert info.target_len == want["target_len"]
    assert info.decode_ok == want["decode_ok"]
    assert info.useful_pairs == want["useful_pairs"]
    assert info.seq_len == len(ids) and info.host_only == 1
    assert info.n_qtiles == -(-len(ids) // info.block_m)
    p.free()


@pytest.mark.parametrize("name", ["tiny", "t2i_1024", "edit_2ref", "long_4ref"])
def test_plan_bit_exact_on_workloads(name):
    assert_plan_matches_oracle(W.WORKLOADS[name].block_ids())


def test_plan_bit_exact_fuzz():
    rng = np.random.default_rng(21)
    cases = [np.array([-1]), np.array([0]), np.full(300, -1), np.zeros(300, np.int32),
             W.block_ids_from_segments([("image", 128), ("image", 1), ("text", 127)]),
             W.block_ids_from_segments([("text", 1), ("image", 255), ("text", 1), ("image", 2)])]
    for _ in range(40):
        S = int(rng.integers(1, 700))
        cases.append(W.random_layout(rng, S, p_text=float(rng.random()),
                                     max_seg=int(rng.integers(1, 300))))
    for ids in cases:
        assert_plan_matches_oracle(ids)


def test_plan_sizes_of_workloads():
    """Sequence lengths, prefix lengths and visible pairs of the five workloads."""
    expect = {"tiny": (146, 82, 14763), "t2i_1024": (4352, 256, 17858688),
              "edit_2ref": (12400, 8304, 102045880), "long_4ref": (32912, 16528, 709372104)}
    for name, (S, P, pairs) in expect.items():
        info = plan_host(W.WORKLOADS[name].block_ids()).info
        assert (info.seq_len, info.prefix_len, info.useful_pairs) == (S, P, pairs)
        assert info.decode_ok == 1


def status_of(fn):
    with pytest.raises(bca.BcaError) as e:
        fn()
    return e.value.status


def test_plan_rejects_bad_ids():
    assert status_of(lambda: plan_host([-1, -2, 0])) == _lib.BCA_ERR_BLOCK_IDS
    assert status_of(lambda: plan_host([0, 0, -1, 0])) == _lib.BCA_ERR_BLOCK_IDS
    assert status_of(lambda: plan_host([1, 1, 1, 2, 1])) == _lib.BCA_ERR_BLOCK_IDS
    assert status_of(lambda: plan_host([])) == _lib.BCA_ERR_ARG
    lib = _lib.load()
    h = ctypes.c_void_p()
    assert lib.bca_plan(None, 4, 1, ctypes.byref(h)) == _lib.BCA_ERR_ARG
    ids = (ctypes.c_int32 * 2)(-1, 0)
    assert lib.bca_plan(ids, 2, 0x10, ctypes.byref(h)) == _lib.BCA_ERR_ARG
    assert lib.bca_plan(ids, 2, 1, None) == _lib.BCA_ERR_ARG
    assert b"out" in lib.bca_last_error()
    assert lib.bca_plan_free(None) == _lib.BCA_OK


def _t(ptr=0x10000, sb=8 * 4096, ss=4096, sh=128):
    return _lib.BcaTensor(ptr, sb, ss, sh)


def call_prefill(plan, B=1, H=2, D=128, scale=0.0, q=None, k=None, v=None, o=None, kc=None,
                 vc=None):
    lib = _lib.load()
    r = lambda t: None if t is None else ctypes.byref(t)
    return lib.bca_prefill(plan, B, H, D, scale, r(q or _t()), r(k or _t()), r(v or _t()),
                           r(o or _t()), r(kc), r(vc), None)


def call_decode(plan, B=1, H=2, D=128, scale=0.0, q=None, kc=None, vc=None, k=None, v=None, o=None):
    lib = _lib.load()
    r = lambda t: None if t is None else ctypes.byref(t)
    return lib.bca_decode(plan, B, H, D, scale, r(q or _t()), r(kc or _t()), r(vc or _t()),
                          r(k or _t()), r(v or _t()), r(o or _t()), None)


def test_launch_validation_before_any_device_work():
    p = plan_host(W.TINY.block_ids())
    h = p.handle
    lib = _lib.load()
    assert call_prefill(None) == _lib.BCA_ERR_ARG
    assert call_prefill(h, B=0) == _lib.BCA_ERR_ARG
    assert call_prefill(h, H=0) == _lib.BCA_ERR_ARG
    assert call_prefill(h, D=64) == _lib.BCA_ERR_UNSUPPORTED
    assert call_prefill(h, scale=float("nan")) == _lib.BCA_ERR_ARG
    assert call_prefill(h, scale=-1.0) == _lib.BCA_ERR_ARG
    assert call_prefill(h, q=_t(ptr=0x10008)) == _lib.BCA_ERR_ARG          # misaligned
    assert call_prefill(h, k=_t(ss=4100)) == _lib.BCA_ERR_ARG              # stride not x8
    assert call_prefill(h, o=_t(sh=130)) == _lib.BCA_ERR_ARG               # fp32 stride not x4
    assert call_prefill(h, o=_t(sh=132)) == _lib.BCA_ERR_ARG               # host-only plan
    assert b"HOST_ONLY" in lib.bca_last_error()
    assert call_prefill(h, v=_t(ptr=0)) == _lib.BCA_ERR_ARG                # NULL data
    assert call_prefill(h, kc=_t()) == _lib.BCA_ERR_ARG                    # half a cache
    assert call_prefill(h, k=_t(ss=1 << 24)) == _lib.BCA_ERR_ARG           # stride_s >= 2^24
    assert b"2^24" in lib.bca_last_error()
    big = plan_host(np.zeros(300000, np.int32))
    assert call_prefill(big.handle, v=_t(ss=8192)) == _lib.BCA_ERR_ARG      # rows*stride >= 2^31
    assert b"2^31" in lib.bca_last_error()
    assert call_prefill(h) == _lib.BCA_ERR_ARG                             # host-only plan
    assert call_decode(h, D=256) == _lib.BCA_ERR_UNSUPPORTED
    assert call_decode(h, o=_t(ptr=0x10004)) == _lib.BCA_ERR_ARG
    assert call_decode(h) == _lib.BCA_ERR_ARG                              # host-only plan
    text_last = plan_host([-1, 0, 0, -1])
    assert text_last.info.decode_ok == 0
    assert call_decode(text_last.handle) == _lib.BCA_ERR_NO_DECODE
    assert lib.bca_status_str(4) == b"BCA_ERR_NO_DECODE"
    assert lib.bca_status_str(99) == b"unknown status"


def test_python_shim_rejects_bad_shapes_without_gpu():
    torch = pytest.importorskip("torch")
    p = plan_host(W.TINY.block_ids())
    x = torch.zeros((1, 10, 2, 128), dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        bca.prefill(p, x, x, x)  # S != plan's S


def test_cache_descriptor_layout_matches_header(tmp_path):
    """ctypes' bca_kv_cache / bca_tensor / bca_plan_info match the C compiler's layout."""
    import shutil
    import subprocess
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    src = tmp_path / "layout.c"
    src.write_text(
        '#include <stddef.h>\n#include <stdio.h>\n#include "bca.h"\n'
        "int main(void) {\n"
        '  printf("%zu %zu %zu %zu %zu %zu %zu\\n", sizeof(bca_kv_cache),\n'
        "         offsetof(bca_kv_cache, k), offsetof(bca_kv_cache, v),\n"
        "         offsetof(bca_kv_cache, k_scale), offsetof(bca_kv_cache, v_scale),\n"
        "         sizeof(bca_tensor), sizeof(bca_plan_info));\n"
        "  return 0;\n}\n")
    exe = tmp_path / "layout"
    subprocess.run([cc, "-std=c99", "-I", os.path.join(ROOT, "include"), str(src), "-o",
                    str(exe)], check=True)
    got = [int(x) for x in subprocess.run([str(exe)], check=True, capture_output=True,
                                          text=True).stdout.split()]
    C = _lib.BcaKvCache
    want = [ctypes.sizeof(C), C.k.offset, C.v.offset, C.k_scale.offset, C.v_scale.offset,
            ctypes.sizeof(_lib.BcaTensor), ctypes.sizeof(_lib.BcaPlanInfo)]
    assert got == want


def _cache(fmt, k=None, v=None, ks=None, vs=None):
    c = _lib.BcaKvCache()
    c.format = fmt
    c.k, c.v = k or _t(), v or _t()
    c.k_scale = ks or _lib.BcaTensor(0x20000, 4096, 32, 1)
    c.v_scale = vs or _lib.BcaTensor(0x30000, 4096, 32, 1)
    return c


def test_fp8_cache_validation_before_any_device_work():
    p = plan_host(W.TINY.block_ids())
    h = p.handle
    lib = _lib.load()
    r = ctypes.byref

    def pre(c, D=128):
        return lib.bca_prefill_ex(h, 1, 2, D, 0.0, r(_t()), r(_t()), r(_t()), r(_t()),
                                  None if c is None else r(c), None)

    def dec(c, D=128):
        return lib.bca_decode_ex(h, 1, 2, D, 0.0, r(_t()), None if c is None else r(c), r(_t()),
                                 r(_t()), r(_t()), None)

    err = lambda: lib.bca_last_error()
    assert pre(_cache(3)) == _lib.BCA_ERR_ARG and b"unknown format" in err()
    assert pre(_cache(-1)) == _lib.BCA_ERR_ARG
    assert pre(_cache(2, k=_t(ss=4104))) == _lib.BCA_ERR_ARG        # codes: stride not x16
    assert b"multiples of 16" in err()
    assert pre(_cache(0, k=_t(ss=4104))) == _lib.BCA_ERR_ARG        # bf16: stride not x8
    assert pre(_cache(1, v=_t(ptr=0x10008))) == _lib.BCA_ERR_ARG    # codes misaligned
    assert pre(_cache(1, vs=_lib.BcaTensor(0x30002, 0, 1, 1))) == _lib.BCA_ERR_ARG
    assert b"4-byte" in err()
    assert pre(_cache(1, vs=_lib.BcaTensor(0, 0, 1, 1))) == _lib.BCA_ERR_ARG
    assert pre(_cache(2, ks=_lib.BcaTensor(0x20000, 0, -1, 1))) == _lib.BCA_ERR_ARG
    assert pre(_cache(2, k=_t(ss=1 << 24))) == _lib.BCA_ERR_ARG     # 32-bit row offsets
    assert pre(_cache(1, vs=_lib.BcaTensor(0x30000, 0, 1 << 24, 1))) == _lib.BCA_ERR_ARG
    assert b"2^24" in err()
    assert pre(_cache(1, vs=_lib.BcaTensor(0x30000, 0, 1 << 23, 1))) == _lib.BCA_ERR_ARG
    assert b"2^29" in err()                                         # 82 rows * 2^23
    # scales a format does not use are ignored: reaches the host-only check
    unused = _lib.BcaTensor(0, 0, 0, 0)
    assert pre(_cache(0, ks=unused, vs=unused)) == _lib.BCA_ERR_ARG and b"HOST_ONLY" in err()
    assert pre(_cache(1, ks=unused)) == _lib.BCA_ERR_ARG and b"HOST_ONLY" in err()
    assert pre(_cache(2)) == _lib.BCA_ERR_ARG and b"HOST_ONLY" in err()
    assert pre(None) == _lib.BCA_ERR_ARG and b"HOST_ONLY" in err()
    assert pre(_cache(2), D=64) == _lib.BCA_ERR_UNSUPPORTED
    assert dec(None) == _lib.BCA_ERR_ARG and b"cache" in err()       # P > 0 needs a cache
    assert dec(_cache(7)) == _lib.BCA_ERR_ARG and b"unknown format" in err()
    assert dec(_cache(2, vs=_lib.BcaTensor(0x30001, 0, 1, 1))) == _lib.BCA_ERR_ARG
    assert dec(_cache(2)) == _lib.BCA_ERR_ARG and b"HOST_ONLY" in err()
    assert dec(_cache(2), D=256) == _lib.BCA_ERR_UNSUPPORTED
    # the plain entry points are the bf16 format of the same calls
    assert call_decode(h, kc=_t(ss=4100)) == _lib.BCA_ERR_ARG
    p0 = plan_host(np.zeros(50, np.int32))                            # P = 0: no cache needed
    assert lib.bca_decode_ex(p0.handle, 1, 2, 128, 0.0, r(_t()), None, r(_t()), r(_t()), r(_t()),
                             None) == _lib.BCA_ERR_ARG and b"HOST_ONLY" in err()


def test_python_kv_cache_shapes_without_gpu():
    torch = pytest.importorskip("torch")
    p = plan_host(W.TINY.block_ids())
    c = bca.KVCache.empty(p, 2, 3, bca.KVCache.FP8_V, device="cpu")
    assert c.k.dtype == torch.bfloat16 and c.v.dtype == torch.uint8
    assert c.k_scale is None and tuple(c.v_scale.shape) == (2, 82, 3)
    assert c.nbytes() == 2 * 82 * 3 * (128 * 2 + 128 + 4)
    kv = bca.KVCache.empty(p, 1, 2, bca.KVCache.FP8_KV, device="cpu")
    assert kv.k.dtype == torch.uint8 and kv.k_scale is not None
    with pytest.raises(ValueError):
        bca.KVCache(5, c.k, c.v)


def varlen_batch(seed, n_seq, max_len):
    rng = np.random.default_rng(seed)
    return [W.random_layout(rng, int(rng.integers(1, max_len)), p_text=float(rng.random()),
                            max_seg=int(rng.integers(1, 200))) for _ in range(n_seq)]


@pytest.mark.parametrize("seed", [41, 42, 43])
def test_varlen_plan_bit_exact(seed):
    ids_list = varlen_batch(seed, int(np.random.default_rng(seed).integers(1, 9)), 900)
    p = bca.Plan.varlen(ids_list, host_only=True)
    info = p.info
    got = p.export()
    want = [O.plan_from_mask(ids, info.block_m) for ids in ids_list]
    for key in ("row_limit", "kv_full", "kv_end"):
        assert np.array_equal(got[key].astype(np.int64), np.concatenate([w[key] for w in want]))
    segs = np.concatenate([w["segments"].reshape(-1, 3) for w in want])
    assert np.array_equal(got["segments"].astype(np.int64), segs)
    kv_end = np.concatenate([w["kv_end"] for w in want])
    assert np.array_equal(got["order"], np.argsort(-kv_end, kind="stable"))
    assert info.n_sequences == len(ids_list)
    # per sequence: prefix and target as the oracle splits them, packed cache and target rows
    split = [O.prefix_split(ids) for ids in ids_list]
    P = np.array([x[0] for x in split]); N = np.array([x[1] for x in split])
    assert info.prefix_len == P.sum() and info.target_len == N.sum()
    assert info.decode_ok == int(all(x[2] for x in split))
    sq = p.sequences()
    lens = [len(i) for i in ids_list]
    assert np.array_equal(sq[:, 0], O.packed_row_starts(lens)) and np.array_equal(sq[:, 1], lens)
    assert np.array_equal(sq[:, 2], P) and np.array_equal(sq[:, 3], N)
    assert np.array_equal(sq[:, 4], np.concatenate([[0], np.cumsum(P)[:-1]]))
    assert np.array_equal(sq[:, 5], np.concatenate([[0], np.cumsum(N)[:-1]]))
    assert info.seq_len == sum(len(i) for i in ids_list) == info.rows
    assert info.useful_pairs == sum(int(w["useful_pairs"]) for w in want)
    assert info.n_qtiles == sum(-(-len(i) // info.block_m) for i in ids_list)
    gaps = bca.Plan.varlen(ids_list, row_start=[1000 * b + 7 for b in range(len(ids_list))],
                           host_only=True)
    assert gaps.info.rows == 1000 * (len(ids_list) - 1) + 7 + len(ids_list[-1])


def test_varlen_plan_errors():
    a, b = np.array([-1, 0, 0], np.int32), np.array([-1, -1], np.int32)
    status = lambda f: status_of(f)
    assert status(lambda: bca.Plan.varlen([a, b], row_start=[0, 2], host_only=True)) == \
        _lib.BCA_ERR_ARG                                                # overlap
    assert b"overlap" in _lib.load().bca_last_error()
    assert status(lambda: bca.Plan.varlen([a, b], row_start=[-1, 5], host_only=True)) == \
        _lib.BCA_ERR_ARG
    assert status(lambda: bca.Plan.varlen([a, np.array([], np.int32)], host_only=True)) == \
        _lib.BCA_ERR_ARG                                                # empty sequence
    assert status(lambda: bca.Plan.varlen([a, np.array([0, -1, 0])], host_only=True)) == \
        _lib.BCA_ERR_BLOCK_IDS
    assert b"sequence 1" in _lib.load().bca_last_error()
    # ids past int32 are rejected before they reach the library (not wrapped)
    assert status(lambda: bca.Plan.varlen([a, np.array([-1, 2**31], np.int64)],
                                          host_only=True)) == _lib.BCA_ERR_BLOCK_IDS
    assert status(lambda: bca.Plan(np.array([0, 2**31, 2**31], np.uint32), host_only=True)) == \
        _lib.BCA_ERR_BLOCK_IDS
    ok = bca.Plan.varlen([a, b], row_start=[3, 0], host_only=True)   # gaps, any order
    assert ok.info.rows == 6
    lib = _lib.load()
    h = ctypes.c_void_p()
    lens = (ctypes.c_int64 * 2)(3, 2)
    assert lib.bca_plan_varlen(None, lens, None, 2, 0, ctypes.byref(h)) == _lib.BCA_ERR_ARG
    # a batch plan is not a single-sequence prefill
    assert call_prefill(ok.handle) == _lib.BCA_ERR_ARG
    assert b"bca_prefill_varlen" in lib.bca_last_error()
    r = ctypes.byref
    assert lib.bca_prefill_varlen(ok.handle, 2, 64, 0.0, r(_t()), r(_t()), r(_t()), r(_t()),
                                  None, None, None) == _lib.BCA_ERR_UNSUPPORTED
    assert lib.bca_prefill_varlen(ok.handle, 2, 128, 0.0, r(_t()), r(_t()), r(_t()), r(_t()),
                                  None, None, None) == _lib.BCA_ERR_ARG  # host-only plan
    assert b"HOST_ONLY" in lib.bca_last_error()
    assert lib.bca_prefill_varlen(ok.handle, 2, 128, 0.0, r(_t()), r(_t()), r(_t()), r(_t()),
                                  r(_t()), None, None) == _lib.BCA_ERR_ARG  # one cache tensor
    assert b"both" in lib.bca_last_error()
    # decode over the batch: sequence 1 ends in text
    assert ok.info.decode_ok == 0
    assert lib.bca_decode_varlen(ok.handle, 2, 128, 0.0, r(_t()), r(_t()), r(_t()), r(_t()),
                                 r(_t()), r(_t()), None) == _lib.BCA_ERR_NO_DECODE
    img = bca.Plan.varlen([a, np.array([-1, 0], np.int32)], host_only=True)
    assert img.info.decode_ok == 1 and img.info.prefix_len == 2 and img.info.target_len == 3
    assert call_decode(img.handle) == _lib.BCA_ERR_ARG                # several sequences
    assert b"bca_decode_varlen" in lib.bca_last_error()
    assert lib.bca_decode_varlen(img.handle, 2, 64, 0.0, r(_t()), r(_t()), r(_t()), r(_t()),
                                 r(_t()), r(_t()), None) == _lib.BCA_ERR_UNSUPPORTED
    assert lib.bca_decode_varlen(img.handle, 2, 128, 0.0, r(_t()), None, None, r(_t()),
                                 r(_t()), r(_t()), None) == _lib.BCA_ERR_ARG  # prefix needs caches
    assert lib.bca_decode_varlen(img.handle, 2, 128, 0.0, r(_t()), r(_t()), r(_t()), r(_t()),
                                 r(_t()), r(_t()), None) == _lib.BCA_ERR_ARG  # host-only plan
    assert b"HOST_ONLY" in lib.bca_last_error()


def test_cache_dequantize_argument_errors():
    """bca_cache_dequantize rejects bad arguments before any device call (only invalid calls are
    made here: a valid one would launch)."""
    lib = _lib.load()
    r = ctypes.byref
    err = lambda: lib.bca_last_error()

    def call(B=1, P=82, H=2, D=128, c="ok", ko=None, vo=None):
        cache = _cache(2) if c == "ok" else c
        return lib.bca_cache_dequantize(B, P, H, D, None if cache is None else r(cache),
                                        r(ko or _t()), r(vo or _t()), None)

    assert call(D=64) == _lib.BCA_ERR_UNSUPPORTED
    assert call(B=0) == _lib.BCA_ERR_ARG
    assert call(P=0) == _lib.BCA_ERR_ARG
    assert call(H=0) == _lib.BCA_ERR_ARG
    assert call(P=1 << 31) == _lib.BCA_ERR_ARG and b"2^31" in err()
    assert call(c=None) == _lib.BCA_ERR_ARG and b"NULL" in err()
    assert call(c=_cache(5)) == _lib.BCA_ERR_ARG and b"unknown format" in err()
    assert call(c=_cache(1, v=_t(ptr=0x10008))) == _lib.BCA_ERR_ARG
    assert call(c=_cache(2, ks=_lib.BcaTensor(0x20002, 0, 1, 1))) == _lib.BCA_ERR_ARG
    assert call(ko=_t(ptr=0x10004)) == _lib.BCA_ERR_ARG and b"k_out" in err()
    assert call(vo=_t(ss=4100)) == _lib.BCA_ERR_ARG and b"v_out" in err()
    assert call(vo=_lib.BcaTensor(0, 0, 4096, 128)) == _lib.BCA_ERR_ARG and b"NULL" in err()


def test_split_workspace_sizing_and_errors():
    lib = _lib.load()
    p = plan_host(W.EDIT_2REF_T512.block_ids())            # P = 8,304, N = 1,024
    # B = 1, H = 32: 8 query tiles x 32 heads = 256 workgroups -> 3 ranges (768 workgroups: one
    # round of three per CU); 16 heads -> 6 ranges
    nbytes, used = bca.split_workspace(p, 1, 32)
    assert used == 3 and nbytes == 3 * 1 * 1024 * 32 * 130 * 4
    assert bca.split_workspace(p, 1, 16)[1] == 6
    assert bca.split_workspace(p, 1, 32, 1) == (0, 1)      # one range: the plain decode
    assert bca.split_workspace(p, 1, 32, 146) == (146 * 1024 * 32 * 520, 146)
    assert bca.split_workspace(p, 1, 32, 500)[1] == 146    # at most one range per key tile
    assert bca.split_workspace(p, 1, 32, 3)[1] == 3
    # the CFG shape already fills the GPU: the library keeps one range
    big = plan_host(W.EDIT_2REF.block_ids())
    assert bca.split_workspace(big, 2, 32) == (0, 1)
    with pytest.raises(bca.BcaError) as e:
        bca.split_workspace(p, 1, 32, -1)
    assert e.value.status == _lib.BCA_ERR_ARG
    text_last = plan_host([-1, 0, 0, -1])
    with pytest.raises(bca.BcaError) as e:
        bca.split_workspace(text_last, 1, 1)
    assert e.value.status == _lib.BCA_ERR_NO_DECODE
    r = ctypes.byref
    c = _cache(0)
    call = lambda n, ws, wsb: lib.bca_decode_split(p.handle, 1, 32, 128, 0.0, r(_t()), r(c),
                                                   r(_t()), r(_t()), r(_t()), n, ws, wsb, None)
    assert call(4, None, 0) == _lib.BCA_ERR_ARG                                # no workspace
    assert call(4, ctypes.c_void_p(0x100008), 1 << 30) == _lib.BCA_ERR_ARG      # misaligned
    assert call(4, ctypes.c_void_p(0x100000), 1000) == _lib.BCA_ERR_ARG        # too small
    assert b"needed" in lib.bca_last_error()
    assert call(-2, None, 0) == _lib.BCA_ERR_ARG
    assert call(4, ctypes.c_void_p(0x100000), 1 << 30) == _lib.BCA_ERR_ARG     # host-only plan
    assert b"HOST_ONLY" in lib.bca_last_error()
    assert call(1, None, 0) == _lib.BCA_ERR_ARG and b"HOST_ONLY" in lib.bca_last_error()


def test_grid_guards_count_work_items():
    """Launch-size checks count work-items (at most 2^32 - 1 per grid dimension), before any
    device call: a host-only plan and fake pointers reach them."""
    lib = _lib.load()
    p = plan_host(W.TINY.block_ids())
    # 12-wave prefill tiles: tiles * B * H * 768 work-items
    assert call_prefill(p.handle, B=1 << 20, H=32) == _lib.BCA_ERR_ARG
    assert b"grid" in lib.bca_last_error()
    # the cache expansion: ceil(B * P * H / 16) blocks of 256
    r = ctypes.byref
    rc = lib.bca_cache_dequantize(1 << 22, 82, 32, 128, r(_cache(2)), r(_t()), r(_t()), None)
    assert rc == _lib.BCA_ERR_ARG and b"too large" in lib.bca_last_error()
    p.free()
