"""Benchmark of the block-causal attention hot path on one MI355X.

A step is one pass of the whole path on the 2-reference 1024^2 edit shape:
  * block-causal prefill of [t48][ref 4096][t40][ref 4096][t24][target 4096] (S = 12,400, B = 1,
    H = 32, D = 128, bf16 in, fp32 out) that also writes the prefix K/V cache (P = 8,304), then
  * one prefix-cached decode step under CFG (B = 2, N = 4,096 target queries over
    8,304 + 4,096 keys, no mask) with fresh target Q/K/V (pre-generated, cycled).
The plan is built once before timing (it serves all layers and steps).  Inputs are resident in
HBM before the timed region.  Useful work = 4 * D flops per visible (query, key) pair.

Beside the step (side keys of the same JSON line, not part of `value`): the text-to-image 1024^2
prefill (S = 4,352) and the four-reference 2048^2-target prefill (S = 32,912); the 49 cached
steps of one generation, each with its own fresh target Q/K/V, timed call by call; the plan's
build time split into host planning, device upload and first launches; the FP8 cache, Q/K
prologue, varlen and split-decode calls.

Prints ONE JSON line on stdout.  Diagnostics go to stderr.
"""
from __future__ import annotations

import argparse
import gc
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "useful attention TFLOP/s + ms/call (prefill, decode), fraction of bf16 MFMA peak"
PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, published figure
HEAD_DIM = 128
N_DECODE_SETS = 4


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def to_dev(torch, bits, dev):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)


KERNEL_SOURCE = os.path.join(ROOT, "block_causal_attention_amd", "csrc", "bca_attention.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.json")
SQ_FILE = os.path.join(ROOT, "profiles", "sq_counters.json")


def kernel_source_sha256():
    import hashlib
    try:
        with open(KERNEL_SOURCE, "rb") as f:
            return hashlib.sha256(f.read()).hexdigest()
    except OSError:
        return None


def profile_entry(path, kernel):
    """The committed rocprofv3 summary of `kernel` in `path` (a JSON file under profiles/), or
    None when it was taken on a different kernel source than the one being benchmarked."""
    try:
        with open(path) as f:
            entry = json.load(f).get(kernel)
    except (OSError, ValueError):
        return None
    if not entry or entry.get("kernel_source_sha256") != kernel_source_sha256():
        return None
    return entry


def measured_traffic(kernel):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 FETCH_SIZE / WRITE_SIZE
    passes (already scaled by the copy calibration), or None when those counters were taken on
    a different kernel source than the one being benchmarked."""
    entry = profile_entry(TRAFFIC_FILE, kernel)
    return None if entry is None else entry.get("bytes_per_launch")


def mfma_utilisation():
    """MFMA busy fractions per kernel from the committed rocprofv3 SQ-counter pass
    (SQ_VALU_MFMA_BUSY_CYCLES over SIMD cycles and over busy-CU cycles), for the kernel source
    being benchmarked only."""
    out = {}
    for key in ("prefill_b1", "decode_cfg_b2"):
        e = profile_entry(SQ_FILE, key)
        if e is not None:
            out[key] = {k: e[k] for k in ("kernel", "mfma_busy_of_simd_cycles",
                                          "mfma_busy_of_busy_cu_cycles", "cu_busy_of_dispatch")
                        if k in e}
    return out or None


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or None


def cpu_baseline(W, lay, ids, P, N, budget_rows, heads):
    """Times the float64 CPU oracle on a bounded sample of the same workload: every query row of
    heads [0, heads) of batch 0 of the prefill, and every target row of those heads of one
    cached decode (about 10 s on the 16 host cores of an MI355X machine at 10 heads)."""
    from oracle import bca_oracle as O
    threads = None
    try:
        from threadpoolctl import threadpool_info
        threads = max((p.get("num_threads") or 0) for p in threadpool_info()) or None
    except Exception:
        pass
    S = lay.seq_len
    q, k, v = W.qkv(W.SEEDS["edit_2ref"], 1, S, heads, scaled=True)
    qf, kf, vf = (W.bf16_bits_to_f32(x) for x in (q, k, v))
    rows = np.arange(min(S, budget_rows))
    t0 = time.perf_counter()
    O.attention(qf, kf, vf, ids, rows=rows)
    t_pre = time.perf_counter() - t0
    hi = O.row_key_limits(ids)
    flops_pre = 4.0 * HEAD_DIM * heads * float(hi[rows].sum())
    t0 = time.perf_counter()
    O.decode(qf[:, P:], kf[:, :P], vf[:, :P], kf[:, P:], vf[:, P:])
    t_dec = time.perf_counter() - t0
    flops_dec = 4.0 * HEAD_DIM * heads * N * (P + N)
    value = (flops_pre + flops_dec) / (t_pre + t_dec) / 1e12
    return {
        "value": value, "unit": "TFLOP/s", "cores": threads or os.cpu_count(), "kind": "oracle",
        "cpu_model": cpu_model(), "host_cpus": os.cpu_count(),
        "sample": (f"float64 NumPy oracle, batch 0, heads 0..{heads - 1}: {rows.size} prefill rows "
                   f"of the S={S} block-causal layout ({t_pre:.2f} s) + all {N} target rows of one "
                   f"cached decode over {P + N} keys ({t_dec:.2f} s); value = useful flops / time"),
        "prefill_ms_per_head": t_pre * 1e3 * S / rows.size / heads,
        "decode_ms_per_head": t_dec * 1e3 / heads,
    }


# Untimed run-in before each measurement.  The card lowers its clocks while it idles (the host
# generates the next inputs between measurements) and raises them over the first tens of
# milliseconds of sustained load; the first dispatches of a cold run are up to a third slower.
SETTLE = {"main_ms": 500.0, "extra_ms": 200.0}


def settle(torch, fn, ms):
    """Calls fn (one unit of the work about to be timed) untimed for `ms` of wall time."""
    t0 = time.perf_counter()
    n = 0
    while (time.perf_counter() - t0) * 1e3 < ms:
        for _ in range(4):
            fn()
            n += 1
        torch.cuda.synchronize()
    return n


def fp8_timings(torch, bca, W, plan, q, k, v, o, sets, od, flops_pre, flops_dec, Bd, S, H, P,
                dev, iters=10):
    """The same prefill and decode calls with the prefix cache stored as FP8 E4M3 (V only, then
    K and V): ms per call, useful TFLOP/s and the cache bytes per layer of the CFG pair; also the
    cache's expansion to bf16 alone (GB/s over codes + scales read and bf16 written) and followed
    by the bf16 decode."""
    out = {}
    wide = bca.KVCache.empty(plan, Bd, H, bca.KVCache.BF16, device=dev)
    for name, fmt in (("fp8_v", bca.KVCache.FP8_V), ("fp8_kv", bca.KVCache.FP8_KV)):
        c1 = bca.KVCache.empty(plan, 1, H, fmt, device=dev)
        c2 = bca.KVCache.empty(plan, Bd, H, fmt, device=dev)
        q2, k2, v2 = (to_dev(torch, x, dev) for x in W.qkv(W.SEEDS["edit_2ref_cfg"], Bd, S, H))
        bca.prefill_ex(plan, q2, k2, v2, c2)
        del q2, k2, v2
        n_unit = [0]

        def unit():
            qt, kt, vt = sets[n_unit[0] % len(sets)]
            n_unit[0] += 1
            bca.prefill_ex(plan, q, k, v, c1, out=o)
            bca.decode_ex(plan, qt, c2, kt, vt, out=od)
        settle(torch, unit, SETTLE["extra_ms"])
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        ev[0].record()
        for i in range(iters):
            bca.prefill_ex(plan, q, k, v, c1, out=o)
        ev[1].record()
        for i in range(iters):
            qt, kt, vt = sets[i % len(sets)]
            bca.decode_ex(plan, qt, c2, kt, vt, out=od)
        ev[2].record()
        # the layer's cache expanded to bf16 first, then the bf16 decode
        for i in range(iters):
            bca.dequantize_cache(c2, wide)
        ev.append(torch.cuda.Event(enable_timing=True))
        ev[3].record()
        for i in range(iters):
            qt, kt, vt = sets[i % len(sets)]
            bca.dequantize_cache(c2, wide)
            bca.decode_ex(plan, qt, wide, kt, vt, out=od)
        ev.append(torch.cuda.Event(enable_timing=True))
        ev[4].record()
        torch.cuda.synchronize()
        pre_ms = ev[0].elapsed_time(ev[1]) / iters
        dec_ms = ev[1].elapsed_time(ev[2]) / iters
        exp_ms = ev[2].elapsed_time(ev[3]) / iters
        both_ms = ev[3].elapsed_time(ev[4]) / iters
        moved = c2.nbytes() + wide.nbytes()          # codes + scales read, bf16 written
        out[name] = {"prefill_ms": round(pre_ms, 4),
                     "prefill_useful_tflops": round(flops_pre / (pre_ms * 1e-3) / 1e12, 2),
                     "decode_ms": round(dec_ms, 4),
                     "decode_useful_tflops": round(flops_dec / (dec_ms * 1e-3) / 1e12, 2),
                     "expand_ms": round(exp_ms, 4),
                     "expand_gbs": round(moved / (exp_ms * 1e-3) / 1e9, 1),
                     "expand_then_decode_ms": round(both_ms, 4),
                     "expand_then_decode_useful_tflops": round(flops_dec / (both_ms * 1e-3) / 1e12, 2),
                     "cache_mb_per_layer_b2": round(c2.nbytes() / 1e6, 2)}
        log(f"{name}: prefill {pre_ms:.3f} ms, decode {dec_ms:.3f} ms, expand {exp_ms:.3f} ms "
            f"({moved / (exp_ms * 1e-3) / 1e9:.0f} GB/s), expand+decode {both_ms:.3f} ms, cache "
            f"{c2.nbytes() / 1e6:.1f} MB per layer (B={Bd})")
        del c1, c2
    out["bf16_cache_mb_per_layer_b2"] = round(2 * Bd * P * H * HEAD_DIM * 2 / 1e6, 2)
    return out


PEAK_HBM_GBS = 8000.0  # MI355X HBM3E, published figure


def prologue_timings(torch, bca, W, ids, Bd, S, N, H, dev, iters=20):
    """The Q/K prologue (per-head RMS norm + three-axis RoPE) on the prefill shape and on the
    CFG target rows: ms per call and effective HBM GB/s.  Algorithmic bytes: Q and K read once
    and written once (bf16), the table rows read once, the weights ignored (1 KB)."""
    table = torch.from_numpy(bca.rope_table(bca.rope_positions(ids))).to(dev)
    wq = torch.ones(HEAD_DIM, dtype=torch.float32, device=dev)
    wk = torch.ones_like(wq)
    out = {}
    for name, B, rows, tab in (("prefill_b1", 1, S, table), ("target_b2", Bd, N, table[S - N:].contiguous())):
        qb, kb, _, _ = W.prologue_inputs(7, B, rows, H)
        q, k = to_dev(torch, qb, dev), to_dev(torch, kb, dev)
        settle(torch, lambda: bca.qk_prologue(q, k, wq, wk, tab, q_out=q, k_out=k),
               SETTLE["extra_ms"])
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(iters):
            bca.qk_prologue(q, k, wq, wk, tab, q_out=q, k_out=k)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / iters
        nbytes = 4 * B * rows * H * HEAD_DIM * 2 + rows * 64 * 2 * 4
        gbs = nbytes / (ms * 1e-3) / 1e9
        out[name] = {"ms": round(ms, 4), "bytes": nbytes, "GB/s": round(gbs, 1),
                     "frac_hbm_peak": round(gbs / PEAK_HBM_GBS, 4)}
        log(f"prologue {name}: {ms:.4f} ms, {gbs:.0f} GB/s ({gbs / PEAK_HBM_GBS:.1%} of HBM peak)")
        del q, k
    return out


def varlen_timing(torch, bca, W, dev, H, iters=10):
    """Batch-of-sequences prefill on a NEO-Unify-table-like batch (batch 16, max_seq_len 8,192,
    246 image tokens; heads and width are not on that page: 32 x 128 assumed), packed."""
    ids_list, lens = W.neo_like_batch(16, 16, 8192, 246)
    plan = bca.Plan.varlen(ids_list)
    R = int(sum(lens))
    q, k, v = (to_dev(torch, x[0], dev) for x in W.qkv(17, 1, R, H))
    o = torch.empty((R, H, HEAD_DIM), dtype=torch.float32, device=dev)
    settle(torch, lambda: bca.prefill_varlen(plan, q, k, v, out=o), SETTLE["extra_ms"])
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(iters):
        bca.prefill_varlen(plan, q, k, v, out=o)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / iters
    flops = 4.0 * HEAD_DIM * H * plan.info.useful_pairs
    tf = flops / (ms * 1e-3) / 1e12
    log(f"varlen NEO-like batch 16 x <=8192 ({R} rows): {ms:.3f} ms = {tf:.1f} TFLOP/s")
    plan.free()
    return {"workload": "16 sequences, max 8192 positions (lengths 4096..8192), 246 image tokens, "
                        f"H={H}, packed ({R} rows)",
            "ms": round(ms, 4), "useful_tflops": round(tf, 2),
            "frac_peak": round(tf / PEAK_BF16_TFLOPS, 4), "useful_gflop": round(flops / 1e9, 1)}


def cfg_varlen_timing(torch, bca, W, dev, iters=10):
    """CFG branches whose prompts differ in length, one launch each for the prefill (storing
    each branch's own prefix cache) and for the cached step over the two caches: the 2-ref edit
    (S = 12,400) as the cond branch and the same layout with an 8-position prompt (S = 12,360)
    as the uncond branch, packed, H = 32."""
    ids_list = [lay.block_ids() for lay in W.CFG_VARLEN]
    H = W.EDIT_2REF.heads
    plan = bca.Plan.varlen(ids_list)
    sq = plan.sequences()
    R, P, N = int(sq[:, 1].sum()), plan.info.prefix_len, plan.info.target_len
    q, k, v = (to_dev(torch, x[0], dev) for x in W.qkv(W.SEEDS["cfg_varlen"], 1, R, H))
    o = torch.empty((R, H, HEAD_DIM), dtype=torch.float32, device=dev)
    kc = torch.empty((P, H, HEAD_DIM), dtype=torch.bfloat16, device=dev)
    vc = torch.empty_like(kc)
    qt, kt, vt = (to_dev(torch, x[0], dev) for x in W.qkv(W.SEEDS["cfg_varlen"] + 1, 1, N, H))
    od = torch.empty((N, H, HEAD_DIM), dtype=torch.float32, device=dev)
    pre = lambda: bca.prefill_varlen(plan, q, k, v, k_cache=kc, v_cache=vc, out=o)
    dec = lambda: bca.decode_varlen(plan, qt, kc, vc, kt, vt, out=od)
    out = {"workload": "CFG pair, packed: cond 2-ref edit S=12400 (P=8304) + uncond with an "
                       f"8-position prompt S=12360 (P=8264), N=4096 each, H={H}"}
    flops = {"prefill": 4.0 * HEAD_DIM * H * plan.info.useful_pairs,
             "decode": sum(4.0 * HEAD_DIM * H * int(n) * int(p + n) for p, n in sq[:, 2:4])}
    for name, fn in (("prefill", pre), ("decode", dec)):
        settle(torch, fn, SETTLE["extra_ms"])
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(iters):
            fn()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / iters
        tf = flops[name] / (ms * 1e-3) / 1e12
        out[name] = {"ms": round(ms, 4), "useful_tflops": round(tf, 2),
                     "frac_peak": round(tf / PEAK_BF16_TFLOPS, 4),
                     "useful_gflop": round(flops[name] / 1e9, 1)}
        log(f"cfg varlen {name}: {ms:.3f} ms = {tf:.1f} TFLOP/s")
    plan.free()
    return out


def split_decode_timing(torch, bca, W, dev, iters=20):
    """Cached step of the 512^2-target edit (N = 1,024 under P = 8,304, B = 1, H = 32): the
    plain decode (8 x 32 = 256 workgroups) against the split-KV decode (library-chosen ranges)."""
    lay = W.EDIT_2REF_T512
    ids = lay.block_ids()
    H = lay.heads
    plan = bca.Plan(ids)
    P, N = plan.info.prefix_len, plan.info.target_len
    qb, kb, vb = W.qkv(W.SEEDS["edit_2ref_t512"], 1, len(ids), H)
    cache = bca.KVCache(bca.KVCache.BF16, to_dev(torch, kb[:, :P], dev), to_dev(torch, vb[:, :P], dev))
    q, k, v = (to_dev(torch, x[:, P:], dev) for x in (qb, kb, vb))
    nbytes, used = bca.split_workspace(plan, 1, H)
    ws = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=dev)
    o = torch.empty((1, N, H, HEAD_DIM), dtype=torch.float32, device=dev)
    flops = 4.0 * HEAD_DIM * H * N * (P + N)
    out = {"workload": f"512^2 target under two 1024^2 references: N={N}, P={P}, B=1, H={H}",
           "useful_gflop": round(flops / 1e9, 2)}
    for name, fn in (("plain", lambda: bca.decode_ex(plan, q, cache, k, v, out=o)),
                     ("split", lambda: bca.decode_split(plan, q, cache, k, v, workspace=ws, out=o))):
        settle(torch, fn, SETTLE["extra_ms"])
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(iters):
            fn()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / iters
        out[name] = {"ms": round(ms, 4), "useful_tflops": round(flops / (ms * 1e-3) / 1e12, 2)}
        log(f"512^2-target decode, {name}: {ms:.4f} ms = {flops / (ms * 1e-3) / 1e12:.1f} TFLOP/s")
    out["split"]["ranges"] = used
    plan.free()
    return out


def decode_b1_timing(torch, bca, plan, kc2, vc2, sets, N, H, S, dev, iters=20):
    """The cached step without CFG (one branch, B = 1; the pages' production default of guidance
    scale 1): batch item 0 of the CFG pair's cache and of the first target set."""
    kc1, vc1 = kc2[:1].contiguous(), vc2[:1].contiguous()
    qt, kt, vt = (x[:1].contiguous() for x in sets[0])
    o = torch.empty((1, N, H, HEAD_DIM), dtype=torch.float32, device=dev)
    fn = lambda: bca.decode(plan, qt, kc1, vc1, kt, vt, out=o)
    settle(torch, fn, SETTLE["extra_ms"])
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(iters):
        fn()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / iters
    flops = 4.0 * HEAD_DIM * H * N * S
    tf = flops / (ms * 1e-3) / 1e12
    log(f"cached step without CFG (B=1): {ms:.4f} ms = {tf:.1f} TFLOP/s")
    return {"workload": f"one cached step without CFG: B=1, N={N} over {S} keys, H={H}, "
                        f"launch {list(bca.decode_layout(N, H))}",
            "ms": round(ms, 4), "useful_tflops": round(tf, 2),
            "frac_peak": round(tf / PEAK_BF16_TFLOPS, 4), "useful_gflop": round(flops / 1e9, 1)}


def prefill_timing(torch, bca, W, name, dev, iters=10):
    """One prefill shape on its own (B = 1, H = 32, writing its prefix cache): ms per call (mean
    and median of event-timed calls) and useful TFLOP/s from the median."""
    lay = W.WORKLOADS[name]
    ids = lay.block_ids()
    S, H = lay.seq_len, lay.heads
    plan = bca.Plan(ids)
    P = plan.info.prefix_len
    q, k, v = (to_dev(torch, x, dev) for x in W.qkv(W.SEEDS[name], 1, S, H))
    o = torch.empty((1, S, H, HEAD_DIM), dtype=torch.float32, device=dev)
    kc = torch.empty((1, P, H, HEAD_DIM), dtype=torch.bfloat16, device=dev)
    vc = torch.empty_like(kc)

    def call():
        bca.prefill(plan, q, k, v, out=o, k_cache=kc, v_cache=vc)
    settle(torch, call, SETTLE["extra_ms"])
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(iters + 1)]
    ev[0].record()
    for i in range(iters):
        call()
        ev[i + 1].record()
    torch.cuda.synchronize()
    ms = np.array([ev[i].elapsed_time(ev[i + 1]) for i in range(iters)])
    flops = 4.0 * HEAD_DIM * H * plan.info.useful_pairs
    tf = flops / (np.median(ms) * 1e-3) / 1e12
    log(f"prefill {name} S={S}: {ms.mean():.3f} ms (median {np.median(ms):.3f}) = {tf:.1f} TFLOP/s")
    plan.free()
    return {"workload": f"{lay.name}, S={S} (P={P}, N={S - P}), B=1, H={H}, writes the prefix cache",
            "ms": round(float(ms.mean()), 4), "ms_median": round(float(np.median(ms)), 4),
            "useful_tflops": round(tf, 2), "frac_peak": round(tf / PEAK_BF16_TFLOPS, 4),
            "useful_gflop": round(flops / 1e9, 1)}


def decode_generation_timing(torch, bca, plan, kc2, vc2, od, Bd, N, H, flops_dec, dev,
                             steps=49, base_seed=4000):
    """The cached steps of one generation (50 denoising steps = one prefill + 49 cached steps):
    49 decode calls over the same CFG-pair prefix cache, each with its own fresh target Q/K/V,
    all drawn and resident before timing, each call timed with its own event pair.  The fresh
    inputs are drawn on the device (torch's Philox generator seeded base_seed + step,
    N(0,1)/sqrt(128) in fp32, rounded to bf16), so that 49 x 201 MB of inputs take no host time."""
    sets = []
    for s in range(1, steps + 1):
        g = torch.Generator(device=dev)
        g.manual_seed(base_seed + s)
        sets.append(tuple((torch.randn((Bd, N, H, HEAD_DIM), generator=g, device=dev,
                                       dtype=torch.float32) * (1.0 / np.sqrt(HEAD_DIM)))
                          .to(torch.bfloat16) for _ in range(3)))
    settle(torch, lambda: bca.decode(plan, *sets[0][:1], kc2, vc2, *sets[0][1:], out=od),
           SETTLE["extra_ms"])
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    ev[0].record()
    for i, (qt, kt, vt) in enumerate(sets):
        bca.decode(plan, qt, kc2, vc2, kt, vt, out=od)
        ev[i + 1].record()
    torch.cuda.synchronize()
    ms = np.array([ev[i].elapsed_time(ev[i + 1]) for i in range(steps)])
    del sets
    tf = flops_dec / (np.median(ms) * 1e-3) / 1e12
    log(f"49 cached steps: median {np.median(ms):.3f} ms, mean {ms.mean():.3f}, total "
        f"{ms.sum():.2f} ms = {tf:.1f} TFLOP/s (median)")
    return {"workload": f"49 cached CFG steps, B={Bd}, N={N}, {H} heads, fresh target Q/K/V per "
                        "step (device-drawn, seeds 4001..4049)",
            "steps": steps, "ms_median": round(float(np.median(ms)), 4),
            "ms_mean": round(float(ms.mean()), 4), "ms_total": round(float(ms.sum()), 3),
            "ms_min": round(float(ms.min()), 4), "ms_max": round(float(ms.max()), 4),
            "useful_tflops_median": round(tf, 2),
            "frac_peak_median": round(tf / PEAK_BF16_TFLOPS, 4)}


def plan_timing(torch, bca, W, ids, dev, reps=5):
    """Where the plan's build time goes: host planning alone (host-only plans: the first call in
    the process, then the median of `reps` more), for this shape, the 4-ref long layout and the
    NEO-like varlen batch; and the full build (host planning + one device allocation and copy)
    twice, the first one in the process paying the runtime's first-use costs."""
    def host_ms(make):
        ts = []
        for _ in range(reps + 1):
            t0 = time.perf_counter()
            h = make()
            ts.append((time.perf_counter() - t0) * 1e3)
            h.free()
        return round(ts[0], 3), round(float(np.median(ts[1:])), 3)
    out = {}
    out["host_first_ms"], out["host_ms"] = host_ms(lambda: bca.Plan(ids, host_only=True))
    ids5 = W.LONG_4REF.block_ids()
    out["host_ms_long_4ref"] = host_ms(lambda: bca.Plan(ids5, host_only=True))[1]
    neo, _ = W.neo_like_batch(16, 16, 8192, 246)
    out["host_ms_varlen_neo16x8192"] = host_ms(lambda: bca.Plan.varlen(neo, host_only=True))[1]
    for key in ("full_first_ms", "full_again_ms"):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        p = bca.Plan(ids)
        out[key] = round((time.perf_counter() - t0) * 1e3, 3)
        p.free()
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--settle-ms", type=float, default=SETTLE["main_ms"],
                    help="untimed steps for this long before the warm-up steps (the side "
                         "measurements get up to 200 ms each): the GPU's clocks ramp up over the "
                         "first tens of milliseconds of sustained load")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=12400,
                    help="prefill rows in the CPU-oracle sample")
    ap.add_argument("--cpu-heads", type=int, default=10,
                    help="heads in the CPU-oracle sample")
    ap.add_argument("--no-fp8", action="store_true",
                    help="skip the FP8 prefix-cache timings (reported beside the bf16 step)")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the prologue, varlen and split-decode timings (profiling runs)")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run a device-to-device copy of MIB MiB (HBM counter calibration)")
    args = ap.parse_args()
    if args.calibrate_copy:
        import torch
        n = args.calibrate_copy << 20
        x = torch.ones(n, dtype=torch.uint8, device="cuda:0")
        y = torch.empty_like(x)
        torch.cuda.synchronize()
        y.copy_(x)
        torch.cuda.synchronize()
        print(json.dumps({"calibration_copy_bytes": n, "read_bytes": n, "write_bytes": n}))
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported (the path "
              "is built and measured on a single MI355X; sharding across GPUs is not built)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import bca_workloads as W
    import block_causal_attention_amd as bca

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    pre = W.EDIT_2REF
    cfg = W.EDIT_2REF_CFG
    ids = pre.block_ids()
    S, H = pre.seq_len, pre.heads
    plan_split = plan_timing(torch, bca, W, ids, dev)
    t0 = time.perf_counter()
    plan = bca.Plan(ids)
    plan_ms = (time.perf_counter() - t0) * 1e3
    info = plan.info
    P, N = info.prefix_len, info.target_len
    pairs = info.useful_pairs

    # prefill inputs (B = 1) and its cache
    qb, kb, vb = W.qkv(W.SEEDS["edit_2ref"], 1, S, H)
    q, k, v = (to_dev(torch, x, dev) for x in (qb, kb, vb))
    o = torch.empty((1, S, H, HEAD_DIM), dtype=torch.float32, device=dev)
    kc1 = torch.empty((1, P, H, HEAD_DIM), dtype=torch.bfloat16, device=dev)
    vc1 = torch.empty_like(kc1)
    # CFG pair (B = 2): prefix cache from a B = 2 prefill, then fresh target Q/K/V per step
    Bd = cfg.batch
    q2, k2, v2 = (to_dev(torch, x, dev) for x in W.qkv(W.SEEDS["edit_2ref_cfg"], Bd, S, H))
    kc2 = torch.empty((Bd, P, H, HEAD_DIM), dtype=torch.bfloat16, device=dev)
    vc2 = torch.empty_like(kc2)
    o2 = torch.empty((Bd, S, H, HEAD_DIM), dtype=torch.float32, device=dev)
    # the process's first launch (module load and first-dispatch costs; wall clock)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    bca.prefill(plan, q2, k2, v2, out=o2, k_cache=kc2, v_cache=vc2)
    torch.cuda.synchronize()
    plan_split["first_prefill_ms"] = round((time.perf_counter() - t0) * 1e3, 3)
    del q2, k2, v2, o2
    sets = [tuple(to_dev(torch, x, dev) for x in W.decode_step_qkv(s + 1, Bd, N, H))
            for s in range(N_DECODE_SETS)]
    od = torch.empty((Bd, N, H, HEAD_DIM), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()
    # the process's first decode launch (wall clock)
    t0 = time.perf_counter()
    bca.decode(plan, *sets[0][:1], kc2, vc2, *sets[0][1:], out=torch.empty(
        (Bd, N, H, HEAD_DIM), dtype=torch.float32, device=dev))
    torch.cuda.synchronize()
    plan_split["first_decode_ms"] = round((time.perf_counter() - t0) * 1e3, 3)
    log(f"setup done: S={S} P={P} N={N} useful pairs/head={pairs} plan {plan_ms:.2f} ms "
        f"({plan_split})")
    # no garbage-collector pauses inside a timed loop (a host stall leaves the GPU idle between
    # launches, and that idle time would count)
    gc.collect()
    gc.disable()

    flops_pre = 4.0 * HEAD_DIM * H * pairs
    flops_dec = 4.0 * HEAD_DIM * Bd * H * N * (P + N)

    def step(i, ev=None):
        if ev is not None:
            ev[0].record()
        bca.prefill(plan, q, k, v, out=o, k_cache=kc1, v_cache=vc1)
        if ev is not None:
            ev[1].record()
        qt, kt, vt = sets[i % N_DECODE_SETS]
        bca.decode(plan, qt, kc2, vc2, kt, vt, out=od)
        if ev is not None:
            ev[2].record()

    # clock run-in (see SETTLE), then the warm-up steps
    SETTLE["main_ms"] = args.settle_ms
    SETTLE["extra_ms"] = min(SETTLE["extra_ms"], args.settle_ms)
    n_run = [0]

    def run_in_step():
        step(n_run[0])
        n_run[0] += 1
    n_settle = settle(torch, run_in_step, args.settle_ms)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record()
    for i in range(args.steps):
        step(i, evs[i])
    t_end.record()
    torch.cuda.synchronize()
    total_ms = t_start.elapsed_time(t_end)
    ms_step = total_ms / args.steps
    pre_ms = np.array([e[0].elapsed_time(e[1]) for e in evs])
    dec_ms = np.array([e[1].elapsed_time(e[2]) for e in evs])
    pre_tf = flops_pre / (pre_ms.mean() * 1e-3) / 1e12
    dec_tf = flops_dec / (dec_ms.mean() * 1e-3) / 1e12
    value = (flops_pre + flops_dec) / (ms_step * 1e-3) / 1e12
    log(f"prefill {pre_ms.mean():.3f} ms (median {np.median(pre_ms):.3f}) = {pre_tf:.1f} TFLOP/s; "
        f"decode {dec_ms.mean():.3f} ms (median {np.median(dec_ms):.3f}) = {dec_tf:.1f} TFLOP/s")

    # the dominant kernel: the call with the larger share of the step
    if dec_ms.mean() >= pre_ms.mean():
        dom, key, achieved = ("decode (bf16 cache, B=2): attn_decode_direct<0, 12> for 384-row "
                              "query tiles, then attn_decode_tail for the rest", "decode_cfg_b2",
                              dec_tf)
    else:
        dom, key, achieved = ("prefill: attn_prefill (writes the bf16 prefix cache), B=1",
                              "prefill_b1", pre_tf)
    roofline = {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                "traffic": measured_traffic(key), "kernel": dom}

    prologue = varlen = split = gen = pre_c2 = pre_c5 = cfg = dec_b1 = None
    if not args.no_extras:
        gen = decode_generation_timing(torch, bca, plan, kc2, vc2, od, Bd, N, H, flops_dec, dev)
        dec_b1 = decode_b1_timing(torch, bca, plan, kc2, vc2, sets, N, H, S, dev)
        pre_c2 = prefill_timing(torch, bca, W, "t2i_1024", dev)
        pre_c5 = prefill_timing(torch, bca, W, "long_4ref", dev)
        prologue = prologue_timings(torch, bca, W, ids, Bd, S, N, H, dev)
        varlen = varlen_timing(torch, bca, W, dev, H)
        cfg = cfg_varlen_timing(torch, bca, W, dev)
        split = split_decode_timing(torch, bca, W, dev)
    fp8 = None if args.no_fp8 else fp8_timings(torch, bca, W, plan, q, k, v, o, sets, od,
                                               flops_pre, flops_dec, Bd, S, H, P, dev)

    cpu = None
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a bounded sample ...")
        cpu = cpu_baseline(W, pre, ids, P, N, args.cpu_rows, args.cpu_heads)
        log(f"cpu oracle: {cpu['value']:.4f} TFLOP/s ({cpu['sample']})")

    line = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "settle": {"ms": args.settle_ms, "steps": n_settle},
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded N(0,1)/sqrt(128) bf16 Q/K/V)",
        "config": {
            "workload": ("2-ref 1024^2 edit: block-causal prefill S=12400 (P=8304, N=4096) B=1 "
                         "H=32 D=128 writing the prefix K/V cache, + one prefix-cached CFG decode "
                         "step B=2 N=4096 over 12400 keys"),
            "seq_len": S, "prefix_len": P, "target_len": N, "heads": H, "head_dim": HEAD_DIM,
            "prefill_batch": 1, "decode_batch": Bd, "useful_pairs_per_head": int(pairs),
        },
        "prefill": {"ms": round(float(pre_ms.mean()), 4), "ms_median": round(float(np.median(pre_ms)), 4),
                    "useful_tflops": round(pre_tf, 2), "frac_peak": round(pre_tf / PEAK_BF16_TFLOPS, 4),
                    "useful_gflop": round(flops_pre / 1e9, 1)},
        "decode": {"ms": round(float(dec_ms.mean()), 4), "ms_median": round(float(np.median(dec_ms)), 4),
                   "useful_tflops": round(dec_tf, 2), "frac_peak": round(dec_tf / PEAK_BF16_TFLOPS, 4),
                   "useful_gflop": round(flops_dec / 1e9, 1)},
        "plan_ms": round(plan_ms, 3),
        "plan_build": plan_split,
        "decode_49_steps": gen,
        "decode_b1": dec_b1,
        "prefill_t2i_1024": pre_c2,
        "prefill_long_4ref": pre_c5,
        "mfma_utilisation": mfma_utilisation(),
        "kernel_source_sha256": kernel_source_sha256(),
        "fp8_cache": fp8,
        "qk_prologue": prologue,
        "varlen_prefill": varlen,
        "cfg_varlen": cfg,
        "split_decode": split,
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)
    plan.free()


if __name__ == "__main__":
    main()
