#!/usr/bin/env python3
"""Throughput of the differential-attention forward on one MI355X.

One step = one pass of the whole forward path (lambda, the two causal
softmax maps over GQA/varlen-packed K/V, the combine, the per-head RMSNorm
and the scale: one launch of the fused kernel) over one batch of synthetic
input already resident in HBM.  The default workload is the 4096-token
causal GQA shape (B=8, N=4096, 16 differential heads, 4 KV heads, d=64 per
half, bf16).

Prints ONE JSON line.  ``value`` is TFLOP/s under the convention 12*d*H
FLOP per unmasked (query, key) pair with n^2/2 pairs per causal sequence;
``roofline`` relates the measured kernel time to MI355X's dense bf16 MFMA
peak; ``cpu_baseline`` times the fp64 oracle on the host cores on a bounded
sample of the same workload.

``--workload decode_...`` measures the key/value-cache path instead (one
step = one diffattn_fwd_kv call: the split-KV partial kernel and the
combine kernel); its ``value`` is GB/s of the bytes the step must move (q,
k, v read once, out written once) against MI355X's 8 TB/s HBM peak.
``--workload chunk_...`` is a chunked prefill through the same call, which
runs on the prefill kernel: TFLOP/s against the bf16 MFMA peak.
"""

from __future__ import annotations

import argparse
import hashlib
import importlib.util
import json
import os
import re
import sys
import time

HERE = os.path.dirname(os.path.abspath(__file__))
if HERE not in sys.path:
    sys.path.insert(0, HERE)

# MI355X dense bf16 MFMA peak: 256 CUs x 2.4 GHz x 4096 FLOP/clk/CU
# (AMD's published figure is 2.5 PFLOP/s dense; this is its unrounded form).
PEAK_BF16_TFLOPS = 256 * 2.4e9 * 4096 / 1e12
# fp32 MFMA (matrix) peak, for fp32-storage workloads.
PEAK_F32_TFLOPS = 157.3
# MI355X HBM3E peak bandwidth
PEAK_HBM_GBS = 8000.0
METRIC = "diff-attention fwd TFLOP/s & % bf16 MFMA peak, 1 MI355X, N=4096 causal"
METRIC_KV = "diff-attention KV-cache decode GB/s & % HBM peak, 1 MI355X"
METRIC_CHUNK = "diff-attention chunked prefill TFLOP/s & % bf16 MFMA peak, 1 MI355X"
GRAPH_STEPS = 10   # decode steps per captured graph (--graph)
_CSRC = os.path.join(HERE, "differential_attention_amd", "csrc")
# the sources whose kernels a stored counter profile measured: a profile
# counts only while their digest matches
KERNEL_SOURCES = [os.path.join(_CSRC, "diffattn_fwd.hip"), os.path.join(_CSRC, "rope.h"),
                  os.path.join(_CSRC, "splits.h")]
KV_KERNEL_SOURCES = [os.path.join(_CSRC, "diffattn_kv.hip"), os.path.join(_CSRC, "rope.h"),
                     os.path.join(_CSRC, "splits.h")]
CHUNK_KERNEL_SOURCES = KERNEL_SOURCES + [os.path.join(_CSRC, "diffattn_kv.hip"),
                                         os.path.join(_CSRC, "chunk.h")]
BWD_KERNEL_SOURCES = [os.path.join(_CSRC, "diffattn_fwd.hip"), os.path.join(_CSRC, "rope.h"),
                      os.path.join(_CSRC, "diffattn_bwd.hip")]


def _build_flags() -> bytes:
    """The compiler flags of the library build (they change the kernels'
    code as much as their sources do)."""
    spec = importlib.util.spec_from_file_location(
        "_diffattn_build", os.path.join(HERE, "differential_attention_amd", "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    # (without the include path, which depends on where the tree is)
    flags = " ".join(f for f in mod.HIPCC_FLAGS if not os.path.isabs(f))
    for src, extra in sorted(getattr(mod, "FILE_FLAGS", {}).items()):
        flags += f" [{src}: {' '.join(extra)}]"
    return flags.encode()


def kernel_digest(sources=KERNEL_SOURCES) -> str:
    h = hashlib.sha256()
    for p in sources:
        with open(p, "rb") as f:
            h.update(f.read())
    h.update(_build_flags())
    return h.hexdigest()[:16]


def per_launch_ms(step, stream, n: int):
    """Median, minimum and maximum of n further launches, each between two
    events recorded back to back on the launch stream (after the timed
    region, which they do not touch)."""
    import torch
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(n + 1)]
    with torch.cuda.stream(stream):
        evs[0].record(stream)
        for i in range(n):
            step()
            evs[i + 1].record(stream)
    torch.cuda.synchronize()
    t = sorted(evs[i].elapsed_time(evs[i + 1]) for i in range(n))
    return {"median": round(t[n // 2], 4), "min": round(t[0], 4), "max": round(t[-1], 4), "n": n}


def traffic_from_profiles(workload: str, sources=KERNEL_SOURCES):
    """HBM bytes per launch from the committed counter summary, if it was
    taken on the current kernel source; else None."""
    path = os.path.join(HERE, "profiles", f"hbm_traffic_{workload}.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m = re.search(r"kernel_digest:\s*([0-9a-f]+)", text)
    t = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not m or not t or m.group(1) != kernel_digest(sources):
        return None
    return float(t.group(1))


def cpu_baseline(wl, inp, flop_budget: float = 1.0e12, rope=None):
    # (with rope, rotated rows are stored in the workload's storage type)
    """The fp64 oracle on every s-th query token of the workload, all heads,
    with the stride s >= 1 chosen so that the sample holds at most
    ``flop_budget`` FLOP under the counting convention (the whole headline
    workload fits; about 6-10 s on 16 host cores)."""
    import numpy as np
    import oracle
    cu = wl.cu_seqlens().astype(np.int64)
    pos = np.concatenate([np.arange(n, dtype=np.int64) for n in wl.seqlens])
    seqlen_of = np.repeat(np.asarray(wl.seqlens, dtype=np.int64), wl.seqlens)
    pairs_per_token = (pos + 1) if wl.causal else seqlen_of
    total = 12.0 * wl.d * wl.H * float(pairs_per_token.sum())
    stride = max(1, int(np.ceil(total / flop_budget)))
    toks = np.arange(0, wl.T, stride, dtype=np.int64)
    rows_t = np.repeat(toks, wl.H)
    rows_h = np.tile(np.arange(wl.H, dtype=np.int32), toks.size)
    arrs = [oracle._f32(x) for x in (inp.q, inp.k, inp.v, inp.lq1, inp.lk1,
                                     inp.lq2, inp.lk2, inp.w)]
    lam0 = oracle.lambda_init(wl.depth)
    oracle.load()
    t0 = time.perf_counter()
    oracle.rows(*arrs[:7], lam0, rows_t, rows_h, arrs[7], wl.eps, wl.causal,
                cu.astype(np.int32), rope=rope,
                rope_round_bf16=wl.dtype == "bf16")
    dt = time.perf_counter() - t0
    flops = 12.0 * wl.d * wl.H * float(pairs_per_token[toks].sum())
    what = ("every query row of the workload" if stride == 1 else
            f"one query token in {stride} across the workload")
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s",
            "cores": oracle.max_threads(), "kind": "oracle",
            "seconds": round(dt, 3),
            "sample": (f"{what} x all {wl.H} heads ({toks.size * wl.H} output "
                       f"rows, {flops / 1e9:.1f} GFLOP under the counting "
                       "convention); fp64 C oracle, OpenMP over rows")}


def cpu_baseline_kv(wl, inp, min_seconds: float = 2.0, flops: bool = False):
    """The fp64 oracle on the cache workload, repeated until ``min_seconds``
    of host time have passed; reported in GB/s of the bytes a step must move
    (q, k, v, out in the storage type), or with ``flops`` in TFLOP/s on the
    first sequence alone (a chunk's compute, sampled)."""
    import oracle
    import workloads
    if flops:   # one sequence of the chunk workload
        wl = workloads.custom_kv(wl.name, wl.dtype, wl.q_lens[:1], wl.k_lens[:1], H=wl.H,
                                 Hkv=wl.Hkv, d=wl.d, depth=wl.depth, causal=wl.causal,
                                 eps=wl.eps)
        nq, nk = wl.Tq, wl.Tk
        inp = type(inp)(**{**inp.__dict__, "q": inp.q[:nq], "k": inp.k[:nk], "v": inp.v[:nk]})
    q, k, v = (oracle._f32(x) for x in (inp.q, inp.k, inp.v))
    lv = [oracle._f32(x) for x in (inp.lq1, inp.lk1, inp.lq2, inp.lk2)]
    w = oracle._f32(inp.w)
    cq, ck = wl.cu_q(), wl.cu_k()
    lam0 = oracle.lambda_init(wl.depth)
    oracle.load()
    runs = 0
    t0 = time.perf_counter()
    while True:
        oracle.fwd_kv(q, k, v, *lv, lam0, w, wl.eps, wl.causal, cq, ck)
        runs += 1
        dt = time.perf_counter() - t0
        if dt >= min_seconds:
            break
    if flops:
        return {"value": wl.flops() * runs / dt / 1e12, "unit": "TFLOP/s",
                "cores": oracle.max_threads(), "kind": "oracle",
                "seconds": round(dt, 3),
                "sample": (f"one sequence of the workload ({wl.Tq} queries x {wl.H} heads "
                           f"against {wl.Tk} keys, {wl.flops() / 1e9:.1f} GFLOP), {runs} "
                           "run(s); fp64 C oracle, OpenMP over output rows")}
    nbytes = wl.bytes()
    return {"value": nbytes * runs / dt / 1e9, "unit": "GB/s",
            "cores": oracle.max_threads(), "kind": "oracle",
            "seconds": round(dt, 3),
            "sample": (f"the whole workload ({wl.Tq} queries x {wl.H} heads "
                       f"against {wl.Tk} cached keys, {nbytes / 1e6:.1f} MB of "
                       f"q/k/v/out in the storage type), {runs} run(s); fp64 C "
                       "oracle, OpenMP over output rows")}


def bench_kv(args, name) -> int:
    import torch
    import workloads
    import differential_attention_amd as da

    wl = workloads.KV_WORKLOADS[name]
    inp = workloads.make_kv_inputs(wl)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    c = lambda t: t.to(dev).contiguous()
    q, k, v = c(inp.q), c(inp.k), c(inp.v)
    lv = [c(x) for x in (inp.lq1, inp.lk1, inp.lq2, inp.lk2)]
    w, cq, ck = c(inp.w), c(inp.cu_q), c(inp.cu_k)
    out = torch.empty((wl.Tq, wl.H, 2 * wl.d), dtype=q.dtype, device=dev)
    # the path the call takes: a chunk on the prefill kernel is bound by MFMA
    # throughput rather than by reading the cache (and alone needs no
    # workspace)
    path = da.kv_path(wl.nseq, wl.max_q, wl.max_k, wl.H, wl.Hkv, wl.d, Tq=wl.Tq, Tk=wl.Tk)
    chunk = path in (da.KV_PATH_PREFILL, da.KV_PATH_PREFILL_SPLIT)
    need = (0 if path == da.KV_PATH_PREFILL
            else da.kv_workspace_size(wl.nseq, wl.max_q, wl.max_k, wl.H, wl.Hkv, wl.d))
    ws = torch.empty(need, dtype=torch.uint8, device=dev)
    stream = torch.cuda.Stream(dev)
    # --rope: a rotary decode step -- the step's new keys (and values) turned
    # into the last rows of each sequence's cache, then the new queries turned
    # at their positions as they attend (tables of base 10000, fp32)
    rope_args = (0, 0, 0, 0)
    append = None
    if args.rope:
        rc, rs = (c(t) for t in workloads.rope_tables(wl.max_k, wl.d))
        gen = torch.Generator().manual_seed(2)
        k_new = c(torch.randn(wl.Tq, wl.Hkv, 2, wl.d, generator=gen).to(q.dtype))
        v_new = c(torch.randn(wl.Tq, wl.Hkv, 2 * wl.d, generator=gen).to(q.dtype))
        rope_args = (rc.data_ptr(), rs.data_ptr(), wl.max_k, da.F32)
        append = (da.BF16, k_new.data_ptr(), v_new.data_ptr(), cq.data_ptr(), ck.data_ptr(),
                  wl.nseq, wl.max_k, wl.Tq, wl.Tk, wl.Hkv, wl.d, *rope_args,
                  k.data_ptr(), v.data_ptr(), stream.cuda_stream)
    ptrs = (da.BF16, q.data_ptr(), k.data_ptr(), v.data_ptr(),
            *[x.data_ptr() for x in lv], 0, da.lambda_init(wl.depth),
            w.data_ptr(), wl.eps, int(wl.causal), cq.data_ptr(), ck.data_ptr(),
            wl.nseq, wl.max_q, wl.max_k, wl.Tq, wl.Tk, wl.H, wl.Hkv, wl.d,
            *rope_args, ws.data_ptr() if need else 0, need, out.data_ptr(), stream.cuda_stream)

    def step():
        if append is not None:
            st = da.kv_append_ptr(*append)
            if st != 0:
                raise da.DiffAttnError(st, "diffattn_kv_append")
        st = da.fwd_kv_ptr(*ptrs)
        if st != 0:
            raise da.DiffAttnError(st, "diffattn_fwd_kv")

    # --graph: the steps are replayed from a HIP graph of GRAPH_STEPS calls
    # (what a serving loop that captures its decode step pays), not launched
    # one by one from the host
    graph = None
    if args.graph:
        if args.steps % GRAPH_STEPS:
            raise SystemExit(f"--graph needs --steps divisible by {GRAPH_STEPS}")
        with torch.cuda.stream(stream):
            step()
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=stream):
            for _ in range(GRAPH_STEPS):
                step()
        torch.cuda.synchronize()

    with torch.cuda.stream(stream):
        for _ in range(args.warmup):
            step()
        torch.cuda.synchronize()
        ev0 = torch.cuda.Event(enable_timing=True)
        ev1 = torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        ev0.record(stream)
        if graph is not None:
            for _ in range(args.steps // GRAPH_STEPS):
                graph.replay()
        else:
            for _ in range(args.steps):
                step()
        ev1.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
    ms = ev0.elapsed_time(ev1) / args.steps
    nbytes = wl.bytes()
    gbs = nbytes / (ms * 1e-3) / 1e9
    tflops = wl.flops() / (ms * 1e-3) / 1e12
    result = {
        "metric": METRIC_CHUNK if chunk else METRIC_KV,
        "value": round(tflops, 2) if chunk else round(gbs, 1),
        "unit": "TFLOP/s" if chunk else "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic (seeded N(0,1) q/k/v, N(0,0.1^2) lambda vectors)",
        "config": {"workload": name + ("+rope" if args.rope else ""), "rope": bool(args.rope),
                   "nseq": wl.nseq, "Tq": wl.Tq, "Tk": wl.Tk,
                   "max_q": wl.max_q, "max_k": wl.max_k, "H": wl.H,
                   "Hkv": wl.Hkv, "d": wl.d, "depth": wl.depth,
                   "causal": wl.causal, "bytes_per_step": nbytes,
                   "tokens_per_s": round(wl.Tq / (ms * 1e-3), 1),
                   "tflops": round(tflops, 2), "gb_per_s": round(gbs, 1),
                   "path": {da.KV_PATH_SPLIT_KV: "split-KV + combine",
                            da.KV_PATH_PREFILL: "prefill kernel",
                            da.KV_PATH_PREFILL_SPLIT: "prefill kernel on key splits + combine"}[path],
                   "workspace_bytes": need,
                   "launch": f"hip graph of {GRAPH_STEPS} steps" if graph is not None else "eager",
                   "wall_s_timed": round(wall, 4),
                   "ms_per_launch": per_launch_ms(step, stream, args.steps) if graph is None else None,
                   "kernel_digest": kernel_digest(KV_KERNEL_SOURCES)},
        # split path: both kernels of the step are in the timed duration, so
        # this is a lower bound on the partial kernel's own rate
        "roofline": ({"bound": "mfma", "achieved": round(tflops, 2),
                      "peak": round(PEAK_BF16_TFLOPS, 1), "unit": "TFLOP/s",
                      "frac": round(tflops / PEAK_BF16_TFLOPS, 4)} if chunk else
                     {"bound": "hbm", "achieved": round(gbs, 1),
                      "peak": PEAK_HBM_GBS, "unit": "GB/s",
                      "frac": round(gbs / PEAK_HBM_GBS, 4)}),
    }
    result["roofline"]["traffic"] = traffic_from_profiles(
        name + ("_rope" if args.rope else ""), CHUNK_KERNEL_SOURCES if chunk else KV_KERNEL_SOURCES)
    result["config"]["kernel_digest"] = kernel_digest(CHUNK_KERNEL_SOURCES if chunk
                                                      else KV_KERNEL_SOURCES)
    result["cpu_baseline"] = (None if args.no_cpu_baseline
                              else None if args.rope  # (the oracle's cache path takes rotated q)
                              else cpu_baseline_kv(wl, inp, flops=chunk))
    print(json.dumps(result), flush=True)
    return 0


METRIC_BWD = "diff-attention fwd+bwd (training step) TFLOP/s & % bf16 MFMA peak, 1 MI355X"


def bench_bwd(args, name) -> int:
    """One step = diffattn_fwd_train + diffattn_bwd on resident inputs."""
    import torch
    import workloads
    import differential_attention_amd as da

    wl = workloads.WORKLOADS[name]
    inp = workloads.make_inputs(wl)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    c = lambda t: t.to(dev).contiguous()
    q, k, v = c(inp.q), c(inp.k), c(inp.v)
    lv = [c(x) for x in (inp.lq1, inp.lk1, inp.lq2, inp.lk2)]
    w, cu = c(inp.w), c(inp.cu_seqlens)
    gen = torch.Generator().manual_seed(1)
    dout = c(torch.randn(wl.T, wl.H, 2 * wl.d, generator=gen).to(q.dtype))
    out = torch.empty_like(dout)
    lse = torch.empty(wl.T, wl.H, 2, dtype=torch.float32, device=dev)
    o12 = torch.empty(wl.T, wl.H, 2, 2 * wl.d, dtype=torch.float32, device=dev)
    grads = [torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)] + \
            [torch.empty_like(x) for x in lv] + [torch.empty(2 * wl.d, device=dev)]
    need = da.bwd_workspace_size(torch.bfloat16, wl.T, wl.H, wl.d)
    ws = torch.empty(need, dtype=torch.uint8, device=dev)
    stream = torch.cuda.Stream(dev)
    lam0 = da.lambda_init(wl.depth)
    lib = da.library()
    common = (da.BF16, q.data_ptr(), k.data_ptr(), v.data_ptr(),
              *[x.data_ptr() for x in lv], 0, lam0, w.data_ptr(), wl.eps,
              int(wl.causal), cu.data_ptr(), wl.nseq, wl.max_seqlen, wl.T, wl.H,
              wl.Hkv, wl.d)

    def step():
        st = lib.diffattn_fwd_train(*common, out.data_ptr(), lse.data_ptr(),
                                    o12.data_ptr(), stream.cuda_stream)
        if st != 0:
            raise da.DiffAttnError(st, "diffattn_fwd_train")
        st = lib.diffattn_bwd(*common, dout.data_ptr(), lse.data_ptr(), o12.data_ptr(),
                              *[g.data_ptr() for g in grads], ws.data_ptr(), need,
                              stream.cuda_stream)
        if st != 0:
            raise da.DiffAttnError(st, "diffattn_bwd")

    with torch.cuda.stream(stream):
        for _ in range(args.warmup):
            step()
        torch.cuda.synchronize()
        ev0 = torch.cuda.Event(enable_timing=True)
        ev1 = torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        ev0.record(stream)
        for _ in range(args.steps):
            step()
        ev1.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
    ms = ev0.elapsed_time(ev1) / args.steps
    fwd_flops = wl.flops()
    bwd_flops = fwd_flops * 28.0 / 12.0
    tflops = (fwd_flops + bwd_flops) / (ms * 1e-3) / 1e12
    result = {
        "metric": METRIC_BWD,
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic (seeded N(0,1) q/k/v/dout, N(0,0.1^2) lambda vectors)",
        "config": {"workload": name + "+bwd", "T": wl.T, "nseq": wl.nseq,
                   "H": wl.H, "Hkv": wl.Hkv, "d": wl.d, "causal": wl.causal,
                   "flops_fwd": fwd_flops, "flops_bwd": bwd_flops,
                   "workspace_bytes": need,
                   "launch": "eager", "wall_s_timed": round(wall, 4),
                   "ms_per_launch": per_launch_ms(step, stream, args.steps),
                   "kernel_digest": kernel_digest(BWD_KERNEL_SOURCES)},
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2),
                     "peak": round(PEAK_BF16_TFLOPS, 1), "unit": "TFLOP/s",
                     "frac": round(tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": traffic_from_profiles(name + "_bwd", BWD_KERNEL_SOURCES)},
        "cpu_baseline": None,
    }
    print(json.dumps(result), flush=True)
    return 0


def copy_calibration(args) -> int:
    """A plain device-to-device copy of known size, for scaling the HBM byte
    counters (FETCH_SIZE, WRITE_SIZE) of the kernel under a profiler."""
    import torch
    dev = torch.device("cuda:0")
    a = torch.ones(args.copy_bytes, dtype=torch.uint8, device=dev)
    b = torch.empty_like(a)
    for _ in range(args.warmup):
        b.copy_(a)
    torch.cuda.synchronize()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    ev0.record()
    for _ in range(args.steps):
        b.copy_(a)
    ev1.record()
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / args.steps
    print(json.dumps({"copy_bytes": args.copy_bytes, "ms_per_copy": round(ms, 4),
                      "GB_per_s_read_plus_write": round(2 * args.copy_bytes / ms / 1e6, 1)}),
          flush=True)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--graph", action="store_true",
                    help="cache workloads: replay the timed steps from a HIP graph")
    ap.add_argument("--bwd", action="store_true",
                    help="a training step instead: the training forward and "
                         "the backward pass (bf16, no rotary prologue)")
    ap.add_argument("--rope", action="store_true",
                    help="prefill with the fused rotary prologue (q and k "
                         "given unrotated, tables of base 10000); with a cache "
                         "workload, a rotary decode step (the new keys turned "
                         "into the cache, then the new queries turned)")
    ap.add_argument("--copy-bytes", type=int, default=0,
                    help="instead of the workload, time a plain device copy of "
                         "this many bytes (calibrates HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: this build measures one GPU only (the forward kernel "
              "on one GPU's share); --gpus above 1 is not supported",
              file=sys.stderr)
        return 2

    import torch
    if args.copy_bytes > 0:
        return copy_calibration(args)
    import workloads
    import differential_attention_amd as da

    name = args.workload or workloads.HEADLINE
    if name in workloads.KV_WORKLOADS:
        return bench_kv(args, name)
    if args.bwd:
        return bench_bwd(args, name)
    wl = workloads.WORKLOADS[name]
    inp = workloads.make_inputs(wl)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    c = lambda t: t.to(dev).contiguous()
    q, k, v = c(inp.q), c(inp.k), c(inp.v)
    lv = [c(x) for x in (inp.lq1, inp.lk1, inp.lq2, inp.lk2)]
    w = c(inp.w)
    cu = c(inp.cu_seqlens)
    out = torch.empty((wl.T, wl.H, 2 * wl.d), dtype=q.dtype, device=dev)
    lam0 = da.lambda_init(wl.depth)
    stream = torch.cuda.Stream(dev)
    dtype_code = da.BF16 if wl.dtype == "bf16" else da.F32
    rope_args = (0, 0, 0, 0, 0, 0)
    if args.rope:
        rc, rs = (c(t) for t in workloads.rope_tables(wl.max_seqlen, wl.d))
        need = da.fwd_workspace_size(q.dtype, wl.T, wl.Hkv, wl.d, True)
        rws = torch.empty(need, dtype=torch.uint8, device=dev)
        rope_args = (rc.data_ptr(), rs.data_ptr(), wl.max_seqlen, da.F32, rws.data_ptr(), need)
    ptrs = (dtype_code, q.data_ptr(), k.data_ptr(), v.data_ptr(),
            *[x.data_ptr() for x in lv], 0, lam0, w.data_ptr(), wl.eps,
            int(wl.causal), cu.data_ptr(), wl.nseq, wl.max_seqlen, wl.T, wl.H,
            wl.Hkv, wl.d, *rope_args, out.data_ptr(), stream.cuda_stream)

    def step():
        st = da.fwd_ptr(*ptrs)
        if st != 0:
            raise da.DiffAttnError(st, "diffattn_fwd")

    with torch.cuda.stream(stream):
        for _ in range(args.warmup):
            step()
        torch.cuda.synchronize()
        ev0 = torch.cuda.Event(enable_timing=True)
        ev1 = torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        ev0.record(stream)
        for _ in range(args.steps):
            step()
        ev1.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
    ms = ev0.elapsed_time(ev1) / args.steps
    flops = wl.flops()
    tflops = flops / (ms * 1e-3) / 1e12
    peak = PEAK_BF16_TFLOPS if wl.dtype == "bf16" else PEAK_F32_TFLOPS
    # (the rotary path runs another instantiation plus the K rotation: its own
    # profile, if one was taken)
    traffic = traffic_from_profiles(name + ("_rope" if args.rope else ""))

    result = {
        "metric": METRIC,
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic (seeded N(0,1) q/k/v, N(0,0.1^2) lambda vectors)",
        "config": {"workload": name + ("+rope" if args.rope else ""),
                   "T": wl.T, "nseq": wl.nseq, "rope": bool(args.rope),
                   "max_seqlen": wl.max_seqlen, "H": wl.H, "Hkv": wl.Hkv,
                   "d": wl.d, "depth": wl.depth, "causal": wl.causal,
                   "flops_per_step": flops,
                   "pct_of_bf16_peak": round(100 * tflops / peak, 2),
                   "wall_s_timed": round(wall, 4),
                   "ms_per_launch": per_launch_ms(step, stream, args.steps),
                   "kernel_digest": kernel_digest()},
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2),
                     "peak": round(peak, 1), "unit": "TFLOP/s",
                     "frac": round(tflops / peak, 4), "traffic": traffic},
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(
            wl, inp, rope=workloads.rope_tables(wl.max_seqlen, wl.d) if args.rope else None)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
