#!/usr/bin/env python3
"""Benchmark chunkwise KDA prefill on one MI355X.

One step = one ``kda_chunk_fwd`` call (metadata lookup, prep kernel, scan kernel; or the
decode kernel alone when no sequence has more than one token) over one batch of
synthetic input already resident in HBM. The default workload is the
1 x 4096-token, 12-head call with a paged fp32 state pool (the per-GPU Kimi-K3 serving
shape); ``--workload`` selects the other shapes. The default run also times the
1 x 16384-token call and both shapes with every call building and uploading its
metadata, each with its own roofline, under ``extra_workloads``.

Prints ONE JSON line with the throughput (tokens/s) and per-call latency of the K timed
calls, the roofline of the dominant kernel and the fp64 oracle timed on the host cores.
Kernel durations come from a second pass of the same K calls with timing events that
the library attaches to each kernel launch on the call's stream (start and end of the
kernel itself); the timed pass carries no per-kernel events.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "KDA prefill µs/call + tokens/s, H=12 1×4K/1×16K; % of MFMA/HBM peak"
HBM_PEAK_GBS = 8000.0  # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak
RECORD_BYTES = 35328  # per (head, chunk) workspace record written by prep, read by scan

HEADLINE = "paged_1x4096_H12"
EXTRA_16K = "paged_1x16384_H12_pad"

WORKLOADS = {
    "paged_1x4096_H12": "1x4096 tokens, H=12, K=V=128, paged fp32 state pool [64,12,128,128]",
    "paged_1x16384_H12_pad": "1x16384 tokens, H=12, K=V=128, paged fp32 pool with stride(0) padded by 4096",
    "paged_1x16384_H12_pad_lb20": "1x16384 tokens, H=12, steep gate (lower bound -20, raw gate +6: ~640 nats per chunk), "
                                  "paged fp32 pool with stride(0) padded by 4096",
    "paged_varlen128_H12": "128 varlen sequences (0..2048 tokens, 4 empty), H=12, paged fp32 pool [256,...]",
    "paged_256x1_H12_bf16": "256 sequences x 1 token, H=12, paged bf16 pool [512,12,128,128]",
    "paged_256x1_H12_f16": "256 sequences x 1 token, H=12, paged fp16 pool [512,12,128,128]",
    "paged_64x1_H12_f16": "64 sequences x 1 token (one decode step), H=12, paged fp16 pool [128,12,128,128]",
    "paged_64x1_H12_f32": "64 sequences x 1 token (one decode step), H=12, paged fp32 pool [128,12,128,128]",
    "paged_256x1_H12_bf16_kfirst": "256 sequences x 1 token, H=12, paged bf16 pool with K-first planes [512,12,128,128]",
    "paged_1x4096_H12_qk6": "1x4096 tokens, 12 value heads sharing 6 q/k heads, paged fp32 pool [64,12,128,128]",
}


def _oracle_head(args):
    # Worker: the oracle on one head of the workload (heads are independent).
    from oracle import kda_forward
    q, k, v, g, b, cu, scale, lb, S = args
    return kda_forward(q, k, v, g, b, cu, scale=scale, lower_bound=lb, **S)


def cpu_baseline(wl, max_tokens: int, workers: int, min_seconds: float):
    """Time the fp64 oracle on a bounded sample of the workload (before any GPU use).

    The sample is repeated until at least ``min_seconds`` of wall time have passed, so a
    small workload still gives a stable rate."""
    import multiprocessing as mp

    import numpy as np
    from threadpoolctl import threadpool_limits

    from gated_delta_rule_pack_amd.workloads import to_f64

    cu = wl.cu_seqlens.numpy().astype(np.int64)
    # Sample: whole sequences in order until max_tokens.
    take = 1
    while take < wl.N and cu[take + 1] <= max_tokens:
        take += 1
    t_end = int(min(cu[take], max_tokens))
    cu_s = np.minimum(cu[: take + 1], t_end)
    q = to_f64(wl.q[0, :t_end]); k = to_f64(wl.k[0, :t_end]); v = to_f64(wl.v[0, :t_end])
    g = to_f64(wl.g_raw[0, :t_end]); b = to_f64(wl.beta_raw[0, :t_end])
    tasks = []
    for h in range(wl.H):
        hq = h // (wl.H // wl.H_qk)  # the q/k head this value head reads
        S = {"state_k_first": wl.state_k_first}
        if wl.state_mode == "paged":
            S = dict(state_cache=to_f64(wl.cache_view()[:, h:h + 1]), state_indices=wl.state_indices.numpy()[:take],
                     has_initial_state=wl.has_initial_state.numpy()[:take])
        elif wl.state_mode == "dense":
            S = dict(initial_state=to_f64(wl.initial_state[:take, h:h + 1]))
        tasks.append((q[:, hq:hq + 1], k[:, hq:hq + 1], v[:, h:h + 1], g[:, h:h + 1], b[:, h:h + 1], cu_s,
                      wl.scale, wl.lower_bound, S))
    workers = max(1, workers)
    # One head per task; with more workers than heads the heads repeat, so that every
    # worker has one task per pass and all of them run at once.
    run = [tasks[i % len(tasks)] for i in range(max(workers, len(tasks)))]
    with threadpool_limits(1):
        ctx = mp.get_context("fork")
        with ctx.Pool(workers) as pool:
            pool.map(abs, range(workers))  # start the workers before timing
            reps = 0
            t0 = time.perf_counter()
            while True:
                pool.map(_oracle_head, run, chunksize=1)
                reps += 1
                wall = time.perf_counter() - t0
                if wall >= min_seconds:
                    break
        # One core: one head in this process, repeated for a quarter of the time; the
        # rate scales by the number of heads.
        reps1 = 0
        t1 = time.perf_counter()
        while True:
            _oracle_head(tasks[0])
            reps1 += 1
            wall1 = time.perf_counter() - t1
            if wall1 >= min_seconds / 4:
                break
    tokens = int(cu_s[-1])
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            model = next((l.split(":", 1)[1].strip() for l in f if l.startswith("model name")), "")
    except OSError:
        pass
    return {
        "value": reps * tokens * len(run) / (wall * wl.H), "unit": "tokens/s", "cores": workers, "kind": "oracle",
        "sample": f"first {tokens} tokens ({take} sequence(s)) of the workload, {len(run)} head tasks per pass "
                  f"(the {wl.H} heads, repeated to give each of {workers} worker processes one), fp64 numpy "
                  f"token loop, {reps} pass(es); tokens/s counts {wl.H} head-tasks as one token",
        "seconds": wall,
        "value_1core": reps1 * tokens / (wall1 * wl.H), "cpu_model": model, "nproc": os.cpu_count(),
    }


def kernel_source_hash(kernel: str) -> str:
    """Hash of the sources one kernel is built from (its .hip file and the shared headers)."""
    csrc = os.path.join(ROOT, "gated_delta_rule_pack_amd", "csrc")
    h = hashlib.sha256()
    for name in (f"kda_{kernel}.hip", "kda_device.h", "kda_internal.h"):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_from_profiles(kernel: str, workload: str):
    """HBM bytes per launch from the committed counter summary, if its kernel source matches."""
    path = os.path.join(ROOT, "profiles", f"kda_{kernel}_traffic_{workload}.txt")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_hash = re.search(r"source_sha256_16:\s*([0-9a-f]+)", text)
    m_bytes = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not m_hash or not m_bytes or m_hash.group(1) != kernel_source_hash(kernel):
        return None
    return float(m_bytes.group(1))


KERNEL_BYTES_BASIS = {
    "prep": "reads q, k, v, raw gate and raw beta per valid token-head; writes one 35328-byte record per chunk-head",
    "scan": "reads one 35328-byte prep record per chunk-head; writes 256 B of output per token-head; reads "
            "(flagged) and writes one V x K state per sequence-head (segment maps and start states of a "
            "segmented call not counted)",
    "decode": "the method's own bytes: q, k, v, raw gate, raw beta and out per token-head, state read and write",
}


def kernel_bytes(wl, kernel: str, n_chunks: int):
    """Per-launch bytes one kernel must move in this design (per-unit figures stated in the
    design notes), or the method's own bytes for ``call``.

    prep: reads q, k, v (3 x 256 B), raw gate (512 B fp32 / 256 B bf16) and raw beta
          (4 / 2 B) per valid token-head; writes one 35328-byte record per chunk-head.
    scan: reads each chunk-head record once; writes 256 B of output per token-head;
          reads (when the flag is set) and writes one V x K state per sequence-head.
    decode: the one-token kernel moves exactly the method's own bytes (as ``call``).
    call: the method's own (algorithmic) bytes: q, k, v, raw gate, raw beta, out per
          token-head plus the state read/write, no intermediates.
    """
    th = wl.T * wl.H
    qk_b = 2 * 256 * wl.H_qk // wl.H  # q and k bytes per token-head (grouped heads share them)
    g_b = wl.g_raw.element_size() * 128
    b_b = wl.beta_raw.element_size()
    s_b = {"f32": 4, "f16": 2, "bf16": 2}[wl.state_dtype] * 128 * 128
    n_read = wl.N if wl.state_mode != "paged" else int(wl.has_initial_state.sum())
    if wl.state_mode == "none":
        n_read = 0
    n_write = wl.N if wl.state_mode in ("paged", "dense") else 0
    state = (n_read + n_write) * wl.H * s_b
    if kernel == "prep":
        return th * (qk_b + 256 + g_b + b_b) + n_chunks * wl.H * RECORD_BYTES
    if kernel == "scan":
        return n_chunks * wl.H * RECORD_BYTES + th * 256 + state
    return th * (qk_b + 256 + g_b + b_b + 256) + state


def algorithmic_flops(wl, kernel: str):
    """Per-launch algorithmic flops of one kernel (per token-head figures at C = 32, K = V = 128).

    prep: the four chunk-local products A, P, W and U, 2 x 32 x 128 each per token-head.
    scan: W S^T, Q~ S^T and Delta^T K^ (2 x 128 x 128 each) plus P Delta (2 x 32 x 128).
    decode: the token recurrence itself: decay, S k^, the rank-one update and S q^, 7 x 128 x 128.
    call: prep + scan, or decode.
    """
    th = wl.T * wl.H
    per = {"prep": 4 * 2 * 32 * 128, "scan": 3 * 2 * 128 * 128 + 2 * 32 * 128, "decode": 7 * 128 * 128}
    per["call"] = per["prep"] + per["scan"]
    return th * per[kernel]


def attainable_peaks(dev):
    """Live attainable peaks on this part: a plain 512 MiB device copy and a bf16 GEMM loop."""
    import torch

    def timed(fn, reps):
        fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps * 1e-3

    src = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    t_copy = timed(lambda: dst.copy_(src), 10)
    del src, dst
    n = 8192
    x = torch.randn(n, n, device=dev, dtype=torch.bfloat16)
    y = torch.randn(n, n, device=dev, dtype=torch.bfloat16)
    t_gemm = timed(lambda: torch.mm(x, y), 10)
    return {"copy_GBps": round(2 * (512 << 20) / t_copy / 1e9, 1),
            "gemm_bf16_TFLOPs": round(2 * n ** 3 / t_gemm / 1e12, 1),
            "how": "512 MiB device-to-device copy; 8192^3 bf16 torch.mm (hipBLASLt), 10 reps each"}


def copy_calibration(mib: int, steps: int, warmup: int):
    """Plain device-to-device copies of a known size, for scaling the HBM byte counters."""
    import torch

    dev = torch.device("cuda", 0)
    n = mib << 18  # fp32 elements
    src = torch.rand(n, device=dev)
    dst = torch.empty_like(src)
    for _ in range(warmup):
        dst.copy_(src)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    nbytes = n * 4
    print(json.dumps({"copy_bytes_read": nbytes, "copy_bytes_written": nbytes, "steps": steps,
                      "us_per_copy": round(ms * 1e3, 2), "GBps": round(2 * nbytes / (ms * 1e-3) / 1e9, 1),
                      "equal": bool(torch.equal(src, dst))}), flush=True)


def _context_with(env: dict):
    """A new library context created with these environment knobs set (read once, at creation)."""
    import gated_delta_rule_pack_amd as kda
    old = {k: os.environ.get(k) for k in env}
    os.environ.update({k: str(v) for k, v in env.items()})
    try:
        return kda.Context(0)
    finally:
        for k, v in old.items():
            if v is None:
                del os.environ[k]
            else:
                os.environ[k] = v


def measure(name: str, steps: int, warmup: int, rotate: int = 0, rotate_bounds: int = 0, ctx=None):
    """Time ``steps`` calls of one workload (inputs resident in HBM, rotated over input sets
    larger than the 256 MB MALL) and, in a second pass, each kernel's own duration.

    Returns the fields of one bench record: throughput, latency, per-kernel times and the
    roofline of the dominant kernel."""
    import torch

    import gated_delta_rule_pack_amd as kda
    from gated_delta_rule_pack_amd import _lib
    from gated_delta_rule_pack_amd.workloads import standard

    wl = standard(name)
    dev = torch.device("cuda", 0)
    lib = _lib.load()
    ctx = ctx if ctx is not None else kda.get_context(dev)
    stream = torch.cuda.current_stream(dev)

    # Input sets resident in HBM, rotated so the caches cannot hold them between steps.
    # Each set has its own state pool: the state a call reads and writes (one V x K
    # block per sequence and head) counts toward the set's footprint.
    s_elem = {"f32": 4, "f16": 2, "bf16": 2}[wl.state_dtype]
    per_set = sum(t.numel() * t.element_size() for t in (wl.q, wl.k, wl.v, wl.g_raw, wl.beta_raw)) + \
        wl.v.numel() * 2 + (2 * wl.N * wl.H * 128 * 128 * s_elem if wl.state_mode == "paged" else 0)
    n_rot = rotate or max(1, min(8, (512 << 20) // per_set + 1))
    base = {n: getattr(wl, n).to(dev) for n in ("q", "k", "v", "g_raw", "beta_raw")}
    cu_d = wl.cu_seqlens.to(dev)
    cu_h = wl.cu_seqlens.clone()
    pools = [{}]
    if wl.state_mode == "paged":
        idx_d, flag_d = wl.state_indices.to(dev), wl.has_initial_state.to(dev)
        pools = []
        for _ in range(n_rot):
            storage = wl.state_storage.to(dev)
            pools.append(dict(state_cache=storage.as_strided((wl.num_slots, wl.H, 128, 128),
                                                             (wl.state_stride0, 128 * 128, 128, 1)),
                              state_indices=idx_d, has_initial_state=flag_d))
    # Bounds sets: the workload's own, or (rotate_bounds K) K seeded permutations of its
    # sequence lengths, so that every call misses the metadata cache (64 entries).
    bounds = [(cu_d, cu_h)]
    if rotate_bounds:
        gen = torch.Generator().manual_seed(7)
        lens = wl.cu_seqlens[1:] - wl.cu_seqlens[:-1]
        bounds = []
        for _ in range(rotate_bounds):
            perm = lens[torch.randperm(wl.N, generator=gen)]
            h_cu = torch.cat([torch.zeros(1, dtype=torch.int32), torch.cumsum(perm, 0).to(torch.int32)])
            bounds.append((h_cu.to(dev), h_cu))
    inputs = []
    for i in range(n_rot):
        s = {n: (t if i == 0 else t.clone()) for n, t in base.items()}
        s["out"] = torch.empty_like(s["v"])
        inputs.append(s)
    sets = []  # (inputs, args, bounds tensors kept alive)
    for i in range(max(n_rot, len(bounds))):
        s = inputs[i % n_rot]
        b_d, b_h = bounds[i % len(bounds)]
        a = kda.make_args(s["q"], s["k"], s["v"], s["g_raw"], s["beta_raw"], b_d, cu_seqlens_cpu=b_h,
                          scale=wl.scale, lower_bound=wl.lower_bound, out=s["out"], state_k_first=wl.state_k_first,
                          **pools[i % len(pools)])
        rc = lib.kda_chunk_fwd_validate(ctypes.byref(a))
        if rc != _lib.KDA_OK:
            raise kda.KDAError(rc, "validate")
        sets.append((s, a, (b_d, b_h)))
    n_rot = len(sets)
    ws_bytes = kda.workspace_bytes(sets[0][1])
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    ws_p, st_p = ws.data_ptr(), stream.cuda_stream

    def step(i):
        rc = ctx.forward(sets[i % n_rot][1], ws_p, ws_bytes, st_p)
        if rc != _lib.KDA_OK:
            raise kda.KDAError(rc, "kda_chunk_fwd")

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    ctx.reset_stats()
    # Timed region: the K calls alone, bracketed by events on the call stream.
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    t0 = time.perf_counter()
    for i in range(steps):
        step(i)
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    stats = ctx.stats()
    # Kernel durations: the same K calls again, with the library's timing events attached
    # to each kernel launch (start and end of the kernel itself, on the call stream).
    ctx.profile(True)
    for i in range(steps):
        step(i)
    torch.cuda.synchronize()
    ctx.profile(False)
    per_call = sorted(ctx.profile_calls(steps))
    prep_ms, scan_ms, ncalls = ctx.profile_read()
    pct = lambda f: 1e3 * per_call[min(len(per_call) - 1, int(f * len(per_call)))]
    ms_step = e0.elapsed_time(e1) / steps
    value = wl.T / (ms_step * 1e-3)

    n_chunks = int(stats["last_n_chunks"])
    if stats["last_path"] == 1:  # one-token call: the decode kernel alone
        k_us = {"decode": 1e3 * scan_ms / max(ncalls, 1)}
    else:
        k_us = {"prep": 1e3 * prep_ms / max(ncalls, 1), "scan": 1e3 * scan_ms / max(ncalls, 1)}
    dom = max(k_us, key=k_us.get)
    kb = kernel_bytes(wl, dom, n_chunks)
    achieved = kb / (k_us[dom] * 1e-6) / 1e9
    traffic = traffic_from_profiles(dom, name)
    call_bytes = kernel_bytes(wl, "call", n_chunks)
    flops = algorithmic_flops(wl, dom)
    call_flops = algorithmic_flops(wl, "decode" if dom == "decode" else "call")
    segmented = dom == "scan" and stats["last_seg_len"] > 0
    roofline = {
        "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
        "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
        "kernel": f"kda_{dom}" + (" phase: segment maps, segment combine, scan" if segmented else ""),
        "kernel_us": round(k_us[dom], 2),
        # The bytes this kernel must move in the two-kernel design (the per-kernel accounting:
        # for the scan, the prep records it reads, its output and the state), which is what
        # `achieved` and `frac` use.
        "kernel_bytes": int(kb),
        "kernel_bytes_basis": KERNEL_BYTES_BASIS[dom],
        # The method's own bytes (q, k, v, raw gate, raw beta and out per token-head plus the
        # state read and write, no intermediates), against the whole call's time.
        "call_algorithmic_bytes": int(call_bytes),
        "call_frac": round(call_bytes / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "kernel_tflops": round(flops / (k_us[dom] * 1e-6) / 1e12, 2),
        "kernel_mfma_frac": round(flops / (k_us[dom] * 1e-6) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
        "call_tflops": round(call_flops / (ms_step * 1e-3) / 1e12, 2),
        "call_mfma_frac": round(call_flops / (ms_step * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
    }
    config = {"workload": name, "description": WORKLOADS[name], "T": wl.T, "N": wl.N, "H": wl.H,
              "H_qk": wl.H_qk, "K": 128, "V": 128, "chunk": 32, "state_k_first": wl.state_k_first,
              "lower_bound": wl.lower_bound, "state": f"{wl.state_mode} {wl.state_dtype}",
              "dv_split": stats["last_dv_split"], "ref_block": stats["last_ref_block"],
              "segment_length": stats["last_seg_len"], "input_sets_rotated": n_rot,
              "bounds_sets": max(1, rotate_bounds), "parallelism": "single GPU"}
    return {
        "value": round(value, 1), "unit": "tokens/s", "ms_per_step": round(ms_step, 5),
        "us_per_call": round(ms_step * 1e3, 2), "steps": steps, "warmup": warmup, "config": config,
        "kernels_us": {k: round(v, 2) for k, v in k_us.items()},
        # Per-call latency from the kernels' own timestamps (first kernel start to scan
        # end), over the profiled pass.
        "call_us_p10_p50_p90": [round(pct(0.1), 2), round(pct(0.5), 2), round(pct(0.9), 2)],
        "host_wall_us_per_call": round(wall / steps * 1e6, 2),
        "metadata": {"cache_hits": stats["cache_hits"], "cache_misses": stats["cache_misses"],
                     "blocking_syncs": stats["blocking_syncs"], "arena_grows": stats["arena_grows"]},
        "roofline": roofline,
    }


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", choices=sorted(WORKLOADS), default=HEADLINE)
    ap.add_argument("--rotate", type=int, default=0,
                    help="input sets cycled through (0: enough to exceed the 256 MB MALL)")
    ap.add_argument("--rotate-bounds", type=int, default=0,
                    help="cycle through this many permutations of the sequence lengths (metadata-cache "
                         "miss mode: every call uploads its metadata)")
    ap.add_argument("--no-extra", action="store_true",
                    help="time only --workload (by default the headline run also times the 1x16384 shape, "
                         "and both headline shapes with every call missing the metadata cache)")
    ap.add_argument("--cpu-tokens", type=int, default=4096, help="oracle sample size (tokens)")
    ap.add_argument("--cpu-workers", type=int, default=0, help="oracle worker processes (0: all host cores, at most 16)")
    ap.add_argument("--cpu-seconds", type=float, default=2.0, help="minimum oracle wall time")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="instead of the workload, run --steps plain device copies of this many MiB "
                         "(the known-size kernel that scales the HBM byte counters)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}, WORLD_SIZE {world}); "
              "the KDA path here is single-GPU: heads and sequences shard without communication, "
              "so per-GPU throughput is the number to read.", file=sys.stderr)
        sys.exit(2)

    if args.copy_mib:
        copy_calibration(args.copy_mib, args.steps, args.warmup)
        return

    from gated_delta_rule_pack_amd.workloads import standard

    # Oracle baseline on the host first, before anything initialises the GPU.
    cpu = None
    if not args.no_cpu_baseline:
        workers = args.cpu_workers or min(16, os.cpu_count() or 1)
        cpu = cpu_baseline(standard(args.workload), args.cpu_tokens, workers, args.cpu_seconds)

    import torch
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    rec = measure(args.workload, args.steps, args.warmup, args.rotate, args.rotate_bounds)
    rec["roofline"]["attainable"] = attainable_peaks(dev)
    extra = None
    if args.workload == HEADLINE and not args.no_extra and not args.rotate_bounds:
        # The second headline shape, and both shapes with every call building and uploading
        # its metadata (a context whose metadata cache is off, as with new bounds each call).
        extra = {}
        for key, name, env in ((EXTRA_16K, EXTRA_16K, None), (HEADLINE + "_meta_miss", HEADLINE, {"KDA_META_CACHE": 0}),
                               (EXTRA_16K + "_meta_miss", EXTRA_16K, {"KDA_META_CACHE": 0})):
            ctx = _context_with(env) if env else None
            extra[key] = measure(name, args.steps, args.warmup, args.rotate, ctx=ctx)
            if env:
                extra[key]["config"]["metadata"] = "every call builds and uploads its metadata (KDA_META_CACHE=0)"
                ctx.close()
    line = {
        "metric": METRIC, "value": rec["value"], "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": rec["ms_per_step"],
        "us_per_call": rec["us_per_call"], "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": rec["config"], "kernels_us": rec["kernels_us"],
        "call_us_p10_p50_p90": rec["call_us_p10_p50_p90"], "host_wall_us_per_call": rec["host_wall_us_per_call"],
        "metadata": rec["metadata"], "roofline": rec["roofline"], "cpu_baseline": cpu,
    }
    if extra is not None:
        line["extra_workloads"] = {
            k: {f: v[f] for f in ("value", "unit", "us_per_call", "ms_per_step", "kernels_us", "call_us_p10_p50_p90",
                                  "metadata", "roofline", "config")} for k, v in extra.items()}
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
