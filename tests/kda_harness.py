"""Test harness: run one seeded workload through the HIP library and through the oracle.

Both sides receive the same stored bits: the GPU gets the workload's tensors copied to
the device; the oracle gets their exact fp64 upcasts.
"""
from __future__ import annotations

import numpy as np
import torch

import gated_delta_rule_pack_amd as kda
from gated_delta_rule_pack_amd.workloads import HEAD_DIM, Workload, to_f64
from oracle import kda_forward

OUT_TOL = 5e-3          # output rel-L2 vs the fp64 oracle
STATE_TOL_F32 = 5e-3    # final state rel-L2 with fp32 state storage
STATE_TOL_2B = 1e-2     # final state rel-L2 with fp16 / bf16 state storage


def rel_l2(x, ref) -> float:
    x = np.asarray(x, np.float64)
    ref = np.asarray(ref, np.float64)
    den = np.linalg.norm(ref)
    num = np.linalg.norm(x - ref)
    if den == 0:
        return 0.0 if num == 0 else float("inf")
    return float(num / den)


class GpuRun:
    def __init__(self, out, final_state, storage_after):
        self.out = out  # [T, H, V] fp64 numpy (bf16 values)
        self.final_state = final_state  # dense: [N, H, V, K] fp64 or None
        self.storage_after = storage_after  # paged: torch CPU tensor (flat storage) or None


def device_inputs(wl: Workload, device="cuda"):
    d = {
        "q": wl.q.to(device), "k": wl.k.to(device), "v": wl.v.to(device),
        "g_raw": wl.g_raw.to(device), "beta_raw": wl.beta_raw.to(device),
        "cu_seqlens": wl.cu_seqlens.to(device),
    }
    if wl.state_mode == "dense":
        d["initial_state"] = wl.initial_state.to(device)
    elif wl.state_mode == "paged":
        storage = wl.state_storage.to(device)
        d["storage"] = storage
        d["state_cache"] = storage.as_strided(
            (wl.num_slots, wl.H, HEAD_DIM, HEAD_DIM), (wl.state_stride0, HEAD_DIM * HEAD_DIM, HEAD_DIM, 1))
        d["state_indices"] = wl.state_indices.to(device)
        d["has_initial_state"] = wl.has_initial_state.to(device)
    return d


def run_gpu(wl: Workload, device="cuda", host_bounds=True, inputs=None, sync=True, **kw):
    d = inputs if inputs is not None else device_inputs(wl, device)
    args = dict(scale=wl.scale, lower_bound=wl.lower_bound, state_k_first=wl.state_k_first)
    if host_bounds:
        args["cu_seqlens_cpu"] = wl.cu_seqlens
    if wl.state_mode == "dense":
        args["initial_state"] = d["initial_state"]
        args["output_final_state"] = wl.want_final_state
    elif wl.state_mode == "paged":
        args["state_cache"] = d["state_cache"]
        args["state_indices"] = d["state_indices"]
        args["has_initial_state"] = d["has_initial_state"]
    args.update(kw)
    out, final = kda.chunk_fwd(d["q"], d["k"], d["v"], d["g_raw"], d["beta_raw"], d["cu_seqlens"], **args)
    if sync:
        torch.cuda.synchronize()
    out_np = to_f64(out[0])
    fin = to_f64(final) if final is not None else None
    storage_after = d["storage"].cpu() if wl.state_mode == "paged" else None
    return GpuRun(out_np, fin, storage_after)


def run_oracle(wl: Workload, seqs=None, heads=None):
    """fp64 oracle on (optionally) a subset of sequences and value heads.

    For a subset of value heads, each one's q/k head (h // (H / H_qk)) is selected here,
    so the oracle sees one q/k head per selected value head."""
    hs = slice(None) if heads is None else list(heads)
    qk_hs = slice(None) if heads is None else [h // (wl.H // wl.H_qk) for h in heads]
    q = to_f64(wl.q[0])[:, qk_hs]
    k = to_f64(wl.k[0])[:, qk_hs]
    v = to_f64(wl.v[0])[:, hs]
    g = to_f64(wl.g_raw[0])[:, hs]
    b = to_f64(wl.beta_raw[0])[:, hs]
    cu = wl.cu_seqlens.numpy()
    kw = {}
    if wl.state_mode == "dense":
        kw["initial_state"] = to_f64(wl.initial_state)[:, hs]
    elif wl.state_mode == "paged":
        kw["state_cache"] = to_f64(wl.cache_view())[:, hs]
        kw["state_indices"] = wl.state_indices.numpy()
        kw["has_initial_state"] = wl.has_initial_state.numpy()
    return kda_forward(q, k, v, g, b, cu, scale=wl.scale, lower_bound=wl.lower_bound, seqs=seqs,
                       state_k_first=wl.state_k_first, **kw)


def gpu_final_states(wl: Workload, run: GpuRun):
    """Per-sequence final states written by the GPU, as fp64 [N][H, V, K] (the stored
    layout: [N][H, K, V] for K-first planes)."""
    if wl.state_mode == "dense":
        return run.final_state
    if wl.state_mode == "paged":
        view = run.storage_after.as_strided(
            (wl.num_slots, wl.H, HEAD_DIM, HEAD_DIM), (wl.state_stride0, HEAD_DIM * HEAD_DIM, HEAD_DIM, 1))
        idx = wl.state_indices.numpy()
        return np.stack([to_f64(view[int(i)]) for i in idx])
    return None


def compare(wl: Workload, run: GpuRun, seqs=None, heads=None, out_tol=OUT_TOL, state_tol=None):
    """rel-L2 of output (valid rows) and final states against the oracle; returns both."""
    ref_out, ref_fin = run_oracle(wl, seqs=seqs, heads=heads)
    hs = slice(None) if heads is None else list(heads)
    cu = wl.cu_seqlens.numpy()
    seq_ids = range(wl.N) if seqs is None else seqs
    rows = np.concatenate([np.arange(cu[n], cu[n + 1]) for n in seq_ids]) if len(list(seq_ids)) else np.zeros(0, int)
    rows = rows.astype(int)
    got = run.out[:, hs][rows]
    ref = ref_out[rows]
    assert np.all(np.isfinite(got)), "non-finite output"
    e_out = rel_l2(got, ref)
    e_state = None
    fins = gpu_final_states(wl, run)
    if fins is not None:
        got_s = np.stack([fins[n][hs] for n in seq_ids])
        ref_s = np.stack([ref_fin[n] for n in seq_ids])
        assert np.all(np.isfinite(got_s)), "non-finite final state"
        e_state = rel_l2(got_s, ref_s)
    if state_tol is None:
        state_tol = STATE_TOL_F32 if wl.state_dtype == "f32" else STATE_TOL_2B
    if rows.size:
        assert e_out <= out_tol, f"{wl.name}: output rel-L2 {e_out:.3e} > {out_tol}"
    if e_state is not None:
        assert e_state <= state_tol, f"{wl.name}: state rel-L2 {e_state:.3e} > {state_tol}"
    return e_out, e_state


def untouched_slots_bitwise(wl: Workload, run: GpuRun):
    """Slots not referenced by state_indices and the stride padding keep their bits."""
    before = wl.state_storage.view(torch.int16 if wl.state_storage.element_size() == 2 else torch.int32)
    after = run.storage_after.view(before.dtype)
    plane = wl.H * HEAD_DIM * HEAD_DIM
    used = set(int(i) for i in wl.state_indices.tolist())
    for s in range(wl.num_slots):
        if s not in used:
            assert torch.equal(before[s], after[s]), f"unreferenced slot {s} changed"
        elif wl.state_stride0 > plane:
            assert torch.equal(before[s, plane:], after[s, plane:]), f"stride padding of slot {s} changed"
