"""Seeded synthetic workloads for chunkwise KDA prefill.

This module only draws inputs; it holds none of the method's arithmetic. Both the
HIP path (through the C-ABI binding) and the fp64 oracle consume what it returns,
so the two sides always see identical bits.

Shapes and value distributions follow the workloads described on the pages:
packed varlen ``[1, T, H, 128]`` bf16 q/k/v, raw (pre-activation) gate per key
channel and raw beta per token-head (aiter PR 4741, Summary), a paged fp32/fp16/bf16
state pool ``[slots, H, V, K]`` with a possibly padded ``stride(0)``, int32
``state_indices`` and bool ``has_initial_state`` (aiter PR 5754, Technical Details),
and host copies of ``cu_seqlens`` (aiter PR 6912, Changes).

Generation order is fixed: lengths -> q -> k -> v -> raw gate -> raw beta -> state ->
indices -> flags, all from one CPU ``torch.Generator`` seeded per workload.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import numpy as np
import torch

HEAD_DIM = 128

_DTYPES = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


@dataclass
class Workload:
    """One synthetic KDA prefill call, all tensors on the CPU."""

    name: str
    q: torch.Tensor  # [1, T, H_qk, K] bf16 (H_qk = H unless value heads are grouped)
    k: torch.Tensor  # [1, T, H_qk, K] bf16
    v: torch.Tensor  # [1, T, H, V] bf16
    g_raw: torch.Tensor  # [1, T, H, K] fp32 (or bf16)
    beta_raw: torch.Tensor  # [1, T, H] fp32 (or bf16)
    cu_seqlens: torch.Tensor  # [N+1] int32
    scale: float
    lower_bound: float
    state_mode: str  # "none" | "dense" | "paged"
    state_dtype: str = "f32"
    initial_state: Optional[torch.Tensor] = None  # dense [N, H, V, K]
    want_final_state: bool = False  # dense mode: also write final_state
    state_storage: Optional[torch.Tensor] = None  # paged: flat storage [slots, stride0]
    state_stride0: int = 0  # paged: elements between slots (>= H*V*K)
    num_slots: int = 0
    state_indices: Optional[torch.Tensor] = None  # [N] int32
    has_initial_state: Optional[torch.Tensor] = None  # [N] bool
    state_k_first: bool = False  # stored state planes are [K, V] rather than [V, K]
    info: dict = field(default_factory=dict)

    @property
    def T(self) -> int:
        return int(self.q.shape[1])

    @property
    def H(self) -> int:
        """Value heads (v, gate, beta, out and state)."""
        return int(self.v.shape[2])

    @property
    def H_qk(self) -> int:
        """q/k heads; each serves H / H_qk consecutive value heads."""
        return int(self.q.shape[2])

    @property
    def N(self) -> int:
        return int(self.cu_seqlens.numel()) - 1

    def cache_view(self) -> torch.Tensor:
        """The pool as ``[slots, H, V, K]`` (a strided view of the flat storage)."""
        assert self.state_storage is not None
        H = self.H
        return self.state_storage.as_strided(
            (self.num_slots, H, HEAD_DIM, HEAD_DIM),
            (self.state_stride0, HEAD_DIM * HEAD_DIM, HEAD_DIM, 1),
        )


def to_f64(t: torch.Tensor) -> np.ndarray:
    """Exact upcast of a stored tensor (bf16/fp16/fp32/int) to an fp64 numpy array."""
    return t.detach().to("cpu").to(torch.float64).numpy()


def _randn(gen: torch.Generator, shape, std: float = 1.0) -> torch.Tensor:
    return torch.randn(shape, generator=gen, dtype=torch.float32) * std


def _lengths_to_cu(lengths) -> torch.Tensor:
    cu = np.zeros(len(lengths) + 1, dtype=np.int64)
    cu[1:] = np.cumsum(np.asarray(lengths, dtype=np.int64))
    return torch.from_numpy(cu.astype(np.int32))


def make_workload(
    name: str,
    lengths,
    H: int,
    *,
    seed: int,
    state_mode: str = "none",
    state_dtype: str = "f32",
    num_slots: int = 0,
    stride_pad: int = 0,
    has_initial: str = "all",  # "all" | "none" | "bernoulli"
    gate_shift: float = 0.0,
    lower_bound: float = -5.0,
    beta_dtype: str = "f32",
    gate_dtype: str = "f32",
    state_std: float = 0.1,
    poison: bool = True,
    want_final_state: bool = True,
    lengths_from_seed: Optional[tuple] = None,
    H_qk: Optional[int] = None,
    state_k_first: bool = False,
) -> Workload:
    """Draw one workload.

    ``lengths`` is a list of per-sequence token counts, or None when
    ``lengths_from_seed=(N, lo, hi, n_zero)`` asks for N lengths uniform in [lo, hi]
    with ``n_zero`` positions (a seeded permutation) forced to 0. ``H_qk`` (dividing
    H) draws q and k with fewer heads than v; ``state_k_first`` marks the stored
    planes as ``[K, V]`` (the random state draws are the same either way).
    """
    gen = torch.Generator("cpu").manual_seed(seed)
    if lengths is None:
        n, lo, hi, n_zero = lengths_from_seed
        lens = torch.randint(lo, hi + 1, (n,), generator=gen).tolist()
        zero_pos = torch.randperm(n, generator=gen)[:n_zero].tolist()
        for p in zero_pos:
            lens[p] = 0
        lengths = lens
    lengths = [int(x) for x in lengths]
    cu = _lengths_to_cu(lengths)
    T = int(cu[-1])
    N = len(lengths)
    K = V = HEAD_DIM

    Hqk = H if H_qk is None else int(H_qk)
    if Hqk < 1 or H % Hqk != 0:
        raise ValueError(f"H_qk={Hqk} must divide H={H}")
    q = _randn(gen, (1, T, Hqk, K)).to(torch.bfloat16)
    k = _randn(gen, (1, T, Hqk, K)).to(torch.bfloat16)
    v = _randn(gen, (1, T, H, V)).to(torch.bfloat16)
    g_raw = (_randn(gen, (1, T, H, K)) + gate_shift).to(_DTYPES[gate_dtype])
    beta_raw = _randn(gen, (1, T, H)).to(_DTYPES[beta_dtype])

    wl = Workload(
        name=name, q=q, k=k, v=v, g_raw=g_raw, beta_raw=beta_raw, cu_seqlens=cu,
        scale=1.0 / float(np.sqrt(K)), lower_bound=float(lower_bound), state_mode=state_mode,
        state_dtype=state_dtype, state_k_first=bool(state_k_first), info={"lengths": lengths, "seed": seed},
    )
    sdt = _DTYPES[state_dtype]
    if state_mode == "dense":
        wl.initial_state = _randn(gen, (N, H, V, K), state_std).to(sdt)
        wl.want_final_state = want_final_state
    elif state_mode == "paged":
        assert num_slots >= N
        plane = H * V * K
        stride0 = plane + int(stride_pad)
        storage = _randn(gen, (num_slots, stride0), state_std)
        if stride_pad and poison:
            storage[:, plane:] = float("nan")  # stride padding: must never be touched
        storage = storage.to(sdt)
        idx = torch.randperm(num_slots, generator=gen)[:N].to(torch.int32)
        if has_initial == "all":
            flags = torch.ones(N, dtype=torch.bool)
        elif has_initial == "none":
            flags = torch.zeros(N, dtype=torch.bool)
        else:
            flags = torch.rand(N, generator=gen) < 0.5
        if poison:
            # A slot whose has_initial_state is false must not be read: poison it.
            for n in range(N):
                if not bool(flags[n]):
                    storage[int(idx[n]), :plane] = float("nan")
        wl.state_storage = storage
        wl.state_stride0 = stride0
        wl.num_slots = num_slots
        wl.state_indices = idx
        wl.has_initial_state = flags
    elif state_mode != "none":
        raise ValueError(state_mode)
    return wl


# The standard shapes: the small dense case the oracle finishes in seconds, the one-GPU
# serving shapes (one long prompt of 4K or 16K tokens, a ragged varlen batch, a batch of
# one-token sequences), each with a fixed seed.
STANDARD = {
    "dense_1x256_H1": dict(lengths=[256], H=1, seed=1001, state_mode="dense"),
    "paged_1x4096_H12": dict(lengths=[4096], H=12, seed=1002, state_mode="paged", num_slots=64),
    "paged_1x16384_H12_pad": dict(lengths=[16384], H=12, seed=1003, state_mode="paged", num_slots=64,
                                  stride_pad=4096),
    # The same call with a steep gate: lower bound -20 and the raw gate shifted by +6, about
    # 640 nats of decay per chunk (prep then uses 4-row reference blocks).
    "paged_1x16384_H12_pad_lb20": dict(lengths=[16384], H=12, seed=1003, state_mode="paged", num_slots=64,
                                       stride_pad=4096, lower_bound=-20.0, gate_shift=6.0),
    "paged_varlen128_H12": dict(lengths=None, H=12, seed=1004, state_mode="paged", num_slots=256,
                                has_initial="bernoulli", lengths_from_seed=(128, 0, 2048, 4)),
    "paged_256x1_H12_bf16": dict(lengths=[1] * 256, H=12, seed=1005, state_mode="paged",
                                 state_dtype="bf16", num_slots=512),
    "paged_256x1_H12_f16": dict(lengths=[1] * 256, H=12, seed=1005, state_mode="paged",
                                state_dtype="f16", num_slots=512),
    # One decode step of 64 sequences at the per-GPU head count, 2-byte and 4-byte state.
    "paged_64x1_H12_f16": dict(lengths=[1] * 64, H=12, seed=1006, state_mode="paged",
                               state_dtype="f16", num_slots=128),
    "paged_64x1_H12_f32": dict(lengths=[1] * 64, H=12, seed=1007, state_mode="paged",
                               state_dtype="f32", num_slots=128),
    # The same shapes with K-first state planes, and with grouped value heads (6 q/k heads
    # for 12 value heads).
    "paged_256x1_H12_bf16_kfirst": dict(lengths=[1] * 256, H=12, seed=1005, state_mode="paged",
                                        state_dtype="bf16", num_slots=512, state_k_first=True),
    "paged_1x4096_H12_qk6": dict(lengths=[4096], H=12, H_qk=6, seed=1002, state_mode="paged", num_slots=64),
}


def standard(name: str, **overrides) -> Workload:
    """One of the standard shapes by name; ``overrides`` adjust it."""
    if name not in STANDARD:
        raise ValueError(f"unknown workload {name!r}; known: {sorted(STANDARD)}")
    kw = dict(STANDARD[name], name=name)
    kw.update(overrides)
    return make_workload(**kw)
