"""CPU tests of the Python binding: argument checks and the shared context's lock.

``make_args`` fills the C struct from tensors and must reject every tensor the C side
cannot check (it only sees raw pointers): a wrong dtype, shape, element count or
non-contiguous layout would otherwise be read or written out of bounds by the kernels.
The tensors here are CPU tensors: ``make_args`` only reads their metadata and pointers.
"""
import ctypes
import threading

import numpy as np
import pytest
import torch

import gated_delta_rule_pack_amd as kda
from gated_delta_rule_pack_amd import _lib
from tests.test_abi_cpu import FakeBufs, FakeRuntime, _valid_args

T, N, H = 70, 3, 2


def _base():
    bf = torch.bfloat16
    d = dict(
        q=torch.zeros(1, T, H, 128, dtype=bf), k=torch.zeros(1, T, H, 128, dtype=bf),
        v=torch.zeros(1, T, H, 128, dtype=bf), g_raw=torch.zeros(1, T, H, 128),
        beta_raw=torch.zeros(1, T, H), cu_seqlens=torch.tensor([0, 10, 10, T], dtype=torch.int32),
    )
    kw = dict(state_cache=torch.zeros(5, H, 128, 128), state_indices=torch.tensor([4, 0, 2], dtype=torch.int32),
              has_initial_state=torch.tensor([True, False, True]), out=torch.zeros(1, T, H, 128, dtype=bf))
    return d, kw


def _make(d, kw):
    return kda.make_args(d["q"], d["k"], d["v"], d["g_raw"], d["beta_raw"], d["cu_seqlens"], **kw)


def test_valid_paged_and_dense_args_fill_the_struct():
    d, kw = _base()
    a = _make(d, kw)
    assert (a.T, a.N, a.H, a.H_qk) == (T, N, H, H) and a.num_slots == 5
    assert a.state_cache_stride0 == H * 128 * 128 and a.state_dtype == _lib.KDA_F32
    init = torch.zeros(N, H, 128, 128, dtype=torch.float16)
    fin = torch.zeros(N, H, 128, 128, dtype=torch.float16)
    a = _make(d, dict(initial_state=init, final_state=fin, out=kw["out"]))
    assert a.state_dtype == _lib.KDA_F16 and a.initial_state and a.final_state


def _mut(name, value):
    def f(d, kw):
        (d if name in d else kw)[name] = value
    return f


BF = torch.bfloat16
REJECT = {
    "int64 state_indices": (_mut("state_indices", torch.tensor([4, 0, 2])), TypeError),
    "short state_indices": (_mut("state_indices", torch.tensor([4, 0], dtype=torch.int32)), ValueError),
    "strided state_indices": (_mut("state_indices", torch.tensor([4, 9, 0, 9, 2, 9], dtype=torch.int32)[::2]),
                              ValueError),
    "float flags": (_mut("has_initial_state", torch.ones(3)), TypeError),
    "short flags": (_mut("has_initial_state", torch.ones(2, dtype=torch.bool)), ValueError),
    "no flags": (_mut("has_initial_state", None), ValueError),
    "fp32 out": (_mut("out", torch.zeros(1, T, H, 128)), TypeError),
    "short out": (_mut("out", torch.zeros(1, T - 1, H, 128, dtype=BF)), ValueError),
    "strided out": (_mut("out", torch.zeros(1, T, H, 256, dtype=BF)[..., ::2]), ValueError),
    "fp32 q": (_mut("q", torch.zeros(1, T, H, 128)), TypeError),
    "fp16 v": (_mut("v", torch.zeros(1, T, H, 128, dtype=torch.float16)), TypeError),
    "fp16 gate": (_mut("g_raw", torch.zeros(1, T, H, 128, dtype=torch.float16)), TypeError),
    "gate per head": (_mut("g_raw", torch.zeros(1, T, H, 1)), ValueError),
    "beta per channel": (_mut("beta_raw", torch.zeros(1, T, H, 128)), ValueError),
    "int64 bounds": (_mut("cu_seqlens", torch.tensor([0, 10, 10, T])), TypeError),
    "pool of wrong heads": (_mut("state_cache", torch.zeros(5, H + 1, 128, 128)), ValueError),
    "pool of ints": (_mut("state_cache", torch.zeros(5, H, 128, 128, dtype=torch.int32)), TypeError),
    "transposed pool planes": (_mut("state_cache", torch.zeros(5, H, 128, 128).transpose(2, 3)), ValueError),
}


@pytest.mark.parametrize("case", sorted(REJECT))
def test_make_args_rejects(case):
    mutate, exc = REJECT[case]
    d, kw = _base()
    mutate(d, kw)
    with pytest.raises(exc):
        _make(d, kw)


def test_dense_state_checks():
    d, kw = _base()
    out = kw["out"]
    for init, exc in ((torch.zeros(N, H, 128, 64), ValueError),            # short planes
                      (torch.zeros(N - 1, H, 128, 128), ValueError),       # one sequence short
                      (torch.zeros(N, H, 128, 128)[:, :, :, :].transpose(2, 3), ValueError),  # not contiguous
                      (torch.zeros(N, H, 128, 128, dtype=torch.float64), TypeError)):
        with pytest.raises(exc):
            _make(d, dict(initial_state=init, out=out))
    with pytest.raises(TypeError):  # final state must take the initial state's dtype
        _make(d, dict(initial_state=torch.zeros(N, H, 128, 128, dtype=BF), final_state=torch.zeros(N, H, 128, 128),
                      out=out))
    # K-first planes are [K, V]: the same shape here, since K = V.
    _make(d, dict(initial_state=torch.zeros(N, H, 128, 128), out=out, state_k_first=True))


def test_host_bounds_checks():
    d, kw = _base()
    with pytest.raises(TypeError):
        _make(d, dict(kw, cu_seqlens_cpu=torch.tensor([0, 10, 10, T])))
    with pytest.raises(ValueError):
        _make(d, dict(kw, cu_seqlens_cpu=torch.tensor([0, 10, T], dtype=torch.int32)))


def test_threads_sharing_a_context_are_serialised():
    """Two threads issue calls on one shared context. Each call runs whole, without the
    other thread's runtime calls in between: every call's callbacks start with its
    capture query and end with its scan launch, and no other thread appears in between."""
    fake = FakeRuntime()
    trace = []
    lock = threading.Lock()
    orig_capt, orig_launch = fake._capt, fake._launch

    def capt(user, s, out):
        with lock:
            trace.append((threading.get_ident(), "begin"))
        return orig_capt(user, s, out)

    def launch(user, k, plan, s, start, stop):
        with lock:
            trace.append((threading.get_ident(), "scan" if k == 1 else "kernel"))
        return orig_launch(user, k, plan, s, start, stop)

    fake._cbs["stream_is_capturing"] = _lib.CAPT(capt)
    fake._cbs["launch"] = _lib.LAUNCH(launch)
    fake.rt.stream_is_capturing = fake._cbs["stream_is_capturing"]
    fake.rt.launch = fake._cbs["launch"]
    ctx = kda.Context(0, runtime=fake.rt, cu_count=256)
    bufs = FakeBufs()

    def worker(base):
        for i in range(150):
            a, _, _ = _valid_args(bufs, T=100 + base + i, N=1, cu=np.array([0, 100 + base + i], np.int32))
            ws = bufs.buf(max(kda.workspace_bytes(a), 256))
            assert ctx.forward(a, ws.ctypes.data, ws.nbytes, 0x10) == _lib.KDA_OK
            fake.complete_all()

    threads = [threading.Thread(target=worker, args=(1000 * j,)) for j in range(2)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert ctx.stats()["calls"] == 300
    owner = None
    for tid, what in trace:
        if what == "begin":
            assert owner is None, "a call began inside another thread's call"
            owner = tid
        else:
            assert tid == owner, "a launch from another thread inside a call"
            if what == "scan":
                owner = None
    assert len({tid for tid, _ in trace}) == 2
    ctx.close()
