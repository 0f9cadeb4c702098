"""CPU tests of the C ABI (no GPU needed): exports, validation, sizing, chunk table,
and the host orchestration driven through a recording fake runtime.

The fake runtime stands in for HIP: "device" memory is host memory, copies are memmoves,
events are integers whose completion the test controls, and kernel launches are only
recorded. This exercises the metadata cache, the device and pinned arenas, the no-sync
contract with host bounds and the capture rules without a GPU.
"""
import ctypes
import os
import re

import numpy as np
import pytest

from gated_delta_rule_pack_amd import _lib
from oracle import chunk_indices

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
REC = 35328


@pytest.fixture(scope="module")
def lib():
    return _lib.load()


def test_header_exports_match_library(lib):
    text = open(os.path.join(ROOT, "include", "kda.h")).read()
    declared = set(re.findall(r"\b(kda_[a-z0-9_]+)\s*\(", text))
    declared -= {"kda_status", "kda_dtype"}
    assert declared == set(_lib.EXPORTS), declared ^ set(_lib.EXPORTS)
    for name in declared:
        assert hasattr(lib, name), name
    assert lib.kda_fwd_args_size() == ctypes.sizeof(_lib.FwdArgs)
    assert lib.kda_stats_size() == ctypes.sizeof(_lib.Stats)


def test_status_strings(lib):
    for code in range(9):
        assert lib.kda_status_str(code)


# ---------------------------------------------------------------- validation
class FakeBufs:
    """Aligned host buffers whose addresses stand in for device pointers."""

    def __init__(self):
        self.keep = []

    def buf(self, nbytes, align=256):
        raw = np.zeros(nbytes + align, np.uint8)
        self.keep.append(raw)
        off = (-raw.ctypes.data) % align
        return raw[off:off + nbytes]


def _valid_args(bufs, T=100, N=3, H=2, paged=False, cu=None):
    a = _lib.FwdArgs()
    a.T, a.N, a.H, a.K, a.V = T, N, H, 128, 128
    a.scale, a.lower_bound = 0.088, -5.0
    tok = T * H * 128
    for name, nb in (("q", 2), ("k", 2), ("v", 2), ("g_raw", 4), ("out", 2)):
        setattr(a, name, bufs.buf(max(tok * nb, 16)).ctypes.data)
    a.beta_raw = bufs.buf(max(T * H * 4, 16)).ctypes.data
    a.g_dtype = a.beta_dtype = _lib.KDA_F32
    if cu is None:
        cu = np.array([0, 40, 40, T][: N] + [T], np.int32) if N == 3 else np.linspace(0, T, N + 1).astype(np.int32)
    cu_dev = bufs.buf(4 * (N + 1), 16).view(np.int32)
    cu_dev[:] = cu
    cu_host = bufs.buf(4 * (N + 1), 16).view(np.int32)
    cu_host[:] = cu
    a.cu_seqlens = cu_dev.ctypes.data
    a.cu_seqlens_host = cu_host.ctypes.data
    a.state_dtype = _lib.KDA_F32
    if paged:
        a.state_cache = bufs.buf(4 * 4 * H * 128 * 128).ctypes.data
        a.num_slots = 4
        a.state_cache_stride0 = H * 128 * 128
        a.state_indices = bufs.buf(4 * N, 16).ctypes.data
        a.has_initial_state = bufs.buf(N, 16).ctypes.data
    return a, cu_dev, cu_host


def _check(lib, a):
    return lib.kda_chunk_fwd_validate(ctypes.byref(a))


def test_validation_accepts_valid_args(lib):
    bufs = FakeBufs()
    for paged in (False, True):
        a, _, _ = _valid_args(bufs, paged=paged)
        assert _check(lib, a) == _lib.KDA_OK


@pytest.mark.parametrize("H_qk,k_first", [(0, 1), (1, 0), (2, 1), (1, 1)])
def test_validation_accepts_grouped_heads_and_k_first(lib, H_qk, k_first):
    bufs = FakeBufs()
    a, _, _ = _valid_args(bufs, paged=True)
    assert a.H == 2
    a.H_qk, a.state_k_first = H_qk, k_first
    assert _check(lib, a) == _lib.KDA_OK


@pytest.mark.parametrize("mutate,code", [
    (lambda a, b: setattr(a, "N", 0), _lib.KDA_ERR_INVALID_ARG),
    (lambda a, b: setattr(a, "T", -1), _lib.KDA_ERR_INVALID_ARG),
    (lambda a, b: setattr(a, "K", 64), _lib.KDA_ERR_UNSUPPORTED),
    (lambda a, b: setattr(a, "V", 256), _lib.KDA_ERR_UNSUPPORTED),
    (lambda a, b: setattr(a, "scale", float("nan")), _lib.KDA_ERR_INVALID_ARG),
    (lambda a, b: setattr(a, "lower_bound", 0.5), _lib.KDA_ERR_UNSUPPORTED),
    (lambda a, b: setattr(a, "g_dtype", _lib.KDA_F16), _lib.KDA_ERR_UNSUPPORTED),
    (lambda a, b: setattr(a, "state_dtype", 7), _lib.KDA_ERR_UNSUPPORTED),
    (lambda a, b: setattr(a, "q", None), _lib.KDA_ERR_INVALID_ARG),
    (lambda a, b: setattr(a, "out", None), _lib.KDA_ERR_INVALID_ARG),
    (lambda a, b: setattr(a, "cu_seqlens", None), _lib.KDA_ERR_INVALID_ARG),
    (lambda a, b: setattr(a, "q", a.q + 2), _lib.KDA_ERR_INVALID_ARG),  # misaligned
    (lambda a, b: setattr(a, "out", a.v), _lib.KDA_ERR_ALIAS),
    (lambda a, b: setattr(a, "out", a.v + 16 * 1024), _lib.KDA_ERR_ALIAS),  # partial overlap
    (lambda a, b: setattr(a, "state_cache_stride0", 2 * 128 * 128 - 1), _lib.KDA_ERR_STRIDE),
    (lambda a, b: setattr(a, "initial_state", b.buf(64).ctypes.data), _lib.KDA_ERR_STATE_MODE),
    (lambda a, b: setattr(a, "final_state", b.buf(64).ctypes.data), _lib.KDA_ERR_STATE_MODE),
    (lambda a, b: setattr(a, "state_indices", None), _lib.KDA_ERR_INVALID_ARG),
    (lambda a, b: setattr(a, "has_initial_state", None), _lib.KDA_ERR_INVALID_ARG),
    (lambda a, b: setattr(a, "num_slots", 0), _lib.KDA_ERR_INVALID_ARG),
    (lambda a, b: setattr(a, "H_qk", -1), _lib.KDA_ERR_INVALID_ARG),
    (lambda a, b: setattr(a, "H_qk", 3), _lib.KDA_ERR_INVALID_ARG),   # more q/k heads than value heads
    (lambda a, b: (setattr(a, "H", 6), setattr(a, "H_qk", 4)), _lib.KDA_ERR_INVALID_ARG),  # 4 does not divide 6
    (lambda a, b: setattr(a, "state_k_first", 2), _lib.KDA_ERR_INVALID_ARG),
])
def test_validation_errors(lib, mutate, code):
    bufs = FakeBufs()
    a, _, _ = _valid_args(bufs, paged=True)
    mutate(a, bufs)
    assert _check(lib, a) == code
    assert lib.kda_chunk_fwd_workspace_bytes(ctypes.byref(a)) == 0


def test_validation_rejects_inconsistent_host_bounds(lib):
    bufs = FakeBufs()
    for bad in ([0, 50, 40, 100], [1, 40, 60, 100], [0, 40, 60, 99]):
        a, _, host = _valid_args(bufs)
        host[:] = bad
        assert _check(lib, a) == _lib.KDA_ERR_INVALID_ARG


def test_padded_stride_and_zero_tokens_accepted(lib):
    bufs = FakeBufs()
    a, _, _ = _valid_args(bufs, paged=True)
    a.state_cache_stride0 = 2 * 128 * 128 + 4096
    assert _check(lib, a) == _lib.KDA_OK
    a.state_cache_stride0 = 2 * 128 * 128 + 3  # breaks the 16-byte alignment of every slot plane
    assert _check(lib, a) == _lib.KDA_ERR_INVALID_ARG
    z, _, _ = _valid_args(bufs, T=0, N=2, cu=np.array([0, 0, 0], np.int32))
    z.q = z.k = z.v = z.g_raw = z.beta_raw = z.out = None
    assert _check(lib, z) == _lib.KDA_OK


MAP_BYTES = 2 * 128 * 128 * 4    # segment map A and C, fp32
START_BYTES = 128 * 128 * 4      # segment start state, fp32


def test_workspace_bytes(lib):
    bufs = FakeBufs()
    for T, N, H in [(100, 3, 2), (4096, 1, 12), (0, 2, 1), (1, 1, 1), (5000, 9, 12), (16384, 8, 12)]:
        cu = np.linspace(0, T, N + 1).astype(np.int32)
        a, _, _ = _valid_args(bufs, T=T, N=N, H=H, cu=cu)
        if T == 0:
            a.q = a.k = a.v = a.g_raw = a.beta_raw = a.out = None
        max_chunks = (T + 31) // 32 + N
        # Records; then, when the call may be segmented (N*H <= 96), room for the maps of
        # segments of at least 8 chunks and two start states per map (the segment after it;
        # at most as many multi-segment sequences, whose first segments get one each).
        want = H * max_chunks * REC
        if N * H <= 96:
            want += (max_chunks // 8) * H * (MAP_BYTES + 2 * START_BYTES)
        assert lib.kda_chunk_fwd_workspace_bytes(ctypes.byref(a)) == want


# ---------------------------------------------------------------- chunk table, policies
def _chunk_table(lib, cu, chunk=32):
    cu = np.ascontiguousarray(cu, np.int32)
    n = ctypes.c_int64()
    rc = lib.kda_prepare_chunk_indices(cu.ctypes.data, len(cu) - 1, chunk, None, 0, ctypes.byref(n))
    out = np.zeros((max(n.value, 1), 2), np.int32)
    rc2 = lib.kda_prepare_chunk_indices(cu.ctypes.data, len(cu) - 1, chunk, out.ctypes.data, n.value,
                                        ctypes.byref(n))
    assert rc2 == _lib.KDA_OK
    return rc, out[: n.value]


@pytest.mark.parametrize("seed", range(6))
def test_chunk_table_matches_repeat_interleave_reference(lib, seed):
    rng = np.random.default_rng(seed)
    lens = rng.integers(0, 200, size=rng.integers(1, 40))
    lens[rng.random(lens.size) < 0.3] = 0  # plenty of empty sequences, also before non-empty ones
    cu = np.concatenate([[0], np.cumsum(lens)])
    rc, got = _chunk_table(lib, cu)
    assert np.array_equal(got, chunk_indices(cu, 32))
    if got.shape[0] > 0:
        assert rc == _lib.KDA_ERR_INVALID_ARG  # first call had cap 0: reports the count only


def test_dv_split_and_ref_block_policies(lib):
    assert lib.kda_dv_split(1, 12, 256) == 8
    assert lib.kda_dv_split(2, 12, 256) == 8
    assert lib.kda_dv_split(3, 12, 256) == 4
    assert lib.kda_dv_split(8, 12, 256) == 2
    assert lib.kda_dv_split(10, 12, 256) == 2
    assert lib.kda_dv_split(11, 12, 256) == 1
    assert lib.kda_dv_split(128, 12, 256) == 1
    assert lib.kda_ref_block(-5.0) == 16
    assert lib.kda_ref_block(-5.4) == 8
    assert lib.kda_ref_block(-20.0) == 4
    assert lib.kda_ref_block(0.0) == 16
    assert lib.kda_ref_block(-200.0) == 1


def test_segment_length_policy(lib):
    # Few long sequences: about 8 segments for the longest, at least 8 chunks each.
    assert lib.kda_seg_len(1, 12, 512, 0) == 64
    assert lib.kda_seg_len(1, 16, 512, 256) == 64    # 10 segments would leave dv_split 2
    assert lib.kda_seg_len(1, 8, 512, 256) == 64     # 8 segments still take dv_split 4
    assert lib.kda_seg_len(8, 12, 256, 256) == 32
    assert lib.kda_seg_len(4, 2, 301, 256) == 38
    # 12 heads on 256 CUs: 8 segments already take dv_split 2 and 10 still do.
    assert lib.kda_seg_len(1, 12, 512, 256) == 52
    assert lib.kda_seg_len(1, 12, 500, 256) == 50
    for L, H in ((52, 12),):
        segs = -(-512 // L)
        assert segs == 10 and lib.kda_dv_split(segs, H, 256) == 2
    # Short sequences, or enough (sequence, head) units already: not segmented.
    assert lib.kda_seg_len(1, 12, 128, 256) == 0
    assert lib.kda_seg_len(1, 12, 255, 256) == 0
    assert lib.kda_seg_len(9, 12, 1000, 256) == 0
    assert lib.kda_seg_len(128, 12, 64, 256) == 0


# ---------------------------------------------------------------- fake runtime
class FakeRuntime:
    def __init__(self):
        self.log = []
        self.next_ev = 1
        self.pending = set()  # events not yet complete
        self.capturing = set()
        self.alloc = {}
        self.uploads = []
        self.launches = []
        self.launch_events = []
        rt = _lib.Runtime()
        rt.user = None
        self._cbs = dict(
            memcpy_h2d_async=_lib.H2D(self._h2d), memcpy_d2h_async=_lib.D2H(self._d2h),
            stream_synchronize=_lib.SYNC(self._sync), stream_is_capturing=_lib.CAPT(self._capt),
            event_create=_lib.EVCREATE(self._ev_create), event_destroy=_lib.EVONE(self._ev_destroy),
            event_record=_lib.EVREC(self._ev_record), event_query=_lib.EVONE(self._ev_query),
            event_synchronize=_lib.EVONE(self._ev_sync), stream_wait_event=_lib.WAIT(self._wait),
            host_alloc_pinned=_lib.ALLOC(self._halloc), host_free_pinned=_lib.FREE(self._hfree),
            device_alloc=_lib.ALLOC(self._dalloc), device_free=_lib.FREE(self._dfree),
            launch=_lib.LAUNCH(self._launch), event_create_timed=_lib.EVCREATE(self._ev_create),
            event_elapsed_ms=_lib.ELAPSED(self._elapsed), event_create_completion=_lib.EVCREATE(self._ev_create),
            upload=_lib.UPLOAD(self._upload))
        for k, v in self._cbs.items():
            setattr(rt, k, v)
        self.rt = rt

    def _h2d(self, user, dst, src, n, s):
        ctypes.memmove(dst, src, n)
        self.uploads.append((dst, n, s, np.frombuffer(ctypes.string_at(src, n), np.int32).copy()))
        self.log.append(("h2d", s))
        return 0

    def _upload(self, user, dst, src, n, s, done):
        # A copy whose completion event the copy records itself (no separate marker).
        self._h2d(user, dst, src, n, s)
        self.pending.add(done)
        self.log.append(("record", done, s))
        return 0

    def _d2h(self, user, dst, src, n, s):
        ctypes.memmove(dst, src, n)
        self.log.append(("d2h", s))
        return 0

    def _sync(self, user, s):
        self.log.append(("stream_sync", s))
        self.pending.clear()
        return 0

    def _capt(self, user, s, out):
        out[0] = 1 if s in self.capturing else 0
        return 0

    def _ev_create(self, user, out):
        out[0] = self.next_ev
        self.next_ev += 1
        return 0

    def _ev_destroy(self, user, e):
        return 0

    def _ev_record(self, user, e, s):
        self.marker_records = getattr(self, "marker_records", 0) + 1
        self.pending.add(e)
        self.log.append(("record", e, s))
        return 0

    def _ev_query(self, user, e):
        return 1 if e in self.pending else 0

    def _ev_sync(self, user, e):
        self.log.append(("event_sync", e))
        self.pending.discard(e)
        return 0

    def _wait(self, user, s, e):
        self.log.append(("wait", s, e))
        return 0

    def _halloc(self, user, out, n):
        buf = ctypes.create_string_buffer(n)
        out[0] = ctypes.addressof(buf)
        self.alloc[out[0]] = buf
        self.log.append(("host_alloc", n))
        return 0

    def _hfree(self, user, p):
        self.alloc.pop(p, None)
        return 0

    def _dalloc(self, user, out, n):
        buf = ctypes.create_string_buffer(n)
        out[0] = ctypes.addressof(buf)
        self.alloc[out[0]] = buf
        self.log.append(("dev_alloc", n))
        return 0

    def _dfree(self, user, p):
        self.alloc.pop(p, None)
        self.log.append(("dev_free", p))
        return 0

    def _launch(self, user, k, plan, s, start, stop):
        # Events attached to a launch are recorded by it, as a marker right after it would be.
        self.launches.append((k, s))
        self.launch_events.append((k, start or 0, stop or 0))
        for e in (start, stop):
            if e:
                self.pending.add(e)
                self.log.append(("record", e, s))
        return 0

    def _elapsed(self, user, out, a, b):
        out[0] = 1.0
        return 0

    def syncs(self):
        return [e for e in self.log if e[0] in ("stream_sync", "event_sync")]

    def complete_all(self):
        self.pending.clear()


@pytest.fixture
def fake(lib):
    f = FakeRuntime()
    ctx = ctypes.c_void_p()
    assert lib.kda_ctx_create_with_runtime(ctypes.byref(f.rt), 256, ctypes.byref(ctx)) == _lib.KDA_OK
    f.ctx = ctx
    f.creation_log, f.log = f.log, []
    yield f
    lib.kda_ctx_destroy(ctx)


def _call(lib, fake, a, stream=0x10, ws=None):
    bufs = FakeBufs()
    need = lib.kda_chunk_fwd_workspace_bytes(ctypes.byref(a))
    ws = ws if ws is not None else bufs.buf(max(need, 256))
    return lib.kda_chunk_fwd(fake.ctx, ctypes.byref(a), ws.ctypes.data, ws.nbytes, stream)


def _stats(lib, fake):
    s = _lib.Stats()
    lib.kda_get_stats(fake.ctx, ctypes.byref(s))
    return s.as_dict()


def test_host_bounds_issue_no_sync_and_one_upload(lib, fake):
    bufs = FakeBufs()
    a, _, host = _valid_args(bufs, T=300, N=4, cu=np.array([0, 0, 100, 100, 300], np.int32), paged=True)
    assert _call(lib, fake, a) == _lib.KDA_OK
    assert fake.syncs() == []
    assert [e[0] for e in fake.log].count("h2d") == 1
    assert [e[0] for e in fake.log].count("d2h") == 0
    assert fake.launches == [(0, 0x10), (1, 0x10)]
    # The uploaded buffer: cu, per-sequence chunk offsets, chunk table (16-byte aligned blocks).
    words = fake.uploads[0][3]
    N = 4
    cu = words[:N + 1]
    co = words[8:8 + N + 1]
    table = words[16:16 + 2 * 11].reshape(-1, 2)
    assert list(cu) == [0, 0, 100, 100, 300]
    assert list(co) == [0, 0, 4, 4, 11]
    ref = chunk_indices(cu, 32)
    assert np.array_equal(table[: ref.shape[0]], ref)
    st = _stats(lib, fake)
    assert st["cache_misses"] == 1 and st["cache_hits"] == 0 and st["blocking_syncs"] == 0
    # Same bounds again: cache hit, no upload, still no sync.
    assert _call(lib, fake, a) == _lib.KDA_OK
    assert [e[0] for e in fake.log].count("h2d") == 1
    assert fake.syncs() == []
    st = _stats(lib, fake)
    assert st["cache_hits"] == 1 and st["calls"] == 2 and st["last_n_chunks"] == 11


def test_hit_path_records_only_the_launch_attached_completion(lib, fake):
    """On a cache hit the only stream operations are the two launches: the entry's use is
    tracked by a completion event the scan launch records itself, the same event on every
    call on one stream, with no marker of its own."""
    bufs = FakeBufs()
    a, _, _ = _valid_args(bufs, T=300, N=4, cu=np.array([0, 0, 100, 100, 300], np.int32), paged=True)
    assert _call(lib, fake, a) == _lib.KDA_OK
    mark = len(fake.log)
    for _ in range(3):
        assert _call(lib, fake, a) == _lib.KDA_OK
    ev = fake.launch_events[1][2]
    assert ev != 0 and fake.launch_events[0] == (0, 0, 0)
    assert fake.launch_events[2:] == [(0, 0, 0), (1, 0, ev)] * 3
    assert fake.log[mark:] == [("record", ev, 0x10)] * 3
    # A second stream gets its own completion event.
    assert _call(lib, fake, a, stream=0x20) == _lib.KDA_OK
    ev2 = fake.launch_events[-1][2]
    assert fake.launch_events[-1][0] == 1 and ev2 not in (0, ev)


def test_profiling_attaches_timing_events_to_launches(lib, fake):
    """While profiling, prep and scan carry start / end timing events; the use event is then
    recorded after the scan. A call without chunks launches the scan alone and reads back
    a zero prep time."""
    bufs = FakeBufs()
    a, _, _ = _valid_args(bufs, T=300, N=4, cu=np.array([0, 0, 100, 100, 300], np.int32), paged=True)
    assert lib.kda_profile_enable(fake.ctx, 1) == _lib.KDA_OK
    assert _call(lib, fake, a) == _lib.KDA_OK
    (k0, s0, e0), (k1, s1, e1) = fake.launch_events
    assert (k0, k1) == (0, 1) and len({s0, e0, s1, e1}) == 4 and 0 not in (s0, e0, s1, e1)
    assert fake.log[-1][0] == "record" and fake.log[-1][1] not in (s0, e0, s1, e1)
    b, _, _ = _valid_args(bufs, T=0, N=2, cu=np.array([0, 0, 0], np.int32), paged=True)
    fake.launches.clear()
    assert _call(lib, fake, b) == _lib.KDA_OK
    assert fake.launches == [(4, 0x10)]  # no sequence longer than one token: decode alone
    per_call, n = (ctypes.c_float * 4)(), ctypes.c_int64()
    assert lib.kda_profile_calls(fake.ctx, per_call, 4, ctypes.byref(n)) == _lib.KDA_OK
    assert n.value == 2 and list(per_call)[:2] == [1.0, 1.0]  # first kernel start to scan end
    assert lib.kda_profile_calls(fake.ctx, None, 0, ctypes.byref(n)) == _lib.KDA_OK and n.value == 2
    assert lib.kda_profile_calls(fake.ctx, None, 4, ctypes.byref(n)) == _lib.KDA_ERR_INVALID_ARG
    prep, scan, calls = ctypes.c_double(), ctypes.c_double(), ctypes.c_int64()
    assert lib.kda_profile_read(fake.ctx, ctypes.byref(prep), ctypes.byref(scan), ctypes.byref(calls)) == _lib.KDA_OK
    assert calls.value == 2 and prep.value == 1.0 and scan.value == 2.0
    assert lib.kda_profile_enable(fake.ctx, 0) == _lib.KDA_OK


def test_one_token_calls_take_the_decode_kernel(lib, fake):
    """Calls whose sequences have at most one token launch the decode kernel alone; a
    single longer sequence brings back prep and scan."""
    bufs = FakeBufs()
    a, _, _ = _valid_args(bufs, T=3, N=4, cu=np.array([0, 1, 1, 2, 3], np.int32), paged=True)
    assert _call(lib, fake, a) == _lib.KDA_OK
    assert fake.launches == [(4, 0x10)]
    assert _stats(lib, fake)["last_path"] == 1
    fake.launches.clear()
    b, _, _ = _valid_args(bufs, T=3, N=2, cu=np.array([0, 1, 3], np.int32), paged=True)
    assert _call(lib, fake, b) == _lib.KDA_OK
    assert fake.launches == [(0, 0x10), (1, 0x10)]
    assert _stats(lib, fake)["last_path"] == 0


def _segments_reference(cu, L):
    """Segments of each sequence: runs of L chunks (the last shorter), one empty segment
    for an empty sequence; map slots numbered over all segments but each sequence's last.
    Start-state slots: the segment after map slot m starts from slot m; the first segment
    of the k-th multi-segment sequence from slot n_maps + k (a copy of the initial state);
    only a single-segment sequence reads the caller's state (-1)."""
    counts = [-(-(int(cu[n + 1]) - int(cu[n])) // 32) for n in range(len(cu) - 1)]
    groups = [1 if nc <= L else -(-nc // L) for nc in counts]
    n_maps = sum(G - 1 for G in groups)
    segs, m2s, comb, mbase = [], [], [], 0
    for n, (nc, G) in enumerate(zip(counts, groups)):
        for g in range(G):
            c0 = g * L
            nch = nc if G == 1 else min(L, nc - c0)
            m_prev = mbase + g - 1 if g > 0 else (n_maps + len(comb) if G > 1 else -1)
            m_self = -1 if g == G - 1 else mbase + g
            if m_self >= 0:
                m2s.append(len(segs))
            segs.append([n, c0, nch, m_prev, m_self, 0, 0, 0])
        if G > 1:
            comb.append([n, mbase, G - 1, n_maps + len(comb)])
        mbase += G - 1
    return np.array(segs, np.int32), np.array(m2s, np.int32), np.array(comb, np.int32).reshape(-1, 4)


def test_segmented_call_launches_and_tables(lib, fake):
    """A long sequence next to short and empty ones: segment maps and combine run between
    prep and scan, and the uploaded segment tables match a plain reference."""
    bufs = FakeBufs()
    lens = [300 * 32 + 5, 0, 100, 40 * 32]   # 301, 0, 4 and 40 chunks
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    N, T, H = len(lens), int(cu[-1]), 2
    a, _, _ = _valid_args(bufs, T=T, N=N, H=H, cu=cu, paged=True)
    L = lib.kda_seg_len(N, H, 301, 256)
    assert L == 38
    assert _call(lib, fake, a) == _lib.KDA_OK
    assert fake.launches == [(0, 0x10), (2, 0x10), (3, 0x10), (1, 0x10)]
    st = _stats(lib, fake)
    segs, m2s, comb = _segments_reference(cu, L)
    assert st["last_seg_len"] == L and st["last_n_segments"] == len(segs)
    # Buffer layout: cu, chunk offsets, chunk table, segment table, map -> segment,
    # multi-segment sequences; every block starts 16-byte aligned.
    words = fake.uploads[0][3]
    a4 = lambda n: (n + 3) // 4 * 4
    n_chunks = int(sum(-(-x // 32) for x in lens))
    off_seg = 2 * a4(N + 1) + a4(2 * n_chunks)
    off_m2s = off_seg + a4(8 * len(segs))
    off_comb = off_m2s + a4(len(m2s))
    assert np.array_equal(words[off_seg:off_seg + 8 * len(segs)].reshape(-1, 8), segs)
    assert np.array_equal(words[off_m2s:off_m2s + len(m2s)], m2s)
    assert np.array_equal(words[off_comb:off_comb + 4 * len(comb)].reshape(-1, 4), comb)
    # The segments tile every sequence's chunks exactly once, in order.
    for n in range(N):
        mine = segs[segs[:, 0] == n]
        nc = -(-lens[n] // 32)
        assert mine[0, 1] == 0 and mine[:, 2].sum() == nc
        assert np.all(mine[1:, 1] == mine[:-1, 1] + mine[:-1, 2])
    # Only a sequence with a single segment reads the caller's state in the scan: the last
    # segment of a longer one writes that plane from another workgroup of the same launch.
    uploaded = words[off_seg:off_seg + 8 * len(segs)].reshape(-1, 8)
    for n in range(N):
        mine = uploaded[uploaded[:, 0] == n]
        if len(mine) > 1:
            assert np.all(mine[:, 3] >= 0), (n, mine[:, 3])
            assert len(set(mine[:, 3].tolist())) == len(mine)
    n_maps = len(m2s)
    assert sorted(comb[:, 3].tolist()) == list(range(n_maps, n_maps + len(comb)))


def test_unsegmented_table_lists_longest_sequences_first(lib, fake):
    """Without segmentation every sequence is one scan unit; the uploaded segment table
    lists them longest first (ties in sequence order), each exactly once, with its whole
    chunk count, no start-state slot and the final-state write."""
    bufs = FakeBufs()
    lens = [100, 0, 2048, 33, 2048, 1, 640, 0]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    N, T, H = len(lens), int(cu[-1]), 16   # N * H > 96: not segmented
    a, _, _ = _valid_args(bufs, T=T, N=N, H=H, cu=cu, paged=True)
    assert _call(lib, fake, a) == _lib.KDA_OK
    assert _stats(lib, fake)["last_seg_len"] == 0
    words = fake.uploads[0][3]
    a4 = lambda n: (n + 3) // 4 * 4
    n_chunks = int(sum(-(-x // 32) for x in lens))
    off_seg = 2 * a4(N + 1) + a4(2 * n_chunks)
    segs = np.asarray(words[off_seg:off_seg + 8 * N]).reshape(N, 8)
    order = sorted(range(N), key=lambda n: -lens[n])
    assert segs[:, 0].tolist() == order
    assert segs[:, 2].tolist() == [-(-lens[n] // 32) for n in order]
    assert np.all(segs[:, 1] == 0) and np.all(segs[:, 3] == -1) and np.all(segs[:, 4] == -1)
    assert np.all(segs[:, 5:] == 0)


def test_device_bounds_read_back_once(lib, fake):
    bufs = FakeBufs()
    a, _, _ = _valid_args(bufs, T=100, N=3)
    a.cu_seqlens_host = None
    assert _call(lib, fake, a) == _lib.KDA_OK
    kinds = [e[0] for e in fake.log]
    assert kinds.count("d2h") == 1 and kinds.count("stream_sync") == 1
    st = _stats(lib, fake)
    assert st["d2h_reads"] == 1 and st["blocking_syncs"] == 1


def test_capture_miss_is_an_error_and_hit_is_retained(lib, fake):
    bufs = FakeBufs()
    a, _, _ = _valid_args(bufs, T=100, N=3)
    fake.capturing.add(0x20)
    assert _call(lib, fake, a, stream=0x20) == _lib.KDA_ERR_CAPTURE_MISS
    assert fake.launches == []
    # Populate the cache outside capture, then hit it under capture. The hit comes from
    # another stream but joins no event recorded outside the capture.
    assert _call(lib, fake, a, stream=0x10) == _lib.KDA_OK
    fake.complete_all()
    assert _call(lib, fake, a, stream=0x20) == _lib.KDA_OK
    assert [e for e in fake.log if e[0] == "wait"] == []
    # Retained: flood the cache with other bounds; the captured entry must survive.
    for i in range(80):
        b, _, _ = _valid_args(bufs, T=100 + i, N=1, cu=np.array([0, 100 + i], np.int32))
        assert _call(lib, fake, b) == _lib.KDA_OK
        fake.complete_all()
    n_up = [e[0] for e in fake.log].count("h2d")
    assert _call(lib, fake, a, stream=0x20) == _lib.KDA_OK  # still a hit under capture
    assert [e[0] for e in fake.log].count("h2d") == n_up
    # Without host bounds a read-back would have to run under capture: refused.
    a.cu_seqlens_host = None
    assert _call(lib, fake, a, stream=0x20) == _lib.KDA_ERR_CAPTURE_MISS


def test_cross_stream_hit_waits_on_upload(lib, fake):
    bufs = FakeBufs()
    a, _, _ = _valid_args(bufs, T=100, N=3)
    assert _call(lib, fake, a, stream=0x10) == _lib.KDA_OK
    up_ev = [e for e in fake.log if e[0] == "record"][0][1]
    assert _call(lib, fake, a, stream=0x30) == _lib.KDA_OK
    waits = [e for e in fake.log if e[0] == "wait"]
    assert waits == [("wait", 0x30, up_ev)]
    assert fake.syncs() == []


def test_context_creation_makes_one_block_of_each_arena(lib, fake):
    assert sorted(e[0] for e in fake.creation_log) == ["dev_alloc", "host_alloc"]
    st = _stats(lib, fake)
    assert st["arena_device_bytes"] == 4 << 20 and st["arena_host_bytes"] == 4 << 20
    assert st["arena_grows"] == 0


def test_misses_behind_pending_work_neither_wait_nor_allocate(lib, fake):
    """Serving with new bounds every call while the device is still busy: 200 misses whose
    work never completes evict cached buffers (the cache holds 64) and keep every staging
    range, yet no call waits, allocates or frees (aiter PR 6912, Tests)."""
    bufs = FakeBufs()
    for i in range(200):
        b, _, _ = _valid_args(bufs, T=50 + i, N=1, cu=np.array([0, 50 + i], np.int32))
        assert _call(lib, fake, b) == _lib.KDA_OK
    kinds = [e[0] for e in fake.log]
    assert fake.syncs() == []
    assert not {"dev_alloc", "host_alloc", "dev_free", "host_free"} & set(kinds)
    st = _stats(lib, fake)
    assert st["cache_misses"] == 200 and st["blocking_syncs"] == 0 and st["arena_grows"] == 0


def test_arena_ranges_come_back_only_after_their_readers_complete(lib, fake):
    """An evicted metadata buffer and a staging range are reused only once the events of
    the work that reads them have completed; until then new ranges come from elsewhere."""
    bufs = FakeBufs()
    dsts = []
    for i in range(70):  # more than the cache holds: six evictions, nothing completed
        b, _, _ = _valid_args(bufs, T=50 + i, N=1, cu=np.array([0, 50 + i], np.int32))
        assert _call(lib, fake, b) == _lib.KDA_OK
        dsts.append(fake.uploads[-1][0])
    assert len(set(dsts)) == 70  # every upload went to a distinct device range
    fake.complete_all()
    b, _, _ = _valid_args(bufs, T=999, N=1, cu=np.array([0, 999], np.int32))
    assert _call(lib, fake, b) == _lib.KDA_OK
    assert fake.uploads[-1][0] in dsts[:6]  # a range of an evicted, completed buffer
    assert not {"dev_alloc", "dev_free"} & set(e[0] for e in fake.log)


def test_metadata_larger_than_the_arena_adds_a_block(lib, fake):
    """A call whose metadata exceeds the free ranges adds one block to each arena (no
    frees, no waits)."""
    bufs = FakeBufs()
    N = 300_000  # (N + 1) * 2 + chunk table + segment table: about 16 MB of metadata
    cu = np.arange(N + 1, dtype=np.int32) * 2
    a, _, _ = _valid_args(bufs, T=int(cu[-1]), N=N, H=1, cu=cu)
    assert _call(lib, fake, a) == _lib.KDA_OK
    kinds = [e[0] for e in fake.log]
    assert kinds.count("dev_alloc") == 1 and kinds.count("host_alloc") == 1
    assert fake.syncs() == [] and "dev_free" not in kinds
    st = _stats(lib, fake)
    assert st["arena_grows"] == 2 and st["arena_device_bytes"] >= 8 << 20


def test_workspace_too_small_is_rejected_before_any_work(lib, fake):
    bufs = FakeBufs()
    a, _, _ = _valid_args(bufs, T=100, N=3)
    need = lib.kda_chunk_fwd_workspace_bytes(ctypes.byref(a))
    ws = bufs.buf(need - 256)
    assert _call(lib, fake, a, ws=ws) == _lib.KDA_ERR_WORKSPACE
    assert fake.log == [] and fake.launches == []


def test_profiling_hook_reads_and_clears(lib, fake):
    bufs = FakeBufs()
    a, _, _ = _valid_args(bufs, T=100, N=3)
    lib.kda_profile_enable(fake.ctx, 1)
    for _ in range(3):
        assert _call(lib, fake, a) == _lib.KDA_OK
    p, s, n = ctypes.c_double(), ctypes.c_double(), ctypes.c_int64()
    assert lib.kda_profile_read(fake.ctx, ctypes.byref(p), ctypes.byref(s), ctypes.byref(n)) == _lib.KDA_OK
    assert n.value == 3 and p.value == 3.0 and s.value == 3.0
    assert lib.kda_profile_read(fake.ctx, ctypes.byref(p), ctypes.byref(s), ctypes.byref(n)) == _lib.KDA_OK
    assert n.value == 0


def test_validation_rejects_record_walk_beyond_32_bits(lib):
    """One head and one very long sequence: the segmented scan walk of 62 500 chunks would
    span more than 2^31 bytes of records (rejected); 58 594 chunks fit. Validation touches
    no device memory, so the device pointers here are placeholders."""
    a = _lib.FwdArgs()
    a.N, a.H, a.K, a.V = 1, 1, 128, 128
    a.scale, a.lower_bound = 0.088, -5.0
    base = 1 << 44
    for i, name in enumerate(("q", "k", "v", "g_raw", "beta_raw", "out", "cu_seqlens")):
        setattr(a, name, base + (i << 36))  # 16-byte aligned, 64 GiB apart: no overlap
    a.g_dtype = a.beta_dtype = a.state_dtype = _lib.KDA_F32
    for T, want in ((16_000_000, _lib.KDA_ERR_UNSUPPORTED), (15_000_000, _lib.KDA_OK)):
        cu = np.array([0, T], np.int32)
        a.T = T
        a.cu_seqlens_host = cu.ctypes.data
        assert lib.kda_seg_len(1, 1, -(-T // 32), 0) > 0
        assert lib.kda_chunk_fwd_validate(ctypes.byref(a)) == want, T


def test_noalloc_entry_point_needs_a_device_context(lib, fake):
    """The allocation-free call uses the device's fixed array, which a context made on a
    stand-in runtime does not have: refused before any work."""
    bufs = FakeBufs()
    a, _, _ = _valid_args(bufs, T=100, N=3)
    assert lib.kda_chunk_fwd_noalloc(fake.ctx, ctypes.byref(a), 0x10) == _lib.KDA_ERR_UNSUPPORTED
    assert lib.kda_chunk_fwd_noalloc(None, ctypes.byref(a), 0x10) == _lib.KDA_ERR_INVALID_ARG
    assert fake.log == [] and fake.launches == []
    assert lib.kda_noalloc_scratch_bytes() == 64 << 20


def test_miss_enqueues_no_separate_event_marker(lib, fake):
    """A metadata miss enqueues the upload, whose completion the copy records itself, and
    the launches: no event is recorded as a separate marker in the stream (each marker costs
    the GPU several microseconds of idle time)."""
    bufs = FakeBufs()
    for i in range(3):
        a, _, _ = _valid_args(bufs, T=300 + i, N=4, cu=np.array([0, 0, 100, 100, 300 + i], np.int32), paged=True)
        assert _call(lib, fake, a) == _lib.KDA_OK
    assert getattr(fake, "marker_records", 0) == 0
    assert [e[0] for e in fake.log].count("h2d") == 3
    assert _stats(lib, fake)["cache_misses"] == 3
