"""Host-side pieces of bench.py: the per-launch byte and flop counts, the refusal of more
than one GPU, and that the committed traffic summaries match the kernel sources. No GPU
is touched."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from gated_delta_rule_pack_amd.workloads import standard  # noqa: E402


def test_decode_bytes_are_tokens_plus_state():
    wl = standard("paged_256x1_H12_bf16")
    # Per token-head q, k, v (3 x 256 B), fp32 raw gate (512 B), fp32 raw beta (4 B) and
    # 256 B of output; every sequence-head reads and writes a 128 x 128 bf16 state.
    tokens = 256 * 12 * (3 * 256 + 512 + 4 + 256)
    state = 2 * 256 * 12 * 128 * 128 * 2
    assert bench.kernel_bytes(wl, "decode", 256) == tokens + state == 206_057_472
    assert bench.kernel_bytes(wl, "call", 256) == tokens + state


def test_4k_call_flops():
    wl = standard("paged_1x4096_H12")
    # 139 264 flops per token-head: 32 768 in the chunk-local products, 106 496 in the scan.
    assert bench.algorithmic_flops(wl, "call") == 4096 * 12 * 139_264
    assert bench.algorithmic_flops(wl, "prep") + bench.algorithmic_flops(wl, "scan") == \
        bench.algorithmic_flops(wl, "call")


def test_scan_bytes_count_records_output_and_state():
    wl = standard("paged_1x4096_H12")
    n_chunks = 128
    want = n_chunks * 12 * bench.RECORD_BYTES + 4096 * 12 * 256 + 2 * 12 * 128 * 128 * 4
    assert bench.kernel_bytes(wl, "scan", n_chunks) == want


@pytest.mark.parametrize("gpus", ["2", "8"])
def test_more_than_one_gpu_is_refused(gpus):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", gpus],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_grouped_heads_read_fewer_qk_bytes():
    # 12 value heads share 6 q/k heads: q and k move 256 B per token-head instead of 512.
    g = standard("paged_1x4096_H12_qk6")
    f = standard("paged_1x4096_H12")
    assert g.H == f.H == 12 and g.H_qk == 6
    th = 4096 * 12
    assert bench.kernel_bytes(f, "call", 128) - bench.kernel_bytes(g, "call", 128) == th * 256
    assert bench.kernel_bytes(f, "scan", 128) == bench.kernel_bytes(g, "scan", 128)


def test_committed_traffic_profiles_match_the_kernel_sources():
    """Every committed HBM-traffic summary was taken from the kernel sources as they are
    now (the bench reports traffic only from a matching summary)."""
    import glob
    import os
    import re
    files = sorted(glob.glob(os.path.join(bench.ROOT, "profiles", "kda_*_traffic_*.txt")))
    assert files
    for path in files:
        kernel = os.path.basename(path)[len("kda_"):].split("_traffic_")[0]
        m = re.search(r"source_sha256_16:\s*([0-9a-f]+)", open(path).read())
        assert m, path
        assert m.group(1) == bench.kernel_source_hash(kernel), f"{path} was taken from other {kernel} sources"
