"""Stored expected values: the chunk numbering of bounds with empty sequences before
non-empty ones, worked out by hand (tests/golden/, with its citation), against the
oracle's chunk table and the library's host function."""
import ctypes
import os

import numpy as np

from gated_delta_rule_pack_amd import _lib
from oracle import chunk_indices

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _read(name):
    chunk, cu, pairs = None, None, []
    for line in open(os.path.join(GOLDEN, name)):
        line = line.split("#")[0].strip()
        if not line:
            continue
        if line.startswith("chunk"):
            chunk = int(line.split()[1])
        elif line.startswith("cu_seqlens"):
            cu = np.array([int(x) for x in line.split()[1:]], np.int32)
        else:
            pairs.append([int(x) for x in line.split()])
    return chunk, cu, np.array(pairs, np.int32)


def test_chunk_indices_with_empty_sequences_match_hand_values():
    chunk, cu, want = _read("chunk_indices_empty_before_nonempty.txt")
    assert np.array_equal(chunk_indices(cu, chunk), want)
    lib = _lib.load()
    out = np.zeros(2 * len(want), np.int32)
    n = ctypes.c_int64()
    rc = lib.kda_prepare_chunk_indices(cu.ctypes.data, len(cu) - 1, chunk, out.ctypes.data, len(want), ctypes.byref(n))
    assert rc == _lib.KDA_OK and n.value == len(want)
    assert np.array_equal(out.reshape(-1, 2), want)
