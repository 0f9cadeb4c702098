"""A shape whose byte offsets pass 2^31: 64 heads x 131 072 tokens in two sequences, so q,
k, v and out hold 2 GiB each and the chunk records 9.3 GB. Inputs are drawn on the GPU
from a seeded generator (same distributions as the standard workloads); the first and
last head of the second sequence, whose token offsets are the largest, are copied back
and checked against the fp64 oracle, output rows and final state."""
import numpy as np
import pytest
import torch

import gated_delta_rule_pack_amd as kda
from oracle import kda_forward
from tests.kda_harness import OUT_TOL, STATE_TOL_F32, rel_l2

pytestmark = pytest.mark.gpu


def test_offsets_beyond_2_31_bytes():
    T, H, D = 131072, 64, 128
    lens = [65536 + 100, 65536 - 100]
    dev = torch.device("cuda", 0)
    gen = torch.Generator(device=dev).manual_seed(91)
    rnd = lambda shape, std=1.0: torch.randn(shape, generator=gen, device=dev) * std
    q = rnd((1, T, H, D)).to(torch.bfloat16)
    k = rnd((1, T, H, D)).to(torch.bfloat16)
    v = rnd((1, T, H, D)).to(torch.bfloat16)
    g = rnd((1, T, H, D))
    b = rnd((1, T, H))
    pool = rnd((4, H, D, D), 0.1)
    pool0 = pool.clone()
    cu_h = torch.tensor([0, lens[0], T], dtype=torch.int32)
    idx = torch.tensor([2, 1], dtype=torch.int32, device=dev)
    flags = torch.ones(2, dtype=torch.bool, device=dev)
    print(f"case T={T} H={H}: q bytes {q.numel() * 2}", flush=True)
    out, _ = kda.chunk_fwd(q, k, v, g, b, cu_h.to(dev), cu_seqlens_cpu=cu_h, scale=D ** -0.5, lower_bound=-5.0,
                           state_cache=pool, state_indices=idx, has_initial_state=flags)
    torch.cuda.synchronize()
    t0, t1 = lens[0], T
    heads = [0, H - 1]
    f64 = lambda x: x.detach().to("cpu").to(torch.float64).numpy()
    sl = lambda x: f64(x[0, t0:t1][:, heads])
    ref_out, ref_fin = kda_forward(sl(q), sl(k), sl(v), sl(g), f64(b[0, t0:t1][:, heads]), [0, t1 - t0],
                                   scale=D ** -0.5, lower_bound=-5.0,
                                   initial_state=f64(pool0[1][heads])[None])
    got_out = sl(out)
    got_fin = f64(pool[1][heads])
    e_out, e_state = rel_l2(got_out, ref_out), rel_l2(got_fin, ref_fin[0])
    print(f"  heads {heads} of sequence 1: out {e_out:.3e} state {e_state:.3e}", flush=True)
    assert np.all(np.isfinite(got_out))
    assert e_out <= OUT_TOL and e_state <= STATE_TOL_F32
    # Slots not addressed by the call keep their bits.
    assert torch.equal(pool[0], pool0[0]) and torch.equal(pool[3], pool0[3])
