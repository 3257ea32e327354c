"""The allocation-free decode entry point (ringattn_decode_partial_noalloc)
against ringattn_decode_partial: same kernels, so the partial triples must be
bit-identical, on two calls in a row, the second with a smaller input (the
static scratch keeps the first call's partials; the second must not read
them).  Both also match the fp64 oracle's decode partial within the decode
tests' bound (O = y/z and LSE = m + ln z within 1e-4)."""

from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import ring_attention_block_step_amd as ra
import workloads as wl

pytestmark = pytest.mark.gpu


def _finish(m, z, y):
    m, z, y = (np.asarray(t, dtype=np.float64) for t in (m, z, y))
    has = z > 0
    zs = np.where(has, z, 1.0)
    o = np.where(has.T[:, :, None], y / zs.T[:, :, None], 0.0)
    lse = np.where(has, m + np.log(zs), -np.inf)
    return o, lse


def _case(n_keys, n_q, Hq, Hkv, d, seed):
    q = wl.token_range(seed, "q", 10 ** 6, 10 ** 6 + n_q, Hq, d, "normal", 1.0, torch.bfloat16)
    k = wl.token_range(seed, "k", 0, n_keys, Hkv, d, "normal", 1.0, torch.bfloat16)
    v = wl.token_range(seed, "v", 0, n_keys, Hkv, d, "normal", 1.0, torch.bfloat16)
    return q, k, v


# First the 31k-token shard with 64/8 heads (4.1 MB of scratch), then a smaller
# ragged shard with d 64 and three new tokens.
CASES = [(31250, 1, 64, 8, 128, 8), (5000, 3, 8, 2, 64, 21)]


def test_noalloc_decode_matches_decode_partial_twice_in_a_row():
    for n_keys, n_q, Hq, Hkv, d, seed in CASES:
        print(f"[gpu] noalloc decode n_keys={n_keys} n_q={n_q} Hq={Hq} Hkv={Hkv} d={d}", flush=True)
        q, k, v = (t.cuda() for t in _case(n_keys, n_q, Hq, Hkv, d, seed))
        ref = ra.decode_partial(q, k, v)
        got = ra.decode_partial_noalloc(q, k, v)
        torch.cuda.synchronize()
        for a, b, name in zip(got, ref, ("m", "z", "y")):
            assert torch.equal(a, b), name
        wm, wz, wy = oracle.decode_partial(q.cpu().double().numpy(), k.cpu().double().numpy(),
                                           v.cpu().double().numpy())
        o, lse = _finish(*(t.cpu().numpy() for t in got))
        wo, wlse = _finish(wm, wz, wy)
        print(f"[gpu]   O max-abs {np.abs(o - wo).max():.3e}, LSE max-abs {np.abs(lse - wlse).max():.3e}",
              flush=True)
        assert np.abs(o - wo).max() <= 1e-4 and np.abs(lse - wlse).max() <= 1e-4


def test_noalloc_decode_empty_shard_gives_the_merge_identity():
    q = torch.randn(2, 4, 128).to(torch.bfloat16).cuda()
    empty = torch.empty(0, 1, 128, dtype=torch.bfloat16, device="cuda")
    m, z, y = ra.decode_partial_noalloc(q, empty, empty)
    torch.cuda.synchronize()
    assert torch.isinf(m).all() and (m < 0).all() and (z == 0).all() and (y == 0).all()
