"""Full-size GPU checks against closed forms, on every row of every head.

With Q = K = 0 every score is 0, so over the keys a causal row may see every
probability is 1 / (number of those keys), whatever the ring order, the tiling
or the running maximum ("Ring Attention" (aarnphm.xyz), the recurrence for m, z,
y; O = y / z).  With V = 1 the output is then exactly 1, and the log-sum-exp is
ln(count), where count = t + 1 for a row at global position t (the causal
predicate of the pages: a key is visible when its position is at most the
query's).  The same launches as the bench's named workloads run, at their full
sizes, so these checks cover every row, including the rows the sampled parity
checks skip, through every tile path of the step kernel (full tiles, the masked
diagonal, the carried state, the hop copies, the epilogue).

The backward with dO = 1 (and the forward's own O, LSE) has closed forms too
(the backward ring of the transformer-math page (aicassindra.com)): dP = dO V^T
= d and D = rowsum(dO * O) = d, so dS = P (dP - D) = 0 and dQ = dK = 0
exactly; dV of a key is the sum over the rows that see it of P = 1 / count,
times the G query heads of its key/value head, in every column.
"""

from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import oracle
import ring_attention_block_step_amd as ra
import workloads as wl

pytestmark = pytest.mark.gpu

FORWARD = ["1m-contiguous-causal", "1m-zigzag-causal", "128k-contiguous-causal", "32k-striped-causal",
           "32k-zigzag-causal"]


def _constant_shards(w, dev="cuda"):
    q = torch.zeros((w.b, w.Hq, w.d), dtype=torch.bfloat16, device=dev)
    k = torch.zeros((w.P, w.b, w.Hkv, w.d), dtype=torch.bfloat16, device=dev)
    v = torch.ones((w.P, w.b, w.Hkv, w.d), dtype=torch.bfloat16, device=dev)
    return q, k, v


@pytest.mark.parametrize("name", FORWARD)
def test_forward_constant_operands_every_row(name):
    w = wl.WORKLOADS[name]
    rank = w.ranks[-1]
    q, k, v = _constant_shards(w)
    print(f"[gpu] closed form forward {name} rank={rank} b={w.b} Hq={w.Hq}", flush=True)
    out, lse = ra.forward(q, k, v, P=w.P, rank=rank, causal=w.causal, layout=w.layout)
    torch.cuda.synchronize()
    assert torch.all(out == 1), "O must be exactly 1 on every row"
    count = oracle.shard_positions(w.layout, rank, w.P, w.b).astype(np.float64) + 1.0
    want = np.log(count)[None, :]
    got = lse.cpu().numpy().astype(np.float64)
    err = np.abs(got - want)
    # LSE = (m + log2 z) ln 2 in fp32 with m = 0 and z an exact integer: about
    # 2e-6 at ln z ~ 14 (an ulp of log2 z, plus the product's rounding).  The
    # bound 6e-6 resolves one key too many or too few (ln(c + 1) - ln c ~ 1/c)
    # up to c ~ 1.6e5; beyond that such an error is below what the fp32 LSE
    # can show, and the sampled parity tests with random data cover it.
    print(f"[gpu]   lse max error {err.max():.3e}", flush=True)
    assert err.max() <= 6e-6, err.max()


BACKWARD = ["32k-contiguous-causal", "32k-striped-causal", "32k-zigzag-causal", "128k-contiguous-causal"]


@pytest.mark.parametrize("name", BACKWARD)
def test_backward_constant_operands_closed_form(name):
    w = wl.WORKLOADS[name]
    rank = w.ranks[-1]
    q, k, v = _constant_shards(w)
    do = torch.ones((w.b, w.Hq, w.d), dtype=torch.bfloat16, device="cuda")
    print(f"[gpu] closed form backward {name} rank={rank} b={w.b} Hq={w.Hq}", flush=True)
    out, lse = ra.forward(q, k, v, P=w.P, rank=rank, causal=w.causal, layout=w.layout)
    dq, dk, dv = ra.backward(q, k, v, out, lse, do, P=w.P, rank=rank, causal=w.causal, layout=w.layout)
    torch.cuda.synchronize()
    assert torch.all(out == 1)
    assert torch.all(dq == 0), "dS = 0, so dQ must be exactly 0"
    assert torch.all(dk == 0), "dS = 0, so dK must be exactly 0"

    # Each row's probability as the kernels form it: P = exp2(-LSE log2 e) in
    # fp32, rounded to bf16 as the MFMA operand of dV = P^T dO.
    lse_h = lse[0].float()
    p = torch.exp2(-(lse_h * math.log2(math.e))).to(torch.bfloat16).double().cpu().numpy()
    assert torch.all(lse == lse[0:1]), "every head has the same LSE when Q = 0"
    tq = oracle.shard_positions(w.layout, rank, w.P, w.b)
    order = np.argsort(tq)
    tq_sorted = tq[order]
    p_sorted = np.concatenate([p[order], [0.0]])
    suffix = np.concatenate([np.cumsum(p[order][::-1])[::-1], [0.0]])   # sum of p over rows with tq >= a bound
    G = w.Hq // w.Hkv
    got = dv.double().cpu().numpy()          # [P, b, Hkv, d]
    assert np.all(got == got[..., :1]), "every column of dV is the same"
    for r in range(w.P):
        tk = oracle.shard_positions(w.layout, r, w.P, w.b)
        first = np.searchsorted(tq_sorted, tk, side="left")   # rows with tq >= tk see key tk
        want = G * suffix[first]                               # [b]
        g = got[r, :, :, 0]                                    # [b, Hkv]
        seen = want > 0
        assert np.all(g[~seen] == 0), f"shard {r}: keys no row sees must get dV = 0"
        # Bound: fp32 accumulation of positive terms in another order (~1e-6
        # relative, 2e-5 allowed), plus two bf16 roundings of P taken the other
        # way (the host's exp2 and the GPU's may differ by an fp32 ulp next to
        # a rounding tie), each 2^-8 of the largest term, that of the first row
        # to see the key.  A row too many or too few near the diagonal, where
        # the terms are alike, moves the entry by a whole term.
        tol = 2e-5 * want + G * 2.0 ** -7 * p_sorted[first]
        excess = np.abs(g - want[:, None]) - tol[:, None]
        assert excess[seen].max() <= 0, (r, excess[seen].max())
