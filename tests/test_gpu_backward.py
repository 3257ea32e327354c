"""GPU parity of the backward ring (ringattn_backward) against the fp64 oracle.

Inputs are seeded and synthetic: Q, K, V and the upstream gradient dO in
bf16; the forward's O and LSE come from the oracle (rounded to bf16 and
fp32), and both sides read the same rounded values.  Compared: dQ of the
rank's rows, and the rank's contributions to every shard's dK and dV.

Bound.  The kernels read bf16 inputs and round P and dS to bf16 only as MFMA
operands, accumulating in fp32.  A bf16 rounding moves a value by at most half
an ulp, 2^-8 of it, so each gradient entry, a sum of products with one rounded
factor, is off by at most 2^-8 of the sum of its terms' magnitudes; with few
terms (a row or key that sees few partners) nothing averages out.  The bound:
mean-abs error <= 2^-8 of the tensor's mean magnitude, max-abs error
<= 1e-2 (about 2.5 half-ulps) of its largest magnitude, and, entry by entry,
relative error <= 2^-5 on every entry of at least a tenth of the largest
magnitude.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import ring_attention_block_step_amd as ra
import workloads as wl

pytestmark = pytest.mark.gpu

REL_MAX = 1e-2
REL_MEAN = 2.0 ** -8


def _inputs(N, P, Hq, Hkv, d, seed, k_scale=1.0):
    k = wl.token_range(seed, "k", 0, N, Hkv, d, "normal", k_scale, torch.bfloat16)
    v = wl.token_range(seed, "v", 0, N, Hkv, d, "normal", 1.0, torch.bfloat16)
    q = wl.token_range(seed, "q", 0, N, Hq, d, "normal", 1.0, torch.bfloat16)
    do = wl.token_range(seed, "do", 0, N, Hq, d, "normal", 1.0, torch.bfloat16)
    return q, k, v, do


# Entries at least BIG_FRAC of the largest magnitude are also checked one by
# one: relative error at most 2^-5, eight bf16 half-ulps (2^-8 each), the
# format P and dS are rounded to as MFMA operands.  (The max-abs bound above allows 10% on
# such an entry; over every case here the worst is about 2%.)
BIG_FRAC = 0.1
REL_BIG = 2.0 ** -5


def _stats(got, want):
    err = np.abs(got - want)
    aw = np.abs(want)
    top = float(aw.max()) if aw.size else 0.0
    big = (aw >= BIG_FRAC * top) & (aw > 0)
    rel_big = float((err[big] / aw[big]).max()) if big.any() else 0.0
    return {"max_abs": float(err.max()), "max_ref": float(aw.max()),
            "mean_abs": float(err.mean()), "mean_ref": float(aw.mean()),
            "rel_big": rel_big, "n_big": int(big.sum())}


def _check(name, got, want, label):
    s = _stats(got, want)
    print(f"[gpu] backward {label} {name}: {s}", flush=True)
    assert s["max_abs"] <= REL_MAX * s["max_ref"] + 1e-6, (label, name, s)
    assert s["mean_abs"] <= REL_MEAN * s["mean_ref"] + 1e-7, (label, name, s)
    assert s["rel_big"] <= REL_BIG, (label, name, s)


def _run_rank(q, k, v, do, N, P, u, layout, causal, Hq, Hkv, d, dk=None, dv=None):
    """Oracle forward for rank u (rounded), GPU backward and oracle backward."""
    b = N // P
    tq = oracle.shard_positions(layout, u, P, b)
    q64, k64, v64, do64 = (t.double().numpy() for t in (q, k, v, do))
    o, lse = oracle.ring_forward(q64[tq], u, k64, v64, P, layout, causal)
    o16 = torch.tensor(o).to(torch.bfloat16)
    lse32 = torch.tensor(lse).to(torch.float32)
    kp = ra.pack_shards(k, P, layout).cuda()
    vp = ra.pack_shards(v, P, layout).cuda()
    gq, gk, gv = ra.backward(q[tq].cuda(), kp, vp, o16.cuda(), lse32.cuda(), do[tq].cuda(), P=P, rank=u,
                             causal=causal, layout=layout, dk=dk, dv=dv)
    torch.cuda.synchronize()
    wq, wk, wv = oracle.ring_backward(q64[tq], u, k64, v64, o16.double().numpy(), lse32.double().numpy(),
                                      do64[tq], P, layout, causal)
    return (gq, gk, gv), (wq, wk, wv)


CASES = [
    # name, N, P, ranks, layout, causal, Hq, Hkv, d
    ("ragged-contig-causal", 800, 4, (0, 1, 2, 3), "contiguous", True, 4, 2, 128),
    ("striped-causal-d64", 1024, 4, (0, 3), "striped", True, 4, 2, 64),
    ("zigzag-causal", 800, 4, (0, 1, 2, 3), "zigzag", True, 4, 2, 128),
    ("contig-noncausal", 512, 2, (0, 1), "contiguous", False, 2, 1, 128),
    ("p1-causal-gqa4", 333, 1, (0,), "contiguous", True, 4, 1, 128),
    ("b1-striped", 8, 8, (0, 5), "striped", True, 2, 1, 128),
    ("gqa8-striped-p8", 2048, 8, (2, 7), "striped", True, 8, 1, 128),
]


@pytest.mark.parametrize("name,N,P,ranks,layout,causal,Hq,Hkv,d", CASES, ids=[c[0] for c in CASES])
def test_backward_matches_oracle(name, N, P, ranks, layout, causal, Hq, Hkv, d):
    q, k, v, do = _inputs(N, P, Hq, Hkv, d, seed=N + P)
    for u in ranks:
        (gq, gk, gv), (wq, wk, wv) = _run_rank(q, k, v, do, N, P, u, layout, causal, Hq, Hkv, d)
        label = f"{name} rank {u}"
        _check("dq", gq.cpu().double().numpy(), wq, label)
        _check("dk", gk.cpu().double().numpy(), wk, label)
        _check("dv", gv.cpu().double().numpy(), wv, label)


def test_backward_all_ranks_accumulate_to_dense_gradient():
    """dK and dV accumulated over every rank's call equal the dense gradient;
    every rank's dQ equals the dense dQ of its rows."""
    N, P, Hq, Hkv, d, layout = 1024, 4, 4, 2, 128, "contiguous"
    q, k, v, do = _inputs(N, P, Hq, Hkv, d, seed=99)
    b = N // P
    dk = torch.zeros(P, b, Hkv, d, device="cuda")
    dv = torch.zeros(P, b, Hkv, d, device="cuda")
    dq = np.zeros((N, Hq, d))
    q64, k64, v64, do64 = (t.double().numpy() for t in (q, k, v, do))
    for u in range(P):
        (gq, _, _), _ = _run_rank(q, k, v, do, N, P, u, layout, True, Hq, Hkv, d, dk=dk, dv=dv)
        dq[oracle.shard_positions(layout, u, P, b)] = gq.cpu().double().numpy()
    # forward O is rounded to bf16 on the GPU side; the dense reference uses exact O
    wq, wk, wv = oracle.backward_dense(q64, np.arange(N), k64, v64, do64, True)
    gk = np.zeros((N, Hkv, d))
    gv = np.zeros((N, Hkv, d))
    for r in range(P):
        tk = oracle.shard_positions(layout, r, P, b)
        gk[tk] = dk[r].cpu().double().numpy()
        gv[tk] = dv[r].cpu().double().numpy()
    _check("dq", dq, wq, "all ranks")
    _check("dk", gk, wk, "all ranks")
    _check("dv", gv, wv, "all ranks")


def test_backward_medium_all_rows():
    """8k tokens, 8 shards of 1024 rows, GQA 8/2, every row of rank 5."""
    N, P, Hq, Hkv, d = 8192, 8, 8, 2, 128
    q, k, v, do = _inputs(N, P, Hq, Hkv, d, seed=123, k_scale=2.0)
    (gq, gk, gv), (wq, wk, wv) = _run_rank(q, k, v, do, N, P, 5, "contiguous", True, Hq, Hkv, d)
    _check("dq", gq.cpu().double().numpy(), wq, "medium rank 5")
    _check("dk", gk.cpu().double().numpy(), wk, "medium rank 5")
    _check("dv", gv.cpu().double().numpy(), wv, "medium rank 5")


@pytest.mark.parametrize("N,P,rank,Hq,Hkv,d,layout", [
    (1024, 4, 3, 4, 2, 128, "contiguous"),
    (1000, 4, 1, 4, 2, 64, "zigzag"),      # ragged b = 250: the last key tile is partial
    (16384, 8, 5, 8, 1, 128, "striped"),   # GQA 8/1, b = 2048: two hop units per dK/dV workgroup
])
def test_backward_hop_modes_are_bit_identical(N, P, rank, Hq, Hkv, d, layout):
    """The dQ workgroups' double buffer must not race in any hop schedule: the
    copies made by the dK/dV workgroups of each visit launch (beside the dQ
    workgroups reading the other slot), serialised on the caller stream, or
    on the second stream give bit-identical gradients (O and LSE from the GPU
    forward)."""
    q, k, v, do = _inputs(N, P, Hq, Hkv, d, seed=7)
    b = N // P
    tq = torch.as_tensor(oracle.shard_positions(layout, rank, P, b))
    kp = ra.pack_shards(k, P, layout).cuda()
    vp = ra.pack_shards(v, P, layout).cuda()
    qr, dor = q[tq].cuda(), do[tq].cuda()
    out, lse = ra.forward(qr, kp, vp, P=P, rank=rank, causal=True, layout=layout)
    res = []
    try:
        for mode in ("fused", "serial", "streams", "fused"):
            ra.set_hop_mode(mode)
            g = ra.backward(qr, kp, vp, out, lse, dor, P=P, rank=rank, causal=True, layout=layout)
            torch.cuda.synchronize()
            res.append(tuple(t.cpu() for t in g))
    finally:
        ra.set_hop_mode("fused")
    for other in res[1:]:
        for a, b_ in zip(res[0], other):
            assert torch.equal(a, b_)


@pytest.mark.parametrize("name", ["32k-contiguous-causal", "128k-contiguous-causal"])
def test_backward_full_size_sampled(name):
    """The workload's full share in the launch configuration the bench times
    (rank 7 of 8 contiguous shards, 32/8 GQA, d 128), checked on sampled
    entries: dQ of 64 local rows (0, 1, b-1 among them) and the rank's dK, dV
    contributions to 48 keys of the diagonal shard 7 and of shards 0 and 3.

    O and LSE are synthetic inputs rather than a forward's: LSE of a row at
    global token t is ln(t + 1) + 1/2, the log-partition of unit-variance
    scores over its t + 1 keys, and O is seeded N(0, 0.05^2).  The backward's
    formulas hold for any such inputs, and both sides read the same values;
    an exact forward of every row on the CPU would take minutes at 128k.
    """
    w = wl.WORKLOADS[name]
    rank = w.ranks[-1]
    b = w.b
    tq = oracle.shard_positions(w.layout, rank, w.P, b)
    k_glob, v_glob = wl.global_kv(w)
    q = wl.query_rows(w, tq)
    do = wl.token_rows(w.seed, "do", tq, w.Hq, w.d, "normal", 1.0, torch.bfloat16)
    out = wl.token_rows(w.seed, "o", tq, w.Hq, w.d, "normal", 0.05, torch.bfloat16)
    lse_row = np.log(tq.astype(np.float64) + 1.0) + 0.5
    lse = torch.tensor(np.broadcast_to(lse_row, (w.Hq, b)).copy(), dtype=torch.float32)
    print(f"[gpu] backward full size {name}: inputs ready", flush=True)

    kp = ra.pack_shards(k_glob, w.P, w.layout).cuda()
    vp = ra.pack_shards(v_glob, w.P, w.layout).cuda()
    dk = torch.zeros(kp.shape, dtype=torch.float32, device="cuda")
    dv = torch.zeros(kp.shape, dtype=torch.float32, device="cuda")
    gq, gk, gv = ra.backward(q.cuda(), kp, vp, out.cuda(), lse.cuda(), do.cuda(), P=w.P, rank=rank,
                             causal=w.causal, layout=w.layout, dk=dk, dv=dv)
    torch.cuda.synchronize()
    del kp, vp

    rows = wl.sample_local_rows(b, 64, w.seed, 0)
    keys = [(r, int(j)) for r in (7, 0, 3) for j in wl.sample_local_rows(b, 16, w.seed + r, 1)]
    wq, wk, wv = oracle.backward_sampled(q.double().numpy(), rank, k_glob.double().numpy(),
                                         v_glob.double().numpy(), out.double().numpy(),
                                         lse.double().numpy(), do.double().numpy(), w.P, w.layout,
                                         w.causal, rows, keys)
    ridx = torch.as_tensor(rows)
    got_q = gq[ridx].cpu().double().numpy()
    got_k = np.stack([gk[r, j].cpu().double().numpy() for r, j in keys])
    got_v = np.stack([gv[r, j].cpu().double().numpy() for r, j in keys])
    _check("dq", got_q, wq, name)
    _check("dk", got_k, wk, name)
    _check("dv", got_v, wv, name)

