"""GPU parity of pass-Q decode (ringattn_decode_partial, then ringattn_merge)
against the fp64 oracle.

The partial triple of a shard is not unique (any common reference for m
cancels), so the comparison is on what is: O_p = y / z and LSE_p = m + ln z
per shard, and O, LSE after the merge.  Bound: the inputs are bf16 (exact in
fp32); the scores are bf16 products accumulated in fp32 on the matrix cores,
the probabilities and their sums are fp32, and each probability enters the
p*V product as two bf16 terms (its rounding and the rounding of the
remainder, a relative error below 2^-17), so the error is fp32 rounding over
at most 2^17 keys: O and LSE within 1e-4 absolute.  The
merged O is written in fp32 here and in bf16 once, where the stated bf16
bounds apply (max-abs 1e-2, mean-abs 1e-3).
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import ring_attention_block_step_amd as ra
import workloads as wl

pytestmark = pytest.mark.gpu

TOL_O = 1e-4
TOL_LSE = 1e-4


def _finish(m, z, y):
    """O = y / z [n_q, Hq, d] and LSE = m + ln z [Hq, n_q] of a triple (numpy)."""
    m, z, y = (np.asarray(t, dtype=np.float64) for t in (m, z, y))
    has = z > 0
    zs = np.where(has, z, 1.0)
    o = np.where(has.T[:, :, None], y / zs.T[:, :, None], 0.0)
    lse = np.where(has, m + np.log(zs), -np.inf)
    return o, lse


def _run_shard(q, k, v):
    m, z, y = ra.decode_partial(q.cuda(), k.cuda(), v.cuda())
    torch.cuda.synchronize()
    return m.cpu().numpy(), z.cpu().numpy(), y.cpu().numpy()


def _check_shard(q, k, v, label):
    m, z, y = _run_shard(q, k, v)
    wm, wz, wy = oracle.decode_partial(q.double().numpy(), k.double().numpy(), v.double().numpy())
    o, lse = _finish(m, z, y)
    wo, wlse = _finish(wm, wz, wy)
    err_o = float(np.abs(o - wo).max()) if o.size else 0.0
    same_inf = np.array_equal(np.isinf(lse), np.isinf(wlse))
    fin = np.isfinite(wlse)
    err_l = float(np.abs(lse[fin] - wlse[fin]).max()) if fin.any() else 0.0
    print(f"[gpu] decode {label}: O max-abs {err_o:.3e}, LSE max-abs {err_l:.3e}", flush=True)
    assert same_inf, label
    assert err_o <= TOL_O, label
    assert err_l <= TOL_LSE, label
    return m, z, y


SHAPES = [
    # n_q, Hq, Hkv, d, n_keys, k_scale
    (1, 4, 1, 128, 1000, 1.0),     # ragged last chunk
    (3, 8, 2, 64, 777, 2.0),       # d 64, 12 rows per key/value head
    (5, 32, 8, 128, 300, 1.0),     # 20 rows, a chunk with empty waves
    (5, 64, 8, 128, 2000, 1.0),    # 40 rows: two row blocks of 32
    (2, 2, 2, 128, 1, 1.0),        # one key
    (1, 16, 1, 128, 4096, 3.0),    # 16 rows, wide score spread
    (4, 4, 4, 64, 256, 1.0),       # exactly one chunk
]


@pytest.mark.parametrize("n_q,Hq,Hkv,d,n_keys,k_scale", SHAPES)
def test_decode_partial_matches_oracle(n_q, Hq, Hkv, d, n_keys, k_scale):
    g = torch.Generator().manual_seed(n_q * 1000 + n_keys)
    q = torch.randn(n_q, Hq, d, generator=g).to(torch.bfloat16)
    k = (torch.randn(n_keys, Hkv, d, generator=g) * k_scale).to(torch.bfloat16)
    v = torch.randn(n_keys, Hkv, d, generator=g).to(torch.bfloat16)
    _check_shard(q, k, v, f"n_q={n_q} Hq={Hq} Hkv={Hkv} d={d} n_keys={n_keys}")


def test_decode_partial_of_empty_shard():
    q = torch.randn(2, 4, 128).to(torch.bfloat16).cuda()
    e = torch.empty(0, 2, 128, dtype=torch.bfloat16, device="cuda")
    m, z, y = ra.decode_partial(q, e, e)
    torch.cuda.synchronize()
    assert torch.all(torch.isinf(m) & (m < 0)) and torch.all(z == 0) and torch.all(y == 0)


@pytest.mark.parametrize("name", ["decode-1m-shard", "decode-31k-gqa64"])
def test_decode_workload_shards_and_merge_equal_dense(name):
    """Every shard's partial written in place into merge's inputs, merged on
    the GPU, equals dense attention of the new token over the whole cache;
    the first and last shard's partials are also checked one by one."""
    w = wl.DECODE_WORKLOADS[name]
    q = wl.decode_query(w)
    qd = q.cuda()
    m = torch.empty(w.P, w.Hq, w.n_q, device="cuda")
    z = torch.empty_like(m)
    y = torch.empty(w.P, w.n_q, w.Hq, w.d, device="cuda")
    ks, vs = [], []
    for p in range(w.P):
        k, v = wl.decode_shard(w, p)
        ks.append(k)
        vs.append(v)
        ra.decode_partial(qd, k.cuda(), v.cuda(), m=m[p], z=z[p], y=y[p])
    for p in (0, w.P - 1):
        _check_shard(q, ks[p], vs[p], f"{name} shard {p}")
    out32, lse = ra.merge(m, z, y, out_dtype=torch.float32)
    out16, _ = ra.merge(m, z, y, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    k_all = torch.cat(ks).double().numpy()
    v_all = torch.cat(vs).double().numpy()
    want_o, want_lse = oracle.dense_attention(q.double().numpy(), np.full(w.n_q, w.N), k_all, v_all, True)
    e32 = np.abs(out32.cpu().double().numpy() - want_o)
    e16 = np.abs(out16.float().cpu().double().numpy() - want_o)
    el = np.abs(lse.cpu().double().numpy() - want_lse)
    print(f"[gpu] decode {name} merged: fp32 O max-abs {e32.max():.3e}, LSE {el.max():.3e}, "
          f"bf16 O max-abs {e16.max():.3e} mean {e16.mean():.3e}", flush=True)
    assert e32.max() <= TOL_O and el.max() <= TOL_LSE
    assert e16.max() <= 1e-2 and e16.mean() <= 1e-3


def test_decode_ragged_shards_with_an_empty_one_merge_to_dense():
    g = torch.Generator().manual_seed(77)
    sizes = [700, 0, 1500, 33]
    Hq, Hkv, d, n_q = 8, 2, 128, 2
    q = torch.randn(n_q, Hq, d, generator=g).to(torch.bfloat16)
    N = sum(sizes)
    k_all = torch.randn(N, Hkv, d, generator=g).to(torch.bfloat16)
    v_all = torch.randn(N, Hkv, d, generator=g).to(torch.bfloat16)
    P = len(sizes)
    m = torch.empty(P, Hq, n_q, device="cuda")
    z = torch.empty_like(m)
    y = torch.empty(P, n_q, Hq, d, device="cuda")
    lo = 0
    for p, n in enumerate(sizes):
        ra.decode_partial(q.cuda(), k_all[lo:lo + n].cuda(), v_all[lo:lo + n].cuda(), m=m[p], z=z[p], y=y[p])
        lo += n
    out, lse = ra.merge(m, z, y, out_dtype=torch.float32)
    torch.cuda.synchronize()
    want_o, want_lse = oracle.dense_attention(q.double().numpy(), np.full(n_q, N), k_all.double().numpy(),
                                              v_all.double().numpy(), True)
    assert np.abs(out.cpu().double().numpy() - want_o).max() <= TOL_O
    assert np.abs(lse.cpu().double().numpy() - want_lse).max() <= TOL_LSE


def test_decode_timing_counts_calls():
    q = torch.randn(1, 4, 128, device="cuda").to(torch.bfloat16)
    k = torch.randn(512, 1, 128, device="cuda").to(torch.bfloat16)
    ra.timing_collect_decode()
    ra.timing_enable(True)
    try:
        for _ in range(3):
            ra.decode_partial(q, k, k)
        got = ra.timing_collect_decode()
    finally:
        ra.timing_enable(False)
    assert got["decode_calls"] == 3 and got["decode_ms"] > 0
