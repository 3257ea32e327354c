"""Pins of the fp64 oracle against what the pages and the mathematics fix.

Nothing here compares the oracle with itself: each check uses a value the pages
print, a closed form, a library routine, or brute force written separately in
pure Python.  The mutation tests at the end plant plausible mistakes in copies of
the oracle's arithmetic and confirm that at least one pin catches each.
"""

import json
import math
import os

import numpy as np
import pytest
from scipy.special import softmax as scipy_softmax

import oracle
from oracle import ring_oracle as ro

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _rand_qkv(rng, N, Hq, Hkv, d, scale=1.0):
    q = rng.standard_normal((N, Hq, d))
    k = rng.standard_normal((N, Hkv, d)) * scale
    v = rng.standard_normal((N, Hkv, d))
    return q, k, v


# ---------------------------------------------------------------------------
# Worked example with printed values.
# ---------------------------------------------------------------------------

def _worked_example_errors():
    g = _load("worked_example.json")
    Q = np.array(g["Q"], float).reshape(4, 1, 1)
    K = np.array(g["K"], float).reshape(4, 1, 1)
    V = np.array(g["V"], float).reshape(4, 1, 1)
    want = np.array(g["outputs"])
    P, b = 2, 2
    ring_out = np.zeros(4)
    for u in range(P):
        o, _ = ro.ring_forward(Q[u * b:(u + 1) * b], u, K, V, P, "contiguous", False)
        ring_out[u * b:(u + 1) * b] = o[:, 0, 0]
    dense_out, _ = ro.dense_attention(Q, np.arange(4), K, V, False)
    _, _, states = ro.ring_forward(Q[0:2], 0, K, V, P, "contiguous", False, trace=True)
    trace_err = 0.0
    for (r, m, z, y), key in zip(states, ["after_step0", "after_step1"]):
        st = g["q1_on_device0"][key]
        trace_err = max(trace_err, abs(m[0, 0] - st["m"]), abs(z[0, 0] - st["l"]),
                        abs(y[0, 0, 0] - st["acc"]))
    visited = [r for (r, *_rest) in states]
    return (np.abs(ring_out - want).max(), np.abs(dense_out[:, 0, 0] - want).max(),
            trace_err, visited)


def test_worked_example_outputs_and_trace():
    ring_err, dense_err, trace_err, visited = _worked_example_errors()
    # outputs printed to 5 decimals, the running state to 6
    assert ring_err <= 5e-6 + 1e-12
    assert dense_err <= 5e-6 + 1e-12
    assert trace_err <= 5e-7 + 1e-12
    assert visited == [0, 1]   # device 0: own block, then the neighbour's


def test_worked_example_final_value_and_weights():
    g = _load("worked_example.json")
    q1 = np.array([[[1.0]]])
    K = np.array(g["K"], float).reshape(4, 1, 1)
    V = np.array(g["V"], float).reshape(4, 1, 1)
    o, lse = ro.dense_attention(q1, np.array([0]), K, V, False)
    assert abs(o[0, 0, 0] - g["q1_on_device0"]["final"]) <= 5e-7
    # LSE = max + ln Z, with the page's max 2 and Z = 1.55300
    assert abs(lse[0, 0] - (2.0 + math.log(g["q1_Z"]))) <= 5e-5


# ---------------------------------------------------------------------------
# Ring recurrence equals the dense definition.
# ---------------------------------------------------------------------------

RING_CASES = [
    # layout, causal, P, b, Hq, Hkv, d
    ("contiguous", False, 1, 13, 2, 1, 8),
    ("contiguous", False, 4, 9, 2, 2, 16),
    ("contiguous", True, 4, 7, 4, 2, 8),
    ("contiguous", True, 8, 5, 4, 1, 4),
    ("striped", True, 2, 11, 2, 1, 8),
    ("striped", True, 8, 6, 4, 2, 8),
    ("striped", False, 4, 5, 3, 1, 4),
    ("contiguous", True, 2, 16, 6, 3, 32),
    ("zigzag", True, 4, 6, 4, 2, 8),
    ("zigzag", True, 8, 4, 2, 1, 4),
    ("zigzag", False, 2, 8, 2, 1, 8),
    ("zigzag", True, 1, 10, 2, 1, 8),
]


@pytest.mark.parametrize("layout,causal,P,b,Hq,Hkv,d", RING_CASES)
def test_ring_equals_dense(layout, causal, P, b, Hq, Hkv, d):
    rng = np.random.default_rng(P * 100 + b)
    N = P * b
    q, k, v = _rand_qkv(rng, N, Hq, Hkv, d, scale=2.0)
    for u in range(P):
        tq = ro.shard_positions(layout, u, P, b)
        o_r, l_r = ro.ring_forward(q[tq], u, k, v, P, layout, causal)
        o_d, l_d = ro.dense_attention(q[tq], tq, k, v, causal)
        np.testing.assert_allclose(o_r, o_d, rtol=0, atol=1e-12)
        np.testing.assert_allclose(l_r, l_d, rtol=0, atol=1e-12)


@pytest.mark.parametrize("layout,causal", [("contiguous", True), ("striped", True),
                                           ("contiguous", False), ("zigzag", True)])
def test_order_invariance(layout, causal):
    rng = np.random.default_rng(7)
    P, b, Hq, Hkv, d = 8, 6, 4, 2, 8
    q, k, v = _rand_qkv(rng, P * b, Hq, Hkv, d, scale=3.0)
    for u in (0, 3, 7):
        tq = ro.shard_positions(layout, u, P, b)
        base_o, base_l = ro.ring_forward(q[tq], u, k, v, P, layout, causal)
        for _ in range(5):
            order = rng.permutation(P)
            o, l = ro.ring_forward(q[tq], u, k, v, P, layout, causal, order=order)
            np.testing.assert_allclose(o, base_o, rtol=0, atol=1e-12)
            np.testing.assert_allclose(l, base_l, rtol=0, atol=1e-12)


def test_p1_is_library_softmax_attention():
    """P = 1, non-causal: one visit, and the result is softmax(QK^T/sqrt(d)) V
    computed with scipy's softmax."""
    rng = np.random.default_rng(11)
    N, Hq, Hkv, d = 37, 3, 1, 16
    q, k, v = _rand_qkv(rng, N, Hq, Hkv, d)
    o, lse = ro.ring_forward(q, 0, k, v, 1, "contiguous", False)
    for h in range(Hq):
        s = q[:, h, :] @ k[:, 0, :].T / math.sqrt(d)
        want = scipy_softmax(s, axis=1) @ v[:, 0, :]
        np.testing.assert_allclose(o[:, h, :], want, rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse[h], np.log(np.exp(s).sum(axis=1)), rtol=0, atol=1e-12)


def test_causal_library_softmax():
    """Causal, P = 1: softmax over the lower triangle, via scipy with -inf."""
    rng = np.random.default_rng(12)
    N, d = 21, 8
    q, k, v = _rand_qkv(rng, N, 1, 1, d)
    o, _ = ro.ring_forward(q, 0, k, v, 1, "contiguous", True)
    s = q[:, 0, :] @ k[:, 0, :].T / math.sqrt(d)
    s = np.where(np.tril(np.ones((N, N), bool)), s, -np.inf)
    np.testing.assert_allclose(o[:, 0, :], scipy_softmax(s, axis=1) @ v[:, 0, :], atol=1e-12, rtol=0)


# ---------------------------------------------------------------------------
# Closed forms and special cases.
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("layout,causal", [("contiguous", True), ("striped", True),
                                           ("contiguous", False)])
def test_all_equal_keys_give_mean_of_allowed_values(layout, causal):
    rng = np.random.default_rng(3)
    P, b, Hq, Hkv, d = 4, 5, 2, 1, 8
    N = P * b
    q = rng.standard_normal((N, Hq, d))
    key = rng.standard_normal(d)
    k = np.broadcast_to(key, (N, Hkv, d)).copy()
    v = rng.standard_normal((N, Hkv, d))
    for u in range(P):
        tq = ro.shard_positions(layout, u, P, b)
        o, lse = ro.ring_forward(q[tq], u, k, v, P, layout, causal)
        for i, t in enumerate(tq):
            count = t + 1 if causal else N
            want = v[:count, 0, :].mean(axis=0)
            for h in range(Hq):
                np.testing.assert_allclose(o[i, h], want, rtol=0, atol=1e-12)
                s0 = q[t, h] @ key / math.sqrt(d)
                assert abs(lse[h, i] - (s0 + math.log(count))) <= 1e-12


def test_dominant_score_returns_that_value_row():
    rng = np.random.default_rng(5)
    N, d, P = 16, 4, 4
    b = N // P
    q = np.zeros((N, 1, d))
    q[:, 0, 0] = 1.0
    k = rng.uniform(-0.5, 0.5, (N, 1, d))
    k[:, 0, 0] = 0.0
    star = 9
    gap = 80.0        # score gap = 80 / sqrt(4) = 40
    k[star, 0, 0] = gap
    v = rng.standard_normal((N, 1, d))
    o, _ = ro.ring_forward(q[0:b], 0, k, v, P, "contiguous", False)
    s = q[0, 0] @ k[:, 0, :].T / math.sqrt(d)
    eff_gap = s[star] - np.delete(s, star).max()
    assert eff_gap >= 39.0
    bound = (N - 1) * math.exp(-eff_gap) * 2 * np.abs(v).max()
    assert np.abs(o[0, 0] - v[star, 0]).max() <= bound + 1e-15


def test_scale_is_one_over_sqrt_d():
    """d = 4: q.k1 = 2 so S1 = 1, S2 = 0; O = (e v1 + v2) / (e + 1)."""
    q = np.ones((1, 1, 4))
    k = np.zeros((2, 1, 4))
    k[0, 0, :2] = 1.0
    v = np.array([[[3.0, -1.0, 0.5, 2.0]], [[-2.0, 4.0, 1.0, 0.0]]])
    o, lse = ro.dense_attention(q, np.array([1]), k, v, False)
    e = math.e
    np.testing.assert_allclose(o[0, 0], (e * v[0, 0] + v[1, 0]) / (e + 1), rtol=0, atol=1e-15)
    assert abs(lse[0, 0] - math.log(e + 1)) <= 1e-15
    o2, _ = ro.ring_forward(np.ones((1, 1, 4)), 1, k, v, 2, "contiguous", False)
    np.testing.assert_allclose(o2[0, 0], o[0, 0], rtol=0, atol=1e-15)


def test_causal_predicate_is_inclusive_on_global_positions():
    rng = np.random.default_rng(8)
    P, b, d = 4, 3, 4
    N = P * b
    q, k, v = _rand_qkv(rng, N, 1, 1, d)
    # token 0 may only see itself
    o, lse = ro.ring_forward(q[0:b], 0, k, v, P, "contiguous", True)
    np.testing.assert_allclose(o[0, 0], v[0, 0], rtol=0, atol=1e-15)
    assert abs(lse[0, 0] - q[0, 0] @ k[0, 0] / 2.0) <= 1e-15
    # striped rank 0 row 0 is token 0 as well; rank 3 row 0 is token 3 and sees tokens 0..3
    o, _ = ro.ring_forward(q[ro.shard_positions("striped", 3, P, b)], 3, k, v, P, "striped", True)
    o_dense, _ = ro.dense_attention(q[3:4], np.array([3]), k[:4], v[:4], False)
    np.testing.assert_allclose(o[0, 0], o_dense[0, 0], rtol=0, atol=1e-12)


def test_gqa_head_map_contiguous_groups():
    """Hq = 4, Hkv = 2: heads 0, 1 read key/value head 0 and heads 2, 3 head 1."""
    rng = np.random.default_rng(9)
    N, d = 8, 4
    q = rng.standard_normal((N, 4, d))
    k = np.zeros((N, 2, d))
    v = np.zeros((N, 2, d))
    v[:, 0, :] = 1.0
    v[:, 1, :] = -5.0
    o, _ = ro.ring_forward(q[:4], 0, k, v, 2, "contiguous", False)
    np.testing.assert_allclose(o[:, 0:2, :], 1.0, atol=1e-15, rtol=0)
    np.testing.assert_allclose(o[:, 2:4, :], -5.0, atol=1e-15, rtol=0)


def _brute_force_row(qv, K, V, allowed, d):
    """Pure Python: weights e^{S_t} without subtracting any maximum, fsum."""
    ws = [math.exp(sum(a * b for a, b in zip(qv, K[t])) / math.sqrt(d)) for t in allowed]
    den = math.fsum(ws)
    out = [math.fsum(w * V[t][c] for w, t in zip(ws, allowed)) / den for c in range(len(V[0]))]
    return out, math.log(den)


@pytest.mark.parametrize("layout,causal,P", [("contiguous", True, 4), ("striped", True, 4),
                                             ("contiguous", False, 2), ("striped", True, 8),
                                             ("zigzag", True, 4), ("zigzag", True, 2)])
def test_brute_force_tiny(layout, causal, P):
    rng = np.random.default_rng(13 + P)
    N, d = 16, 3
    b = N // P
    q = rng.uniform(-1, 1, (N, 1, d))
    k = rng.uniform(-1, 1, (N, 1, d))
    v = rng.uniform(-1, 1, (N, 1, d))
    Kl = k[:, 0, :].tolist()
    Vl = v[:, 0, :].tolist()
    for u in range(P):
        # positions written out by hand, independent of shard_positions
        if layout == "contiguous":
            tq = list(range(u * b, u * b + b))
        elif layout == "striped":
            tq = [t for t in range(N) if t % P == u]
        else:   # zigzag: chunks of b/2 tokens, chunk u then chunk 2P-1-u
            c = b // 2
            tq = list(range(u * c, u * c + c)) + list(range((2 * P - 1 - u) * c, (2 * P - u) * c))
        o, lse = ro.ring_forward(q[tq], u, k, v, P, layout, causal)
        o_d, lse_d = ro.dense_attention(q[tq], np.array(tq), k, v, causal)
        for i, t in enumerate(tq):
            allowed = [s for s in range(N) if (s <= t or not causal)]
            want, want_lse = _brute_force_row(q[t, 0].tolist(), Kl, Vl, allowed, d)
            np.testing.assert_allclose(o[i, 0], want, rtol=0, atol=1e-12)
            np.testing.assert_allclose(o_d[i, 0], want, rtol=0, atol=1e-12)
            assert abs(lse[0, i] - want_lse) <= 1e-12
            assert abs(lse_d[0, i] - want_lse) <= 1e-12


# ---------------------------------------------------------------------------
# Layouts and counts.
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("P,b", [(1, 5), (4, 3), (8, 7)])
def test_shard_positions(P, b):
    N = P * b
    seen = []
    for r in range(P):
        c = ro.shard_positions("contiguous", r, P, b)
        assert c.tolist() == list(range(r * b, (r + 1) * b))
        s = ro.shard_positions("striped", r, P, b)
        assert s.tolist() == [t for t in range(N) if t % P == r]
        seen.extend(s.tolist())
    assert sorted(seen) == list(range(N))


@pytest.mark.parametrize("P,c", [(1, 3), (2, 1), (4, 3), (8, 5)])
def test_zigzag_positions(P, c):
    """Shard r holds chunk r, then chunk 2P-1-r, each in token order; the
    shards together hold every token once."""
    b, N = 2 * c, 2 * P * c
    seen = []
    for r in range(P):
        z = ro.shard_positions("zigzag", r, P, b).tolist()
        assert z[:c] == list(range(r * c, (r + 1) * c))
        assert z[c:] == list(range((2 * P - 1 - r) * c, (2 * P - r) * c))
        seen.extend(z)
    assert sorted(seen) == list(range(N))
    with pytest.raises(ValueError):
        ro.shard_positions("zigzag", 0, P, b + 1)


def _chunk_interactions(P, c, u):
    """For each chunk that zigzag shard u holds (early, then late): the number
    of the 2P chunks of keys it has at least one allowed pair with, from the
    oracle's positions and causal mask."""
    b = 2 * c
    tq = ro.shard_positions("zigzag", u, P, b)
    per = []
    for half in (tq[:c], tq[c:]):
        n = 0
        for ck in range(2 * P):
            tk = np.arange(ck * c, (ck + 1) * c)
            n += bool(ro.allowed_mask(half, tk, True).any())
        per.append(n)
    return per


def test_zigzag_balance_matches_page():
    g = _load("zigzag_balance.json")
    P, c = g["P"], 3
    held, per_chunk, per_gpu = [], [], []
    for u in range(P):
        tq = ro.shard_positions("zigzag", u, P, 2 * c)
        held.append(sorted({int(t) // c for t in tq}))
        pc = _chunk_interactions(P, c, u)
        per_chunk.append(pc)
        per_gpu.append(sum(pc))
    assert held == g["assignment"]
    assert per_chunk == g["per_chunk_interactions"]
    assert per_gpu == g["small_block_interactions_per_gpu"]
    assert sum(per_gpu) == g["total_small_interactions"]
    assert per_gpu[0] / 4 == g["big_block_equivalents_per_gpu"]
    # the contiguous bottleneck from the oracle's own masks
    worst = max(sum(bool(ro.allowed_mask(ro.shard_positions("contiguous", u, P, c),
                                         ro.shard_positions("contiguous", r, P, c), True).any())
                    for r in range(P)) for u in range(P))
    assert worst == g["contiguous_bottleneck_big_blocks"]


def test_zigzag_speedup_matches_page():
    """Every rank carries 2P+1 small-block interactions, so the wall-clock gain
    over contiguous shards (P big blocks on the last rank) is P / ((2P+1)/4);
    the page prints it to two decimals for 8 .. 64 GPUs."""
    g = _load("zigzag_balance.json")
    for ps, want in g["speedup_by_gpus"].items():
        P = int(ps)
        ranks = range(P) if P <= 16 else (0, P // 2, P - 1)
        counts = {sum(_chunk_interactions(P, 1, u)) for u in ranks}
        assert counts == {2 * P + 1}
        assert round(P / ((2 * P + 1) / 4), g["speedup_decimals"]) == want


def test_causal_block_counts_match_page():
    g = _load("causal_block_counts.json")
    P, b = g["P"], 3
    counts = []
    for u in range(P):
        tq = ro.shard_positions("contiguous", u, P, b)
        n = sum(bool(ro.allowed_mask(tq, ro.shard_positions("contiguous", r, P, b), True).any())
                for r in range(P))
        counts.append(n)
    assert counts == g["blocks_needed_per_gpu"]
    assert sum(counts) == g["total_blocks"]
    assert P * P == g["total_without_mask"]


@pytest.mark.parametrize("P,b", [(1, 4), (2, 5), (4, 6), (8, 3)])
def test_pair_count_closed_forms(P, b):
    """The closed forms the bench uses for useful FLOPs, against the brute-force mask."""
    import bench
    for u in range(P):
        assert ro.allowed_pair_count("contiguous", u, P, b, True) == \
            bench.useful_pairs("contiguous", u, P, b, True) == u * b * b + b * (b + 1) // 2
        assert ro.allowed_pair_count("striped", u, P, b, True) == \
            bench.useful_pairs("striped", u, P, b, True) == P * b * (b - 1) // 2 + (u + 1) * b
        assert ro.allowed_pair_count("striped", u, P, b, False) == \
            bench.useful_pairs("striped", u, P, b, False) == P * b * b


@pytest.mark.parametrize("P,c", [(1, 3), (2, 4), (4, 3), (8, 2)])
def test_zigzag_pair_count_closed_form(P, c):
    """Zigzag rank u: chunk u sees u full chunks and its own triangle, chunk
    2P-1-u sees 2P-1-u full chunks and its triangle: (2P-1) c^2 + c (c+1)
    pairs, the same on every rank."""
    import bench
    b = 2 * c
    for u in range(P):
        want = (2 * P - 1) * c * c + c * (c + 1)
        assert ro.allowed_pair_count("zigzag", u, P, b, True) == \
            bench.useful_pairs("zigzag", u, P, b, True) == want
        assert ro.allowed_pair_count("zigzag", u, P, b, False) == \
            bench.useful_pairs("zigzag", u, P, b, False) == P * b * b


def test_bandwidth_budget_figures():
    """FLOP and byte accounting reproduces the figures printed on the pages."""
    import bench
    g = _load("bandwidth_budget.json")
    f = g["flops_per_block_pair"]
    got = bench.useful_flops(f["b"] * f["b"], f["d"], 1)
    assert abs(got / f["printed_flops"] - 1) <= f["printed_rel_precision"]
    h = g["hop_bytes"]
    for case in h["cases"]:
        got = bench.hop_bytes(h["b"], case["d_kv"], 1, h["bytes_per_elem"])
        assert abs(got / case["printed_bytes"] - 1) <= h["printed_rel_precision"]
    p = g["per_head_flops_llama70b"]
    per_head = bench.useful_flops(p["b"] * p["b"], p["d_h"], 1)
    assert abs(per_head / p["printed_flops_per_head"] - 1) <= p["printed_rel_precision"]
    all_heads = bench.useful_flops(p["b"] * p["b"], p["d_h"], p["heads"])
    assert abs(all_heads / p["printed_flops_all_heads"] - 1) <= p["printed_rel_precision"]


# ---------------------------------------------------------------------------
# Merge of partial triples.
# ---------------------------------------------------------------------------

def _block_partials(q_local, u, k, v, P, layout, causal):
    """One partial (m, z, y) per visiting block, each folded from the empty state."""
    b, Hq, d = q_local.shape
    G = Hq // k.shape[1]
    tq = ro.shard_positions(layout, u, P, b)
    ms, zs, ys = [], [], []
    for r in range(P):
        tk = ro.shard_positions(layout, r, P, b)
        allow = ro.allowed_mask(tq, tk, causal)
        m, z, y = ro.empty_state(b, Hq, d)
        for h in range(Hq):
            s = np.where(allow, q_local[:, h, :] @ k[tk, h // G, :].T / math.sqrt(d), -np.inf)
            m[h], z[h], y[:, h, :] = ro.online_fold(m[h], z[h], y[:, h, :], s, v[tk, h // G, :])
        ms.append(m)
        zs.append(z)
        ys.append(np.transpose(y, (1, 0, 2)))   # [Hq, b, d] to match m, z
    return np.stack(ms), np.stack(zs), np.stack(ys)


@pytest.mark.parametrize("layout", ["contiguous", "striped", "zigzag"])
def test_merge_of_block_partials_equals_dense(layout):
    rng = np.random.default_rng(21)
    P, b, Hq, Hkv, d = 4, 6, 2, 1, 8
    q, k, v = _rand_qkv(rng, P * b, Hq, Hkv, d, scale=2.0)
    u = 2 if layout == "contiguous" else 1   # contiguous rank 2 has fully masked block 3
    tq = ro.shard_positions(layout, u, P, b)
    m, z, y = _block_partials(q[tq], u, k, v, P, layout, True)
    o, lse = ro.merge_partials(m, z, y)
    o_d, lse_d = ro.dense_attention(q[tq], tq, k, v, True)
    np.testing.assert_allclose(np.transpose(o, (1, 0, 2)), o_d, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, lse_d, rtol=0, atol=1e-12)


# ---------------------------------------------------------------------------
# Backward: gradients of L = sum(dO * O).
# ---------------------------------------------------------------------------

def _loss(q, tq, k, v, dout, causal):
    o, _ = ro.dense_attention(q, tq, k, v, causal)
    return float((o * dout).sum())


@pytest.mark.parametrize("causal", [True, False])
def test_backward_dense_matches_finite_differences(causal):
    """Central differences of L = sum(dO * O) through the dense forward, on
    every element of q, k and v of a tiny problem."""
    rng = np.random.default_rng(61)
    N, Hq, Hkv, d = 5, 2, 1, 3
    q, k, v = _rand_qkv(rng, N, Hq, Hkv, d, scale=1.0)
    dout = rng.standard_normal((N, Hq, d))
    tq = np.arange(N)
    dq, dk, dv = ro.backward_dense(q, tq, k, v, dout, causal)
    h = 1e-6
    for arr, grad in ((q, dq), (k, dk), (v, dv)):
        for idx in np.ndindex(arr.shape):
            old = arr[idx]
            arr[idx] = old + h
            lp = _loss(q, tq, k, v, dout, causal)
            arr[idx] = old - h
            lm = _loss(q, tq, k, v, dout, causal)
            arr[idx] = old
            assert abs((lp - lm) / (2 * h) - grad[idx]) <= 1e-7, (idx, grad[idx])


def test_backward_dense_matches_torch_autograd():
    """float64 autograd of a plain masked softmax attention written here."""
    import torch
    rng = np.random.default_rng(62)
    N, Hq, Hkv, d = 9, 4, 2, 8
    q, k, v = _rand_qkv(rng, N, Hq, Hkv, d, scale=2.0)
    dout = rng.standard_normal((N, Hq, d))
    tq = np.array([2, 3, 5, 8, 8, 0, 7, 1, 4])          # query positions in any order
    for causal in (True, False):
        dq, dk, dv = ro.backward_dense(q, tq, k, v, dout, causal)
        tqq = torch.tensor(q, requires_grad=True)
        tk = torch.tensor(k, requires_grad=True)
        tv = torch.tensor(v, requires_grad=True)
        G = Hq // Hkv
        ke = tk.repeat_interleave(G, dim=1)                # [N, Hq, d]
        ve = tv.repeat_interleave(G, dim=1)
        sc = torch.einsum("ihc,jhc->hij", tqq, ke) / np.sqrt(d)
        if causal:
            mask = torch.tensor(np.arange(N)[None, :] > tq[:, None])
            sc = sc.masked_fill(mask[None], float("-inf"))
        o = torch.einsum("hij,jhc->ihc", torch.softmax(sc, dim=-1), ve)
        (o * torch.tensor(dout)).sum().backward()
        np.testing.assert_allclose(dq, tqq.grad.numpy(), rtol=0, atol=1e-12)
        np.testing.assert_allclose(dk, tk.grad.numpy(), rtol=0, atol=1e-12)
        np.testing.assert_allclose(dv, tv.grad.numpy(), rtol=0, atol=1e-12)


BWD_CASES = [
    # layout, causal, P, b, Hq, Hkv, d
    ("contiguous", True, 4, 5, 4, 2, 8),
    ("contiguous", False, 2, 6, 2, 1, 4),
    ("striped", True, 4, 4, 2, 1, 8),
    ("zigzag", True, 4, 6, 4, 2, 8),
    ("contiguous", True, 1, 7, 2, 2, 4),
]


def _ring_backward_all_ranks(layout, causal, P, b, Hq, Hkv, d, seed):
    rng = np.random.default_rng(seed)
    N = P * b
    q, k, v = _rand_qkv(rng, N, Hq, Hkv, d, scale=2.0)
    dout = rng.standard_normal((N, Hq, d))
    dq = np.zeros((N, Hq, d))
    dk = np.zeros((N, Hkv, d))
    dv = np.zeros((N, Hkv, d))
    for u in range(P):
        tq = ro.shard_positions(layout, u, P, b)
        out, lse = ro.ring_forward(q[tq], u, k, v, P, layout, causal)
        gq, gk, gv = ro.ring_backward(q[tq], u, k, v, out, lse, dout[tq], P, layout, causal)
        dq[tq] = gq
        for r in range(P):
            tk = ro.shard_positions(layout, r, P, b)
            dk[tk] += gk[r]
            dv[tk] += gv[r]
    return (q, k, v, dout), (dq, dk, dv)


@pytest.mark.parametrize("layout,causal,P,b,Hq,Hkv,d", BWD_CASES)
def test_ring_backward_over_all_ranks_equals_dense_gradient(layout, causal, P, b, Hq, Hkv, d):
    """Every rank's dQ, and the contributions of all ranks to each block's dK,
    dV summed as the rotating accumulators sum them, give the dense gradient."""
    (q, k, v, dout), (dq, dk, dv) = _ring_backward_all_ranks(layout, causal, P, b, Hq, Hkv, d, P * 10 + b)
    N = P * b
    wq, wk, wv = ro.backward_dense(q, np.arange(N), k, v, dout, causal)
    np.testing.assert_allclose(dq, wq, rtol=0, atol=1e-12)
    np.testing.assert_allclose(dk, wk, rtol=0, atol=1e-12)
    np.testing.assert_allclose(dv, wv, rtol=0, atol=1e-12)


def test_ring_backward_order_invariance():
    rng = np.random.default_rng(63)
    P, b, Hq, Hkv, d = 4, 5, 2, 1, 8
    q, k, v = _rand_qkv(rng, P * b, Hq, Hkv, d, scale=2.0)
    dout = rng.standard_normal((P * b, Hq, d))
    u = 2
    tq = ro.shard_positions("striped", u, P, b)
    out, lse = ro.ring_forward(q[tq], u, k, v, P, "striped", True)
    base = ro.ring_backward(q[tq], u, k, v, out, lse, dout[tq], P, "striped", True)
    for _ in range(3):
        got = ro.ring_backward(q[tq], u, k, v, out, lse, dout[tq], P, "striped", True, order=rng.permutation(P))
        for a, b_ in zip(got, base):
            np.testing.assert_allclose(a, b_, rtol=0, atol=1e-12)


@pytest.mark.parametrize("layout,causal,P,b,Hq,Hkv,d", BWD_CASES)
def test_backward_sampled_equals_ring_backward_entries(layout, causal, P, b, Hq, Hkv, d):
    """The sampled backward (whole-sequence sums per row and per key) gives the
    same entries as the visit-by-visit ring backward, also for O and LSE that
    are not the forward's (any finite LSE; one row with LSE = -inf)."""
    rng = np.random.default_rng(P * 100 + b)
    N = P * b
    q, k, v = _rand_qkv(rng, N, Hq, Hkv, d, scale=2.0)
    dout = rng.standard_normal((N, Hq, d))
    for u in range(P):
        tq = ro.shard_positions(layout, u, P, b)
        out = 0.3 * rng.standard_normal((b, Hq, d))
        lse = rng.uniform(1.0, 4.0, (Hq, b))
        lse[0, -1] = -math.inf
        gq, gk, gv = ro.ring_backward(q[tq], u, k, v, out, lse, dout[tq], P, layout, causal)
        rows = np.arange(b)
        keys = [(r, j) for r in range(P) for j in range(b)]
        sq, sk, sv = ro.backward_sampled(q[tq], u, k, v, out, lse, dout[tq], P, layout, causal, rows, keys)
        np.testing.assert_allclose(sq, gq, rtol=0, atol=1e-12)
        np.testing.assert_allclose(sk, gk.reshape(P * b, Hkv, d), rtol=0, atol=1e-12)
        np.testing.assert_allclose(sv, gv.reshape(P * b, Hkv, d), rtol=0, atol=1e-12)
        part = ro.backward_sampled(q[tq], u, k, v, out, lse, dout[tq], P, layout, causal, rows[::2], keys[1::3])
        np.testing.assert_allclose(part[0], sq[::2], rtol=0, atol=1e-12)
        np.testing.assert_allclose(part[1], sk[1::3], rtol=0, atol=1e-12)
        np.testing.assert_allclose(part[2], sv[1::3], rtol=0, atol=1e-12)


def _bwd_without_d_term(q_local, u, k, v, out, lse, dout, P, layout, causal, order=None):
    return _REAL_BWD(q_local, u, k, v, out * 0.0, lse, dout, P, layout, causal, order)


def _bwd_unscaled_dk(q_local, u, k, v, out, lse, dout, P, layout, causal, order=None):
    dq, dk, dv = _REAL_BWD(q_local, u, k, v, out, lse, dout, P, layout, causal, order)
    return dq, dk * math.sqrt(q_local.shape[2]), dv


def _bwd_dense_no_centering(q_rows, tq, k, v, dout, causal):
    dq, dk, dv = _REAL_BWD_DENSE(q_rows, tq, k, v, dout, causal)
    return dq * 1.0001, dk, dv


_REAL_BWD = ro.ring_backward
_REAL_BWD_DENSE = ro.backward_dense


@pytest.mark.parametrize("replacement", [_bwd_without_d_term, _bwd_unscaled_dk])
def test_planted_ring_backward_mistakes_are_caught(monkeypatch, replacement):
    monkeypatch.setattr(ro, "ring_backward", replacement)
    with pytest.raises(AssertionError):
        test_ring_backward_over_all_ranks_equals_dense_gradient(*BWD_CASES[0])


def test_planted_dense_backward_mistake_is_caught(monkeypatch):
    monkeypatch.setattr(ro, "backward_dense", _bwd_dense_no_centering)
    with pytest.raises(AssertionError):
        test_backward_dense_matches_torch_autograd()
    with pytest.raises(AssertionError):
        test_backward_dense_matches_finite_differences(True)


# ---------------------------------------------------------------------------
# Decode: partial triples of resident shards.
# ---------------------------------------------------------------------------

def test_decode_partial_single_shard_is_softmax():
    """One shard: y / z is scipy's softmax of the scaled scores times V,
    m is the largest scaled score and LSE = m + ln z = logsumexp."""
    from scipy.special import logsumexp
    rng = np.random.default_rng(41)
    R, Hq, Hkv, d, n = 3, 4, 2, 16, 37
    q = rng.standard_normal((R, Hq, d))
    k = rng.standard_normal((n, Hkv, d)) * 2
    v = rng.standard_normal((n, Hkv, d))
    m, z, y = ro.decode_partial(q, k, v)
    for h in range(Hq):
        s = q[:, h, :] @ k[:, h // 2, :].T / np.sqrt(d)
        np.testing.assert_allclose(y[:, h, :] / z[h][:, None], scipy_softmax(s, axis=1) @ v[:, h // 2, :],
                                   rtol=0, atol=1e-12)
        np.testing.assert_allclose(m[h], s.max(axis=1), rtol=0, atol=1e-12)
        np.testing.assert_allclose(m[h] + np.log(z[h]), logsumexp(s, axis=1), rtol=0, atol=1e-12)


@pytest.mark.parametrize("sizes", [(8, 8, 8, 8), (5, 0, 11, 1, 7), (0, 0, 3)])
def test_decode_partials_merge_to_dense(sizes):
    """Pass-Q decode: each shard's partial against the broadcast query,
    merged, equals dense attention of the new tokens over the whole cache
    (every cached key precedes them); empty shards are neutral."""
    rng = np.random.default_rng(sum(sizes))
    N = sum(sizes)
    n_q, Hq, Hkv, d = 2, 4, 2, 8
    q = rng.standard_normal((n_q, Hq, d))
    k = rng.standard_normal((N, Hkv, d)) * 1.5
    v = rng.standard_normal((N, Hkv, d))
    parts = []
    lo = 0
    for n in sizes:
        parts.append(ro.decode_partial(q, k[lo:lo + n], v[lo:lo + n]))
        lo += n
    m = np.stack([p[0] for p in parts])
    z = np.stack([p[1] for p in parts])
    y = np.stack([np.transpose(p[2], (1, 0, 2)) for p in parts])   # [n, Hq, R, d]
    o, lse = ro.merge_partials(m, z, y)
    o_d, lse_d = ro.dense_attention(q, np.full(n_q, N), k, v, causal=True)
    np.testing.assert_allclose(np.transpose(o, (1, 0, 2)), o_d, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, lse_d, rtol=0, atol=1e-12)


def test_decode_partial_of_empty_shard_is_merge_identity():
    m, z, y = ro.decode_partial(np.ones((2, 2, 4)), np.zeros((0, 1, 4)), np.zeros((0, 1, 4)))
    assert np.all(m == -np.inf) and np.all(z == 0) and np.all(y == 0)


def test_decode_budget_figures():
    """Decode accounting reproduces the per-GPU figures printed for 1M context
    on 32 GPUs: 128 MB of K and V, 1.02e9 attention FLOPs, a 16 KB query."""
    import bench
    g = _load("decode_budget.json")
    tol = g["printed_rel_precision"]
    kv = bench.decode_kv_bytes(g["local_tokens"], g["kv_heads"], g["d_h"], g["bytes_per_elem"])
    assert abs(kv / g["printed_kv_bytes"] - 1) <= tol
    assert abs(kv / 2e12 * 1e3 / g["printed_kv_read_ms_at_2TBps"] - 1) <= tol
    fl = bench.decode_flops(g["new_tokens"], g["local_tokens"], g["d_h"], g["query_heads"])
    assert abs(fl / g["printed_attention_flops"] - 1) <= tol
    assert abs(fl / 175e12 * 1e3 / g["printed_attention_ms_at_175TFLOPs"] - 1) <= 0.1   # printed to 1 digit
    q_bytes = g["new_tokens"] * g["query_heads"] * g["d_h"] * g["bytes_per_elem"]
    assert q_bytes == g["printed_q_bytes_one_token"]
    # the decode partial's byte count is the shard plus the query and the fp32 triple
    full = bench.decode_bytes(1, g["local_tokens"], g["query_heads"], g["kv_heads"], g["d_h"])
    assert full == kv + q_bytes + g["query_heads"] * (g["d_h"] + 2) * 4


def test_merge_identity_associativity_commutativity():
    rng = np.random.default_rng(22)
    n, R, d = 5, 7, 4
    m = rng.standard_normal((n, R)) * 3
    z = rng.uniform(0.5, 2.0, (n, R))
    y = rng.standard_normal((n, R, d))
    o, lse = ro.merge_partials(m, z, y)
    # identity: an empty partial (-inf, 0, 0) changes nothing
    o2, lse2 = ro.merge_partials(np.concatenate([m, np.full((1, R), -np.inf)]),
                                 np.concatenate([z, np.zeros((1, R))]),
                                 np.concatenate([y, np.zeros((1, R, d))]))
    np.testing.assert_allclose(o2, o, atol=1e-14, rtol=0)
    np.testing.assert_allclose(lse2, lse, atol=1e-14, rtol=0)
    # commutativity
    perm = rng.permutation(n)
    o3, lse3 = ro.merge_partials(m[perm], z[perm], y[perm])
    np.testing.assert_allclose(o3, o, atol=1e-13, rtol=0)
    np.testing.assert_allclose(lse3, lse, atol=1e-13, rtol=0)
    # associativity: a merged pair re-enters as the triple (LSE, 1, O)
    oa, la = ro.merge_partials(m[:2], z[:2], y[:2])
    ob, lb = ro.merge_partials(m[2:], z[2:], y[2:])
    o4, lse4 = ro.merge_partials(np.stack([la, lb]), np.ones((2, R)), np.stack([oa, ob]))
    np.testing.assert_allclose(o4, o, atol=1e-13, rtol=0)
    np.testing.assert_allclose(lse4, lse, atol=1e-13, rtol=0)
    # closed form for two partials with equal maxima: (y1 + y2) / (z1 + z2)
    mm = np.zeros((2, R))
    o5, lse5 = ro.merge_partials(mm, z[:2], y[:2])
    np.testing.assert_allclose(o5, (y[0] + y[1]) / (z[0] + z[1])[:, None], atol=1e-14, rtol=0)
    np.testing.assert_allclose(lse5, np.log(z[0] + z[1]), atol=1e-14, rtol=0)


def test_merge_all_empty():
    o, lse = ro.merge_partials(np.full((3, 2), -np.inf), np.zeros((3, 2)), np.zeros((3, 2, 4)))
    assert np.all(o == 0.0)
    assert np.all(np.isneginf(lse))


def test_fold_of_fully_masked_block_keeps_state():
    m0 = np.array([-np.inf, 1.5])
    z0 = np.array([0.0, 2.0])
    y0 = np.array([[0.0, 0.0], [1.0, -1.0]])
    s = np.full((2, 3), -np.inf)
    m, z, y = ro.online_fold(m0, z0, y0, s, np.ones((3, 2)))
    assert np.isneginf(m[0]) and z[0] == 0 and np.all(y[0] == 0)
    assert m[1] == 1.5 and z[1] == 2.0 and np.all(y[1] == y0[1])
    assert not np.isnan(np.concatenate([m, z, y.ravel()])).any()


# ---------------------------------------------------------------------------
# Planted mistakes: each plausible error in the oracle must fail some pin.
# ---------------------------------------------------------------------------

def _fold_without_rescale(m, z, y, s, vals):
    m_new = np.maximum(m, s.max(axis=1))
    live = np.isfinite(m_new)
    m_safe = np.where(live, m_new, 0.0)
    p = np.where(np.isfinite(s), np.exp(s - m_safe[:, None]), 0.0)
    return m_new, z + p.sum(axis=1), y + p @ vals


def _fold_sign_flipped(m, z, y, s, vals):
    m_new = np.maximum(m, s.max(axis=1))
    live = np.isfinite(m_new)
    m_safe = np.where(live, m_new, 0.0)
    alpha = np.where(np.isfinite(m), np.exp(m_safe - np.where(np.isfinite(m), m, 0.0)),
                     np.where(live, 0.0, 1.0))
    p = np.where(np.isfinite(s), np.exp(s - m_safe[:, None]), 0.0)
    return m_new, z * alpha + p.sum(axis=1), y * alpha[:, None] + p @ vals


_REAL_FOLD = ro.online_fold


def _fold_rescale_y_only(m, z, y, s, vals):
    m_new, z_new, y_new = _REAL_FOLD(m, z, y, s, vals)
    p_sum = np.where(np.isfinite(s), np.exp(s - np.where(np.isfinite(m_new), m_new, 0)[:, None]), 0).sum(1)
    return m_new, z + p_sum, y_new          # forgets to rescale z


def _exclusive_mask(tq, tk, causal):
    tq = np.asarray(tq)
    tk = np.asarray(tk)
    if not causal:
        return np.ones((tq.size, tk.size), bool)
    return tk[None, :] < tq[:, None]


def _striped_transposed(layout, r, P, b):
    j = np.arange(b, dtype=np.int64)
    if layout == "striped":
        return r * P + j          # wrong: mixes up local row and shard index
    return r * b + j


def _zigzag_off_by_one(layout, r, P, b):
    j = np.arange(b, dtype=np.int64)
    if layout == "zigzag":
        c = b // 2
        return np.where(j < c, r * c + j, (2 * P - 2 - r) * c + (j - c))   # wrong late chunk
    if layout == "striped":
        return j * P + r
    return r * b + j


def _pins_fail():
    """Run a representative set of pins; return True if any of them fails."""
    checks = [test_worked_example_outputs_and_trace, test_p1_is_library_softmax_attention,
              test_causal_library_softmax, test_scale_is_one_over_sqrt_d,
              test_causal_predicate_is_inclusive_on_global_positions,
              test_gqa_head_map_contiguous_groups]
    checks += [lambda: test_shard_positions(4, 3),
               lambda: test_brute_force_tiny("striped", True, 4),
               lambda: test_all_equal_keys_give_mean_of_allowed_values("contiguous", True),
               lambda: test_ring_equals_dense(*RING_CASES[3]),
               lambda: test_brute_force_tiny("zigzag", True, 4),
               test_zigzag_balance_matches_page,
               test_decode_partial_single_shard_is_softmax]
    for c in checks:
        try:
            with np.errstate(all="ignore"):
                c()
        except (AssertionError, ValueError, IndexError, FloatingPointError):
            return True
    return False


@pytest.mark.parametrize("target,replacement", [
    ("online_fold", _fold_without_rescale),
    ("online_fold", _fold_sign_flipped),
    ("online_fold", _fold_rescale_y_only),
    ("allowed_mask", _exclusive_mask),
    ("shard_positions", _striped_transposed),
    ("shard_positions", _zigzag_off_by_one),
])
def test_planted_mistakes_are_caught(monkeypatch, target, replacement):
    assert not _pins_fail()
    monkeypatch.setattr(ro, target, replacement)
    assert _pins_fail(), f"no pin caught a mistake planted in {target}"


def test_planted_scale_mistake_is_caught(monkeypatch):
    real_sqrt = ro.math.sqrt

    class _M:
        inf = math.inf
        log = staticmethod(math.log)

        @staticmethod
        def sqrt(x):
            return 1.0      # drops the 1/sqrt(d) scale

    assert real_sqrt(4) == 2
    monkeypatch.setattr(ro, "math", _M)
    assert _pins_fail()


def test_planted_gqa_mistake_is_caught(monkeypatch):
    real = ro.ring_forward

    def wrong_map(q_local, u, k, v, P, layout, causal, order=None, trace=False):
        # interleaved head groups instead of contiguous ones
        Hq, Hkv = q_local.shape[1], k.shape[1]
        G = Hq // Hkv
        perm = [(h % Hkv) * G + h // Hkv for h in range(Hq)]
        res = real(q_local[:, perm, :], u, k, v, P, layout, causal, order, trace)
        inv = np.argsort(perm)
        return (res[0][:, inv, :], res[1][inv]) + tuple(res[2:])

    monkeypatch.setattr(ro, "ring_forward", wrong_map)
    assert _pins_fail()


def test_planted_decode_mistake_is_caught(monkeypatch):
    real = ro.decode_partial

    def no_rescale_of_v(q, k, v):
        m, z, y = real(q, k, v)
        return m, z, y * 1.01          # y off by a constant factor
    monkeypatch.setattr(ro, "decode_partial", no_rescale_of_v)
    with pytest.raises(AssertionError):
        test_decode_partial_single_shard_is_softmax()
    with pytest.raises(AssertionError):
        test_decode_partials_merge_to_dense((5, 0, 11, 1, 7))


def test_package_exports():
    assert oracle.ring_backward is ro.ring_backward
    assert oracle.backward_dense is ro.backward_dense
    assert oracle.decode_partial is ro.decode_partial
    assert oracle.ring_forward is ro.ring_forward
    assert oracle.merge_partials is ro.merge_partials
