"""Plain fp64 NumPy oracle: dense attention, the ring recurrence, the triple merge.

TEST INFRASTRUCTURE (see the package docstring): never imported by the product.

Array conventions (batch 1, all float64):
  q rows      [R, Hq, d]    query vectors of R rows
  k, v        [N, Hkv, d]   keys / values in GLOBAL token order (token t at index t)
  O           [R, Hq, d]
  LSE         [Hq, R]       natural log: LSE = m + ln z
  state m, z  [Hq, R];  y [R, Hq, d]   (unnormalised accumulator)

Query head h reads key/value head h // (Hq // Hkv) (contiguous groups of query
heads share one key/value head, the grouped-query reading of the pages, which
give GQA only as head counts).
"""

from __future__ import annotations

import math

import numpy as np

NEG_INF = -math.inf


# ---------------------------------------------------------------------------
# Shard layout (which global tokens a shard holds) and the causal predicate.
# ---------------------------------------------------------------------------

def shard_positions(layout: str, r: int, P: int, b: int) -> np.ndarray:
    """Global token index of every local row of shard r.

    contiguous: the sequence is cut into P consecutive blocks of b tokens and
      shard r holds tokens r*b .. r*b + b - 1 ("Ring Attention" (aarnphm.xyz):
      device u owns Q^(u), K^(u), V^(u) of L/p tokens; transformer-math page,
      "The mechanism, compressed": P contiguous blocks of b = N/P tokens).
    striped: token t lives on device t mod P, so local row j of shard r is
      token j*P + r ("Ring Attention" (aarnphm.xyz): Striped Attention keeps the
      ring schedule but alternates shard ownership).
    zigzag: the sequence is cut into 2P chunks of c = b/2 tokens and shard r
      holds chunk r, then chunk 2P-1-r: local row j < c is token r*c + j and
      local row j >= c is token (2P-1-r)*c + (j - c) ("Ring Attention"
      (darshanfofadiya.com) 4.8.3, the zigzag assignment table: each GPU gets
      one early and one late block; transformer-math page, "Causal masking
      wastes half the ring": device i gets chunks i and 2P-1-i).  Requires an
      even b.
    """
    j = np.arange(b, dtype=np.int64)
    if layout == "contiguous":
        return r * b + j
    if layout == "striped":
        return j * P + r
    if layout == "zigzag":
        if b % 2:
            raise ValueError("zigzag needs an even shard size")
        c = b // 2
        early = j < c
        return np.where(early, r * c + j, (2 * P - 1 - r) * c + (j - c))
    raise ValueError(f"unknown layout {layout!r}")


def allowed_mask(tq: np.ndarray, tk: np.ndarray, causal: bool) -> np.ndarray:
    """allowed[i, j] is True when query token tq[i] may attend to key token tk[j].

    Causal: key position <= query position on GLOBAL indices ("Ring Attention"
    (darshanfofadiya.com) 4.8: token i attends to tokens 0 through i; the
    transformer-math page, "Composing with tensor parallelism": positions are
    global).  Non-causal: every key is allowed.
    """
    tq = np.asarray(tq, dtype=np.int64)
    tk = np.asarray(tk, dtype=np.int64)
    if not causal:
        return np.ones((tq.size, tk.size), dtype=bool)
    return tk[None, :] <= tq[:, None]


def allowed_pair_count(layout: str, u: int, P: int, b: int, causal: bool) -> int:
    """Number of allowed (query, key) pairs of rank u over the whole ring, per head.

    Brute force: the mask of every visiting block, summed.
    """
    tq = shard_positions(layout, u, P, b)
    total = 0
    for r in range(P):
        total += int(allowed_mask(tq, shard_positions(layout, r, P, b), causal).sum())
    return total


# ---------------------------------------------------------------------------
# Dense definition.
# ---------------------------------------------------------------------------

def dense_attention(q_rows, tq, k, v, causal: bool, max_chunk_elems: int = 1 << 22):
    """Softmax attention of the given query rows against the whole sequence.

    For query head h and row i at global token tq[i], with A the allowed keys:
      S_t = q . k_t / sqrt(d)            ("Ring Attention" (aarnphm.xyz), eq. S)
      O   = sum_{t in A} e^{S_t - M} v_t / sum_{t in A} e^{S_t - M},  M = max_{t in A} S_t
      LSE = M + ln sum_{t in A} e^{S_t - M}
    Rows with no allowed key get O = 0 and LSE = -inf.  Rows are processed in
    chunks only to bound memory; every row is computed independently.
    """
    q_rows = np.asarray(q_rows, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    tq = np.asarray(tq, dtype=np.int64)
    R, Hq, d = q_rows.shape
    N, Hkv, _ = k.shape
    G = Hq // Hkv
    out = np.zeros((R, Hq, d))
    lse = np.full((Hq, R), NEG_INF)
    n_keys = N if not causal else int(min(N, tq.max(initial=-1) + 1))
    if R == 0 or n_keys <= 0:
        return out, lse
    tk = np.arange(n_keys, dtype=np.int64)
    step = max(1, max_chunk_elems // n_keys)
    scale = 1.0 / math.sqrt(d)
    for h in range(Hq):
        kh = k[:n_keys, h // G, :]
        vh = v[:n_keys, h // G, :]
        for lo in range(0, R, step):
            hi = min(R, lo + step)
            s = (q_rows[lo:hi, h, :] @ kh.T) * scale
            allow = allowed_mask(tq[lo:hi], tk, causal)
            s = np.where(allow, s, NEG_INF)
            mx = s.max(axis=1)
            has = np.isfinite(mx)
            mref = np.where(has, mx, 0.0)
            e = np.where(allow, np.exp(s - mref[:, None]), 0.0)
            z = e.sum(axis=1)
            zs = np.where(has, z, 1.0)
            out[lo:hi, h, :] = np.where(has[:, None], (e @ vh) / zs[:, None], 0.0)
            lse[h, lo:hi] = np.where(has, mref + np.log(zs), NEG_INF)
    return out, lse


# ---------------------------------------------------------------------------
# The ring recurrence.
# ---------------------------------------------------------------------------

def empty_state(R: int, Hq: int, d: int):
    """The state before any block is seen: m = -inf, z = 0, y = 0 (the worked
    example of the aicomputerinstitute page starts every query there)."""
    return (np.full((Hq, R), NEG_INF), np.zeros((Hq, R)), np.zeros((R, Hq, d)))


def online_fold(m, z, y, s, vals):
    """Fold one visiting block into one head's running (m, z, y).

    m, z: [R]; y: [R, d]; s: [R, n] scores with masked entries = -inf;
    vals: [n, d].  Following "Ring Attention" (aarnphm.xyz), eqs. m, z, y:
      m' = max(m, max_j s_j)
      z' = z e^{m - m'} + sum_j e^{s_j - m'}
      y' = y e^{m - m'} + sum_j e^{s_j - m'} v_j
    When m' is still -inf (no allowed key seen yet) the row is unchanged: the
    empty set adds nothing and the rescale factor is taken as 1, never
    e^{-inf - (-inf)}.
    """
    blk_max = s.max(axis=1) if s.shape[1] else np.full(s.shape[0], NEG_INF)
    m_new = np.maximum(m, blk_max)
    live = np.isfinite(m_new)
    m_safe = np.where(live, m_new, 0.0)
    # A finite m implies a finite m'.  From m = -inf the old (z, y) are zero,
    # so the factor only has to be finite: 0 once a key is seen, else 1.
    alpha = np.where(np.isfinite(m), np.exp(m - m_safe), np.where(live, 0.0, 1.0))
    p = np.where(np.isfinite(s), np.exp(s - m_safe[:, None]), 0.0)
    z_new = z * alpha + p.sum(axis=1)
    y_new = y * alpha[:, None] + p @ vals
    return m_new, z_new, y_new


def finish(m, z, y):
    """O = y / z and LSE = m + ln z ("Ring Attention" (aarnphm.xyz), eq. O).

    m, z: [Hq, R]; y: [R, Hq, d].  A row that saw no allowed key (z = 0) gets
    O = 0 and LSE = -inf.
    """
    has = z > 0
    zs = np.where(has, z, 1.0)
    out = np.where(has.T[:, :, None], y / zs.T[:, :, None], 0.0)
    lse = np.where(has, m + np.log(zs), NEG_INF)
    return out, lse


def ring_forward(q_local, u: int, k, v, P: int, layout: str, causal: bool,
                 order=None, trace: bool = False):
    """Rank u's share of the ring, step by step.

    q_local [b, Hq, d] holds rank u's query rows in local order; k, v are the
    whole sequence in global order.  At step s the visiting block is shard
    b(u, s) = (u - s) mod P ("Ring Attention" (aarnphm.xyz); darshanfofadiya.com
    4.3.2-4.3.4: own block first, then the upstream neighbour's).  ``order``
    overrides the visiting order (any permutation of 0..P-1) to test order
    invariance.  Each visit forms S = Q K^T / sqrt(d) on the block's tokens,
    masks it with global positions and folds it in; after all P visits
    O = y / z.  With trace=True the state after every visit is also returned.
    """
    q_local = np.asarray(q_local, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    b, Hq, d = q_local.shape
    N, Hkv, _ = k.shape
    if N != P * b:
        raise ValueError("the sequence must split into P shards of b tokens")
    G = Hq // Hkv
    scale = 1.0 / math.sqrt(d)
    tq = shard_positions(layout, u, P, b)
    visits = [(u - s) % P for s in range(P)] if order is None else list(order)
    m, z, y = empty_state(b, Hq, d)
    states = []
    for r in visits:
        tk = shard_positions(layout, r, P, b)
        allow = allowed_mask(tq, tk, causal)
        for h in range(Hq):
            s = (q_local[:, h, :] @ k[tk, h // G, :].T) * scale
            s = np.where(allow, s, NEG_INF)
            m[h], z[h], y[:, h, :] = online_fold(m[h], z[h], y[:, h, :], s, v[tk, h // G, :])
        if trace:
            states.append((r, m.copy(), z.copy(), y.copy()))
    out, lse = finish(m, z, y)
    if trace:
        return out, lse, states
    return out, lse


# ---------------------------------------------------------------------------
# Backward: gradients of L = sum(dO * O).
# ---------------------------------------------------------------------------

def backward_dense(q_rows, tq, k, v, dout, causal: bool):
    """Gradients of L = sum_{i,h,c} dO[i,h,c] O[i,h,c] for O = dense attention.

    The softmax Jacobian written out, per query head h (KV head h // G), with
    P the masked softmax of S = Q K^T / sqrt(d) and O = P V:
      dV = P^T dO,   dP = dO V^T,   dS = P * (dP - rowsum(dP * P)),
      dQ = dS K / sqrt(d),   dK = dS^T Q / sqrt(d).
    Query heads of one group add into their key/value head's dK, dV.  Returns
    dq [R, Hq, d] and dk, dv [N, Hkv, d] over the whole sequence.
    """
    q_rows = np.asarray(q_rows, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    dout = np.asarray(dout, dtype=np.float64)
    R, Hq, d = q_rows.shape
    N, Hkv, _ = k.shape
    G = Hq // Hkv
    scale = 1.0 / math.sqrt(d)
    allow = allowed_mask(tq, np.arange(N), causal)
    has = allow.any(axis=1)
    dq = np.zeros((R, Hq, d))
    dk = np.zeros((N, Hkv, d))
    dv = np.zeros((N, Hkv, d))
    for h in range(Hq):
        kh, vh = k[:, h // G, :], v[:, h // G, :]
        s = np.where(allow, (q_rows[:, h, :] @ kh.T) * scale, NEG_INF)
        mx = np.where(has, s.max(axis=1), 0.0)
        e = np.where(allow, np.exp(s - mx[:, None]), 0.0)
        p = e / np.where(has, e.sum(axis=1), 1.0)[:, None]
        do = dout[:, h, :]
        dv[:, h // G, :] += p.T @ do
        dp = do @ vh.T
        ds = p * (dp - (dp * p).sum(axis=1, keepdims=True))
        dq[:, h, :] = ds @ kh * scale
        dk[:, h // G, :] += ds.T @ q_rows[:, h, :] * scale
    return dq, dk, dv


def ring_backward(q_local, u: int, k, v, out, lse, dout, P: int, layout: str, causal: bool, order=None):
    """Rank u's share of the backward ring.

    The transformer-math page ("The backward pass costs a second ring"): the
    key/value blocks rotate again with their gradient accumulators, every
    device adds its contribution as a block passes, and the [b, b] scores are
    rebuilt from the saved row statistics and output instead of being stored.
    For each visiting block r (order as in ring_forward):
      S = Q K_r^T / sqrt(d) (masked),  P = e^{S - LSE}  (LSE saved by the
      forward, natural log),  D = rowsum(dO * O)  (O saved by the forward),
      dV_r += P^T dO,  dP = dO V_r^T,  dS = P * (dP - D),
      dQ += dS K_r / sqrt(d),  dK_r += dS^T Q / sqrt(d).
    q_local, out, dout [b, Hq, d]; lse [Hq, b]; k, v global [N, Hkv, d].
    Returns dq [b, Hq, d] and rank u's contributions dk, dv [P, b, Hkv, d] to
    every shard (local row order; zero for blocks it never sees).  A row with
    LSE = -inf saw no key and contributes nothing.
    """
    q_local = np.asarray(q_local, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    out = np.asarray(out, dtype=np.float64)
    lse = np.asarray(lse, dtype=np.float64)
    dout = np.asarray(dout, dtype=np.float64)
    b, Hq, d = q_local.shape
    N, Hkv, _ = k.shape
    if N != P * b:
        raise ValueError("the sequence must split into P shards of b tokens")
    G = Hq // Hkv
    scale = 1.0 / math.sqrt(d)
    tq = shard_positions(layout, u, P, b)
    live = np.isfinite(lse)                                   # [Hq, b]
    lse_safe = np.where(live, lse, 0.0)
    D = (dout * out).sum(axis=2).T                            # [Hq, b]
    dq = np.zeros((b, Hq, d))
    dk = np.zeros((P, b, Hkv, d))
    dv = np.zeros((P, b, Hkv, d))
    visits = [(u - s) % P for s in range(P)] if order is None else list(order)
    for r in visits:
        tk = shard_positions(layout, r, P, b)
        allow = allowed_mask(tq, tk, causal)
        for h in range(Hq):
            kr, vr = k[tk, h // G, :], v[tk, h // G, :]
            s = (q_local[:, h, :] @ kr.T) * scale
            p = np.where(allow & live[h][:, None], np.exp(s - lse_safe[h][:, None]), 0.0)
            do = dout[:, h, :]
            dv[r, :, h // G, :] += p.T @ do
            dp = do @ vr.T
            ds = p * (dp - D[h][:, None])
            dq[:, h, :] += ds @ kr * scale
            dk[r, :, h // G, :] += ds.T @ q_local[:, h, :] * scale
    return dq, dk, dv


def backward_sampled(q_local, u: int, k, v, out, lse, dout, P: int, layout: str, causal: bool, rows, keys):
    """Selected entries of rank u's backward share (ring_backward), each summed
    over the whole sequence at once instead of visit by visit.

    The formulas of "The backward pass costs a second ring" (transformer-math
    page) for one query row i at global token t_i, head h (key/value head
    g = h // G), with D_i = dO_i . O_i and, for each key token t that row i
    may see, S = q_i . k_t / sqrt(d), p = e^{S - LSE_i}, dP = dO_i . v_t,
    dS = p (dP - D_i):
      dQ_i  = sum_t dS k_t / sqrt(d)
    and for one key token t (shard r, local row j), over the rank's rows i
    that may see it, summed over the query heads of its group:
      dV_r[j] = sum_i p dO_i,    dK_r[j] = sum_i dS q_i / sqrt(d).
    rows: local query rows of rank u; keys: (r, j) pairs.  Returns dq
    [len(rows), Hq, d], dk and dv [len(keys), Hkv, d].  A row with
    LSE = -inf saw no key and contributes nothing.
    """
    q_local = np.asarray(q_local, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    out = np.asarray(out, dtype=np.float64)
    lse = np.asarray(lse, dtype=np.float64)
    dout = np.asarray(dout, dtype=np.float64)
    b, Hq, d = q_local.shape
    N, Hkv, _ = k.shape
    G = Hq // Hkv
    scale = 1.0 / math.sqrt(d)
    rows = np.asarray(rows, dtype=np.int64)
    tq = shard_positions(layout, u, P, b)
    tk = np.array([shard_positions(layout, r, P, b)[j] for r, j in keys], dtype=np.int64)
    live = np.isfinite(lse)
    lse_safe = np.where(live, lse, 0.0)
    D = (dout * out).sum(axis=2).T                            # [Hq, b]
    dq = np.zeros((rows.size, Hq, d))
    dk = np.zeros((tk.size, Hkv, d))
    dv = np.zeros((tk.size, Hkv, d))
    allow_rows = allowed_mask(tq[rows], np.arange(N), causal)  # [R, N]
    allow_keys = allowed_mask(tq, tk, causal)                  # [b, K]
    for h in range(Hq):
        g = h // G
        # dQ of the selected rows against every key of the sequence.
        s = (q_local[rows, h, :] @ k[:, g, :].T) * scale
        p = np.where(allow_rows & live[h, rows][:, None], np.exp(s - lse_safe[h, rows][:, None]), 0.0)
        dp = dout[rows, h, :] @ v[:, g, :].T
        ds = p * (dp - D[h, rows][:, None])
        dq[:, h, :] = ds @ k[:, g, :] * scale
        # dK, dV of the selected keys from every row of the rank.
        s = (q_local[:, h, :] @ k[tk, g, :].T) * scale
        p = np.where(allow_keys & live[h][:, None], np.exp(s - lse_safe[h][:, None]), 0.0)
        dv[:, g, :] += p.T @ dout[:, h, :]
        dp = dout[:, h, :] @ v[tk, g, :].T
        ds = p * (dp - D[h][:, None])
        dk[:, g, :] += ds.T @ q_local[:, h, :] * scale
    return dq, dk, dv


# ---------------------------------------------------------------------------
# Decode: the query passes, the key/value shard stays.
# ---------------------------------------------------------------------------

def decode_partial(q_rows, k_shard, v_shard):
    """Partial (m, z, y) of new query rows against one resident key/value shard.

    q_rows [R, Hq, d]; k_shard, v_shard [n, Hkv, d] (the shard's cached keys
    and values, any n >= 0).  In decode the new token comes after every cached
    one, so every key of the shard is allowed.  The transformer-math page ("The
    ring is a prefill algorithm") keeps the cache sharded and stationary,
    broadcasts the query, and has each device return a partial (m, l, o) for
    one small reduction to combine; darshanfofadiya.com 4.9.4.4 passes Q
    around the ring for the same split.  The partial is one fold of the shard
    into the empty state, so m, z: [Hq, R] (natural log), y: [R, Hq, d]
    unnormalised; an empty shard gives (-inf, 0, 0).
    """
    q_rows = np.asarray(q_rows, dtype=np.float64)
    k_shard = np.asarray(k_shard, dtype=np.float64)
    v_shard = np.asarray(v_shard, dtype=np.float64)
    R, Hq, d = q_rows.shape
    n, Hkv, _ = k_shard.shape
    G = Hq // Hkv
    scale = 1.0 / math.sqrt(d)
    m, z, y = empty_state(R, Hq, d)
    for h in range(Hq):
        s = (q_rows[:, h, :] @ k_shard[:, h // G, :].T) * scale
        m[h], z[h], y[:, h, :] = online_fold(m[h], z[h], y[:, h, :], s, v_shard[:, h // G, :])
    return m, z, y


# ---------------------------------------------------------------------------
# Merge of partial (m, z, y) triples.
# ---------------------------------------------------------------------------

def merge_partials(m, z, y):
    """Combine n partial triples of the same query rows with one rescale-and-add.

    m, z: [n, ...]; y: [n, ..., d]; m in natural-log units.  With
    m* = max_i m_i and w_i = e^{m_i - m*}:  z* = sum_i w_i z_i,
    y* = sum_i w_i y_i, O = y* / z*, LSE = m* + ln z*  (transformer-math page,
    "The ring is a prefill algorithm": each shard returns a partial (m, l, o)
    and one small reduction combines them).  A partial with m = -inf, z = 0,
    y = 0 is neutral; if every partial is empty, O = 0 and LSE = -inf.
    """
    m = np.asarray(m, dtype=np.float64)
    z = np.asarray(z, dtype=np.float64)
    y = np.asarray(y, dtype=np.float64)
    m_star = m.max(axis=0)
    live = np.isfinite(m_star)
    m_safe = np.where(live, m_star, 0.0)
    w = np.where(np.isfinite(m), np.exp(m - m_safe[None]), 0.0)
    z_star = (w * z).sum(axis=0)
    y_star = (w[..., None] * y).sum(axis=0)
    has = z_star > 0
    zs = np.where(has, z_star, 1.0)
    out = np.where(has[..., None], y_star / zs[..., None], 0.0)
    lse = np.where(has, m_safe + np.log(zs), NEG_INF)
    return out, lse
