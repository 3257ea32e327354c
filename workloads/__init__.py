"""Seeded synthetic inputs and named workload presets.

This module is shared by the tests, the bench and smoke(): it only draws random
numbers and names shapes.  It holds none of the attention arithmetic, no shard
layout and no masking: the oracle and the HIP path each do that on their own.

Generation is counter-based per chunk of CHUNK tokens: chunk c of tensor
``name`` under ``seed`` is drawn from its own torch CPU generator, seeded with a
SplitMix64 hash of (seed, name, c).  Any subset of rows can therefore be drawn
without drawing the whole tensor, and the same row always gets the same values.
Values are drawn in float32 and then rounded to the workload dtype with torch's
round-to-nearest-even cast; the oracle reads those rounded values upcast
exactly.
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np
import torch

CHUNK = 256
_MASK64 = (1 << 64) - 1
_NAME_IDS = {"q": 1, "k": 2, "v": 3, "do": 4, "o": 5}   # "do": the upstream gradient dL/dO; "o": a stand-in output


def _splitmix64(x: int) -> int:
    x = (x + 0x9E3779B97F4A7C15) & _MASK64
    x = ((x ^ (x >> 30)) * 0xBF58476D1CE4E5B9) & _MASK64
    x = ((x ^ (x >> 27)) * 0x94D049BB133111EB) & _MASK64
    return x ^ (x >> 31)


def _chunk_seed(seed: int, name: str, chunk: int) -> int:
    h = _splitmix64(seed)
    h = _splitmix64(h ^ _NAME_IDS[name])
    h = _splitmix64(h ^ chunk)
    return h & ((1 << 63) - 1)


@dataclass(frozen=True)
class Workload:
    """One named configuration: sizes, value distributions, rank(s), dtype."""

    name: str
    N: int
    P: int
    ranks: tuple
    layout: str          # "contiguous" | "striped" | "zigzag"
    causal: bool
    Hq: int
    Hkv: int
    d: int
    dtype: str           # "f32" | "bf16"
    seed: int
    q_dist: str = "normal"
    k_dist: str = "normal"
    v_dist: str = "normal"
    k_scale: float = 1.0
    note: str = field(default="", compare=False)

    @property
    def b(self) -> int:
        return self.N // self.P

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "f32" else torch.bfloat16


WORKLOADS = {
    "tiny-ring-f32": Workload(
        "tiny-ring-f32", N=1024, P=4, ranks=(0, 1, 2, 3), layout="contiguous",
        causal=False, Hq=1, Hkv=1, d=64, dtype="f32", seed=1,
        note="N=1024, P=4 contiguous, 1 head, d=64, fp32, non-causal, all 4 ranks"),
    "32k-contiguous-causal": Workload(
        "32k-contiguous-causal", N=32768, P=8, ranks=(7,), layout="contiguous",
        causal=True, Hq=32, Hkv=8, d=128, dtype="bf16", seed=2,
        note="N=32768, P=8 contiguous, rank 7, 32/8 GQA, d=128, bf16, causal"),
    "32k-striped-causal": Workload(
        "32k-striped-causal", N=32768, P=8, ranks=(3,), layout="striped",
        causal=True, Hq=32, Hkv=8, d=128, dtype="bf16", seed=3,
        note="N=32768, P=8 striped (t mod 8), rank 3, 32/8 GQA, d=128, bf16, causal"),
    "128k-contiguous-causal": Workload(
        "128k-contiguous-causal", N=131072, P=8, ranks=(7,), layout="contiguous",
        causal=True, Hq=32, Hkv=8, d=128, dtype="bf16", seed=4, v_dist="uniform",
        note="N=131072, P=8 contiguous, rank 7, 32/8 GQA, d=128, bf16, V~U(-1,1), causal"),
    "1m-contiguous-causal": Workload(
        "1m-contiguous-causal", N=1048576, P=8, ranks=(7,), layout="contiguous",
        causal=True, Hq=4, Hkv=1, d=128, dtype="bf16", seed=5, k_scale=2.0,
        note="N=1048576, P=8 contiguous, rank 7, 4/1 GQA, d=128, bf16, K x 2.0, causal"),
    # Zigzag shards (2P chunks, shard r = chunks r and 2P-1-r): the balanced
    # causal layout, at the 32k and million-token shapes of the workloads above.
    "32k-zigzag-causal": Workload(
        "32k-zigzag-causal", N=32768, P=8, ranks=(2,), layout="zigzag",
        causal=True, Hq=32, Hkv=8, d=128, dtype="bf16", seed=6,
        note="N=32768, P=8 zigzag (chunks r, 15-r), rank 2, 32/8 GQA, d=128, bf16, causal"),
    "1m-zigzag-causal": Workload(
        "1m-zigzag-causal", N=1048576, P=8, ranks=(3,), layout="zigzag",
        causal=True, Hq=4, Hkv=1, d=128, dtype="bf16", seed=7, k_scale=2.0,
        note="N=1048576, P=8 zigzag (chunks r, 15-r), rank 3, 4/1 GQA, d=128, bf16, K x 2.0, causal"),
}


@dataclass(frozen=True)
class DecodeWorkload:
    """Pass-Q decode: n_q new tokens (global positions N .. N+n_q-1) against a
    cache of N = P * n_keys tokens held as P resident shards of n_keys tokens
    (shard p holds tokens p*n_keys .. p*n_keys + n_keys - 1); bf16."""

    name: str
    P: int
    n_keys: int
    n_q: int
    Hq: int
    Hkv: int
    d: int
    seed: int
    k_scale: float = 1.0
    note: str = field(default="", compare=False)

    @property
    def N(self) -> int:
        return self.P * self.n_keys


DECODE_WORKLOADS = {
    # Per GPU of 32 at 1M context with Llama-70B's heads (64 query, 8 key/value).
    "decode-31k-gqa64": DecodeWorkload(
        "decode-31k-gqa64", P=32, n_keys=31250, n_q=1, Hq=64, Hkv=8, d=128, seed=8,
        note="1 new token, 32 shards of 31,250 cached tokens, 64/8 GQA, d=128, bf16"),
    # The million-token share's shape: 8 shards of 131,072 tokens, 4/1 GQA, K x 2.
    "decode-1m-shard": DecodeWorkload(
        "decode-1m-shard", P=8, n_keys=131072, n_q=1, Hq=4, Hkv=1, d=128, seed=9, k_scale=2.0,
        note="1 new token, 8 shards of 131,072 cached tokens, 4/1 GQA, d=128, bf16, K x 2.0"),
}


def decode_query(w: DecodeWorkload) -> torch.Tensor:
    """The new tokens' query rows, [n_q, Hq, d] bf16."""
    return token_range(w.seed, "q", w.N, w.N + w.n_q, w.Hq, w.d, "normal", 1.0, torch.bfloat16)


def decode_shard(w: DecodeWorkload, p: int):
    """Cached K and V of shard p, [n_keys, Hkv, d] bf16 each."""
    lo, hi = p * w.n_keys, (p + 1) * w.n_keys
    k = token_range(w.seed, "k", lo, hi, w.Hkv, w.d, "normal", w.k_scale, torch.bfloat16)
    v = token_range(w.seed, "v", lo, hi, w.Hkv, w.d, "normal", 1.0, torch.bfloat16)
    return k, v


def _draw(gen: torch.Generator, shape, dist: str) -> torch.Tensor:
    if dist == "normal":
        return torch.randn(shape, generator=gen, dtype=torch.float32)
    if dist == "uniform":
        return torch.rand(shape, generator=gen, dtype=torch.float32) * 2.0 - 1.0
    raise ValueError(f"unknown distribution {dist!r}")


def token_rows(seed: int, name: str, rows, H: int, d: int, dist: str = "normal",
               scale: float = 1.0, dtype=torch.float32) -> torch.Tensor:
    """Rows ``rows`` (global token indices) of tensor ``name``: [len(rows), H, d]."""
    rows = torch.as_tensor(np.asarray(rows, dtype=np.int64))
    out = torch.empty((rows.numel(), H, d), dtype=torch.float32)
    if rows.numel() == 0:
        return out.to(dtype)
    chunks = torch.div(rows, CHUNK, rounding_mode="floor")
    order = torch.argsort(chunks, stable=True)
    sorted_chunks = chunks[order]
    uniq, counts = torch.unique_consecutive(sorted_chunks, return_counts=True)
    start = 0
    for c, n in zip(uniq.tolist(), counts.tolist()):
        sel = order[start:start + n]
        start += n
        gen = torch.Generator().manual_seed(_chunk_seed(seed, name, c))
        block = _draw(gen, (CHUNK, H, d), dist)
        out[sel] = block[rows[sel] - c * CHUNK]
    if scale != 1.0:
        out = out * scale
    return out.to(dtype)


def token_range(seed: int, name: str, start: int, stop: int, H: int, d: int,
                dist: str = "normal", scale: float = 1.0, dtype=torch.float32) -> torch.Tensor:
    """Rows start..stop-1 of tensor ``name``: [stop - start, H, d]."""
    return token_rows(seed, name, np.arange(start, stop), H, d, dist, scale, dtype)


def global_kv(w: Workload, seed: int | None = None):
    """K and V of the whole sequence in global token order, [N, Hkv, d] each."""
    s = w.seed if seed is None else seed
    k = token_range(s, "k", 0, w.N, w.Hkv, w.d, w.k_dist, w.k_scale, w.torch_dtype)
    v = token_range(s, "v", 0, w.N, w.Hkv, w.d, w.v_dist, 1.0, w.torch_dtype)
    return k, v


def query_rows(w: Workload, rows, seed: int | None = None) -> torch.Tensor:
    """Query vectors of the given global token indices, [len(rows), Hq, d]."""
    s = w.seed if seed is None else seed
    return token_rows(s, "q", rows, w.Hq, w.d, w.q_dist, 1.0, w.torch_dtype)


def sample_local_rows(b: int, count: int, seed: int, head: int) -> np.ndarray:
    """Sorted sample of ``count`` local row indices in [0, b), drawn without
    replacement from numpy's default_rng(seed * 1000 + head), always including
    rows 0, 1 and b - 1."""
    if count >= b:
        return np.arange(b, dtype=np.int64)
    rng = np.random.default_rng(seed * 1000 + head)
    must = np.unique(np.array([0, min(1, b - 1), b - 1], dtype=np.int64))
    pool = np.setdiff1d(np.arange(b, dtype=np.int64), must)
    extra = rng.choice(pool, size=max(0, count - must.size), replace=False)
    return np.sort(np.concatenate([must, extra]))
