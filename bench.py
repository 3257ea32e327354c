"""Throughput of one device's share of a causal Ring Attention forward pass.

One "step" is one call of the whole hot path for rank u: the P ring steps (hop
copies into the double buffer, by default carried in the tails of the step
launches; the step kernels with the online-softmax fold; the fused O/LSE
epilogue) over one batch of synthetic input already resident in HBM.  Default workload: the million-token share (N = 1,048,576, P = 8, contiguous
shards, rank 7, 4 query heads / 1 key-value head, d_h = 128, bf16, K scaled by 2,
causal).

Prints ONE JSON line.  ``value`` is useful (mask-aware) attention TFLOP/s: 4*d_h
FLOPs per allowed (query, key) pair and query head, divided by the wall time per
step.  ``roofline`` reports the step kernel against the MI355X bf16 dense MFMA
peak, with its average launch duration measured by HIP events around every step
kernel inside the timed region.  ``cpu_baseline`` times the fp64 oracle on the
host cores on a bounded sample of query rows of the same workload.
``other_workloads`` times the forward on the other named bf16 workloads (the
striped and zigzag layouts, 32k and 128k shares), and
``backward_other_workloads`` the backward on the 128k share.
``reference_gemm`` times the vendor's dense bf16 GEMM on the same GPU (the
practical dense-MFMA rate under sustained load, for context), and
``reference_attention`` the vendor's own fused causal attention forward (torch
SDPA, flash backend) on a 16k-token, 32-head input, both for context.
``sclk_during_timed_region`` is the engine clock the driver reported while the
timed steps ran, and ``pct_of_bf16_peak_at_measured_clock`` the rate against
the peak scaled to that clock.
``merge_kernel`` and ``decode_kernel`` report the two HBM-bound kernels (the
triple merge; the pass-Q decode partial of one resident shard) as achieved GB/s
against 8 TB/s, the merge with the HBM bytes its counters measured
(``traffic``); ``backward`` reports the backward ring of a workload's rank as
useful TFLOP/s.  ``same_launches_on_constant_inputs`` times the headline
launches again on operands that do not toggle (Q = K = 0, V = 1), with the
engine clock then held: the rate the kernel's schedule sustains when the power
limit does not lower the clock (context, not the metric); the ``backward``
object carries the same diagnostic for the backward calls.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                       [--cpu-seconds S] [--no-cpu-baseline] [--no-merge]
                       [--no-decode] [--decode-workload NAME] [--decode-only]
                       [--no-backward] [--backward-workload NAME] [--backward-only]
                       [--no-gemm-ref] [--no-workloads] [--merge-only] [--no-constant-inputs]
                       [--hop-mode fused|serial|streams] [--hop-compare]
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))

# MI355X published dense peaks used as roofline denominators.
PEAK_BF16_TFLOPS = 2516.6     # 256 CUs x 4096 FLOP/clk/CU x 2.4 GHz
PEAK_HBM_GBS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "step_bf16_traffic.json")
MERGE_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "merge_traffic.json")
MERGE_SOURCE = os.path.join(ROOT, "ring_attention_block_step_amd", "csrc", "merge.hip")
# Sources of the step kernel (its own file and the hop copy it carries).
STEP_SOURCE = (os.path.join(ROOT, "ring_attention_block_step_amd", "csrc", "step_bf16.hip"),
               os.path.join(ROOT, "ring_attention_block_step_amd", "csrc", "pack_unit.h"))


# ---------------------------------------------------------------------------
# Accounting (pinned against the pages' figures and the oracle's mask counts).
# ---------------------------------------------------------------------------

def useful_pairs(layout: str, u: int, P: int, b: int, causal: bool) -> int:
    """Allowed (query, key) pairs of rank u over all P visiting blocks, per head.

    Non-causal: every pair, P*b^2.  Causal, contiguous shards: blocks r < u are
    fully allowed, block u is the lower triangle with its diagonal, blocks r > u
    are fully masked: u*b^2 + b(b+1)/2.  Causal, striped shards (token t on
    device t mod P): local key j of block r may be seen by local query i iff
    j <= i when r <= u and j < i when r > u, so blocks r <= u give b(b+1)/2 and
    blocks r > u give b(b-1)/2: P*b(b-1)/2 + (u+1)*b.  Causal, zigzag shards
    (chunks u and 2P-1-u of c = b/2 tokens): each chunk sees every earlier
    chunk in full and its own lower triangle, (2P-1)*c^2 + c(c+1) on every rank.
    """
    if not causal:
        return P * b * b
    if layout == "contiguous":
        return u * b * b + b * (b + 1) // 2
    if layout == "striped":
        return P * b * (b - 1) // 2 + (u + 1) * b
    if layout == "zigzag":
        c = b // 2
        return (2 * P - 1) * c * c + c * (c + 1)
    raise ValueError(layout)


def decode_flops(n_q: int, n_keys: int, d: int, heads: int) -> float:
    """Decode attention of n_q new tokens against n_keys cached keys: every key
    is allowed, 4*d FLOPs per (query, key) pair and head (darshanfofadiya.com
    4.9.4.2: heads x 4 x 1 x keys x d)."""
    return 4.0 * d * heads * n_q * n_keys


def decode_kv_bytes(n_keys: int, Hkv: int, d: int, elem: int = 2) -> int:
    """Bytes of the resident key/value shard a decode step reads: K and V,
    n_keys x Hkv x d each (darshanfofadiya.com 4.9.4.2, "KV cache reading")."""
    return 2 * n_keys * Hkv * d * elem


def decode_bytes(n_q: int, n_keys: int, Hq: int, Hkv: int, d: int) -> int:
    """Algorithmic HBM bytes of one decode partial: the bf16 key/value shard
    and query rows read, the fp32 partial (m, z, y) written."""
    return decode_kv_bytes(n_keys, Hkv, d) + n_q * Hq * d * 2 + n_q * Hq * (d + 2) * 4


def useful_flops(pairs: int, d: int, heads: int) -> float:
    """Two contractions per allowed pair and head, QK^T and PV: 4*d FLOPs
    (the transformer-math page's 4*b^2*d per block pair, counted on allowed
    pairs only)."""
    return 4.0 * d * pairs * heads


def hop_bytes(b: int, d: int, heads_kv: int, elem_bytes: int) -> int:
    """Bytes of one key/value block on the wire: K and V, b tokens each."""
    return 2 * b * d * heads_kv * elem_bytes


def source_digest(path=STEP_SOURCE) -> str:
    """sha256 (16 hex digits) of a source file, or of several concatenated."""
    h = hashlib.sha256()
    for p in ([path] if isinstance(path, str) else path):
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str):
    """HBM bytes per step-kernel launch from committed rocprofv3 counter runs,
    or None when they are missing or were taken on a different kernel source."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("workload") != workload or rec.get("step_source_sha256_16") != source_digest():
        return None
    return rec.get("bytes_per_launch")


def measured_merge_traffic():
    """HBM bytes per merge launch at the bench's merge shape from committed
    rocprofv3 counter runs, or None when they are missing or were taken on a
    different kernel source."""
    try:
        with open(MERGE_TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("shape") != dict(MERGE_SHAPE) or rec.get("merge_source_sha256_16") != source_digest(MERGE_SOURCE):
        return None
    return rec.get("bytes_per_launch")


# ---------------------------------------------------------------------------
# CPU baseline: the oracle, as it stands, on a bounded sample of rows.
# ---------------------------------------------------------------------------

def _blas_threads() -> int:
    try:
        from threadpoolctl import threadpool_info
        n = [p.get("num_threads", 0) for p in threadpool_info() if p.get("user_api") == "blas"]
        return max(n) if n else 1
    except Exception:
        return 1


def cpu_baseline(w, rank, k_glob, v_glob, seconds: float, gpu_out=None, gpu_lse=None):
    """Time oracle.dense_attention on growing batches of the 4096 sampled query
    rows (per head) that the parity checks use, until about ``seconds`` of
    work; report useful fp64 TFLOP/s over exactly the rows timed, with BLAS
    on every host core this process may run on.  The times for all 4096
    sampled rows and for the whole share are extrapolated from the timed rows
    by their allowed pairs, and labelled so."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    import oracle
    import workloads as wl

    host_cores = len(os.sched_getaffinity(0))
    k = k_glob.double().numpy()
    v = v_glob.double().numpy()
    tq_all = oracle.shard_positions(w.layout, rank, w.P, w.b)
    rows = wl.sample_local_rows(w.b, min(w.b, 4096), w.seed, 0)

    def allowed(tq):
        return (tq + 1) if w.causal else np.full(tq.shape, w.N)

    done, elapsed, pairs_done = 0, 0.0, 0
    batch = 4
    max_err = mean_err_sum = 0.0
    n_err = 0
    with threadpool_limits(host_cores, user_api="blas"):
        blas = _blas_threads()
        while done < rows.size and elapsed < seconds:
            sel = rows[done:done + batch]
            tq = tq_all[sel]
            q = wl.query_rows(w, tq).double().numpy()
            t0 = time.perf_counter()
            o, lse = oracle.dense_attention(q, tq, k, v, w.causal)
            elapsed += time.perf_counter() - t0
            pairs_done += int(allowed(tq).sum())
            if gpu_out is not None:
                err = np.abs(gpu_out[sel].astype(np.float64) - o)
                max_err = max(max_err, float(err.max()))
                mean_err_sum += float(err.sum())
                n_err += err.size
            done += sel.size
            batch = min(batch * 2, 256)
    flops = 4.0 * w.d * pairs_done * w.Hq
    pairs_sample = int(allowed(tq_all[rows]).sum())
    pairs_full = int(allowed(tq_all).sum())
    per_pair = elapsed / max(1, pairs_done)
    res = {
        "value": flops / elapsed / 1e12,
        "unit": "TFLOP/s",
        "cores": host_cores,
        "blas_threads": blas,
        "kind": "oracle",
        "sample": (f"{done} of the 4096 sampled query rows x {w.Hq} heads of rank {rank} "
                   f"({w.name}); fp64 NumPy dense oracle; {elapsed:.1f} s"),
        "rows_timed_per_head": int(done),
        "seconds_timed": elapsed,
        "extrapolated_4096_rows_per_head_s": per_pair * pairs_sample,
        "extrapolated_full_share_s": per_pair * pairs_full,
        "extrapolation": "seconds per allowed pair of the timed rows x allowed pairs (extrapolated, not timed)",
    }
    parity = None
    if gpu_out is not None and n_err:
        parity = {"rows": int(done), "max_abs": max_err, "mean_abs": mean_err_sum / n_err}
    return res, parity


# ---------------------------------------------------------------------------
# The triple-merge kernel (HBM-bound) and a plain copy for counter calibration.
# ---------------------------------------------------------------------------

MERGE_SHAPE = {"nparts": 8, "rows": 16384, "Hq": 32, "d_h": 128}


def merge_bytes(nparts: int, rows: int, Hq: int, d: int, out_bytes: int = 2) -> int:
    """Algorithmic HBM bytes of one merge: every (m, z, y) read once, O and LSE
    written once."""
    return nparts * rows * Hq * (4 * d + 8) + rows * Hq * (out_bytes * d + 4)


def measure_merge(reps: int = 10) -> dict:
    """Time ringattn_merge on seeded partial triples (HIP events around each
    kernel, inside the library) and report achieved GB/s against 8 TB/s."""
    import torch

    import ring_attention_block_step_amd as ra

    n, rows, Hq, d = (MERGE_SHAPE[k] for k in ("nparts", "rows", "Hq", "d_h"))
    g = torch.Generator(device="cuda").manual_seed(7)
    m = torch.randn(n, Hq, rows, device="cuda", generator=g) * 4
    z = torch.rand(n, Hq, rows, device="cuda", generator=g) + 0.5
    y = torch.randn(n, rows, Hq, d, device="cuda", generator=g)
    out = torch.empty(rows, Hq, d, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty(Hq, rows, dtype=torch.float32, device="cuda")
    for _ in range(2):
        ra.merge(m, z, y, out=out, lse=lse)
    torch.cuda.synchronize()
    ra.timing_collect()
    ra.timing_enable(True)
    for _ in range(reps):
        ra.merge(m, z, y, out=out, lse=lse)
    torch.cuda.synchronize()
    ra.timing_enable(False)
    t = ra.timing_collect()
    avg_ms = t["merge_ms"] / max(1, t["merge_launches"])
    nbytes = merge_bytes(n, rows, Hq, d)
    gbs = nbytes / (avg_ms * 1e-3) / 1e9
    return {"kernel": "merge_kernel<128,bf16>", "shape": dict(MERGE_SHAPE), "bytes_per_launch": nbytes,
            "avg_launch_ms": avg_ms, "achieved": gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": gbs / PEAK_HBM_GBS, "launches": t["merge_launches"], "traffic": measured_merge_traffic()}


BACKWARD_OTHER_WORKLOADS = ("128k-contiguous-causal",)
OTHER_WORKLOADS = ("32k-contiguous-causal", "32k-striped-causal", "32k-zigzag-causal", "128k-contiguous-causal",
                   "1m-zigzag-causal")


def measure_workloads(names=OTHER_WORKLOADS, reps: int = 3) -> list:
    """The forward call on the other named bf16 workloads (the other shard
    layouts and sizes), timed like the main line: useful TFLOP/s per call.
    Shares up to 128k tokens take 20 timed calls after at least 3 warm-up calls
    and 150 ms of them (a call is a few ms), the larger ones `reps` after one."""
    import torch

    import ring_attention_block_step_amd as ra
    import workloads as wl

    res = []
    for name in names:
        w = wl.WORKLOADS[name]
        rank = w.ranks[-1]
        k_glob, v_glob = wl.global_kv(w)
        idx = ra.shard_index(w.N, w.P, w.layout, rank)
        q = wl.query_rows(w, idx.numpy()).cuda()
        k = ra.pack_shards(k_glob, w.P, w.layout).cuda()
        v = ra.pack_shards(v_glob, w.P, w.layout).cuda()
        del k_glob, v_glob
        out = torch.empty_like(q)
        lse = torch.empty((w.Hq, w.b), dtype=torch.float32, device="cuda")
        small = w.N <= 131072
        n_warm, n_timed = (3, 20) if small else (1, reps)
        # Warm-up: at least n_warm calls and, for the small shares, 150 ms of
        # them (the first ~0.1 s of work after an idle spell runs a few percent
        # slow).
        t_warm = time.perf_counter()
        calls = 0
        while calls < n_warm or (small and time.perf_counter() - t_warm < 0.15):
            ra.forward(q, k, v, P=w.P, rank=rank, causal=w.causal, layout=w.layout, out=out, lse=lse)
            torch.cuda.synchronize()
            calls += 1
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(n_timed):
            ra.forward(q, k, v, P=w.P, rank=rank, causal=w.causal, layout=w.layout, out=out, lse=lse)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / n_timed
        flops = useful_flops(useful_pairs(w.layout, rank, w.P, w.b, w.causal), w.d, w.Hq)
        res.append({"workload": name, "layout": w.layout, "rank": rank, "ms_per_call": ms,
                    "value": flops / (ms * 1e-3) / 1e12, "unit": "TFLOP/s", "calls": n_timed})
        del q, k, v, out, lse
    return res


def compare_hop_modes(name: str, passes: int = 3) -> dict:
    """Forward call time of one workload under each hop schedule (fused,
    serial, streams), interleaved over `passes` passes after an untimed one
    (the order rotates, so that each schedule leads one pass),
    without the library's per-launch timing events; the outputs of every
    schedule must match the first bit for bit."""
    import torch

    import ring_attention_block_step_amd as ra
    import workloads as wl

    w = wl.WORKLOADS[name]
    rank = w.ranks[-1]
    k_glob, v_glob = wl.global_kv(w)
    idx = ra.shard_index(w.N, w.P, w.layout, rank)
    q = wl.query_rows(w, idx.numpy()).cuda()
    k = ra.pack_shards(k_glob, w.P, w.layout).cuda()
    v = ra.pack_shards(v_glob, w.P, w.layout).cuda()
    del k_glob, v_glob
    out = torch.empty_like(q)
    lse = torch.empty((w.Hq, w.b), dtype=torch.float32, device="cuda")
    n_timed = 20 if w.N <= 131072 else 2
    res = {m: [] for m in ra.HOP_MODES}
    ref = None
    identical = True
    try:
        for mode in ra.HOP_MODES:   # an untimed pass: clocks and caches settle before any figure
            ra.set_hop_mode(mode)
            for _ in range(n_timed):
                ra.forward(q, k, v, P=w.P, rank=rank, causal=w.causal, layout=w.layout, out=out, lse=lse)
        torch.cuda.synchronize()
        modes = list(ra.HOP_MODES)
        for p in range(passes):
            for mode in modes[p % 3:] + modes[:p % 3]:   # each schedule leads one pass
                ra.set_hop_mode(mode)
                for _ in range(2):
                    ra.forward(q, k, v, P=w.P, rank=rank, causal=w.causal, layout=w.layout, out=out, lse=lse)
                torch.cuda.synchronize()
                if ref is None:
                    ref = (out.clone(), lse.clone())
                identical = identical and torch.equal(out, ref[0]) and torch.equal(lse, ref[1])
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record()
                for _ in range(n_timed):
                    ra.forward(q, k, v, P=w.P, rank=rank, causal=w.causal, layout=w.layout, out=out, lse=lse)
                e1.record()
                torch.cuda.synchronize()
                res[mode].append(e0.elapsed_time(e1) / n_timed)
    finally:
        ra.set_hop_mode("fused")
    return {"workload": name, "ms_per_call": res, "calls_per_figure": n_timed, "bit_identical": identical}


def measure_reference_gemm(n: int = 16384, reps: int = 10) -> dict:
    """Context for the MFMA roofline, not a step of the path: the vendor
    library's dense bf16 GEMM (torch.matmul, which dispatches to hipBLASLt) on
    N(0,1) operands of n x n x n, timed with events on the same GPU in the same
    run.  Under sustained MFMA load the chip lowers its clock well below the
    2.4 GHz of the published peak, so this is the practical dense-MFMA rate the
    attention kernel is compared with."""
    import torch

    g = torch.Generator(device="cuda").manual_seed(11)
    a = torch.randn(n, n, device="cuda", generator=g).to(torch.bfloat16)
    b = torch.randn(n, n, device="cuda", generator=g).to(torch.bfloat16)
    for _ in range(3):
        c = a @ b
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        c = a @ b
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    tflops = 2.0 * n ** 3 / (ms * 1e-3) / 1e12
    # The same GEMM on constant operands (all ones): no operand toggles, so
    # the clock the power limit allows rises (compare the attention launches'
    # same_launches_on_constant_inputs).
    a.fill_(1.0)
    b.fill_(1.0)
    for _ in range(2):
        c = a @ b
    torch.cuda.synchronize()
    clock = ClockSampler()
    with clock:
        e0.record()
        for _ in range(reps):
            c = a @ b
        e1.record()
        torch.cuda.synchronize()
    cms = e0.elapsed_time(e1) / reps
    ctf = 2.0 * n ** 3 / (cms * 1e-3) / 1e12
    cs = clock.summary()
    del a, b, c
    return {"op": "bf16 GEMM (torch.matmul -> hipBLASLt), fp32 accumulate", "shape": [n, n, n], "ms": ms,
            "value": tflops, "unit": "TFLOP/s", "frac_of_peak": tflops / PEAK_BF16_TFLOPS,
            "constant_operands": {"inputs": "all ones", "ms": cms, "value": ctf, "frac_of_peak": ctf / PEAK_BF16_TFLOPS,
                                  "sclk_mean_mhz": cs["mean_mhz"] if cs else None}}


def measure_reference_attention(heads: int = 32, seq: int = 16384, d: int = 128, reps: int = 5) -> dict | None:
    """Context, not a step of the path: the vendor's own fused attention
    forward (torch's scaled_dot_product_attention restricted to its flash
    backend, bf16, causal, batch 1) on the same GPU in the same run, as useful
    (mask-aware) TFLOP/s: 4 d FLOPs per allowed pair and head.  Restricting the
    backend means a missing flash kernel raises here instead of running the
    bf16 math path; then the field is None."""
    import torch
    from torch.nn.attention import SDPBackend, sdpa_kernel

    g = torch.Generator(device="cuda").manual_seed(13)
    q, k, v = (torch.randn(1, heads, seq, d, device="cuda", generator=g).to(torch.bfloat16) for _ in range(3))
    try:
        with sdpa_kernel(SDPBackend.FLASH_ATTENTION):
            for _ in range(2):
                o = torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=True)
            torch.cuda.synchronize()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(reps):
                o = torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=True)
            e1.record()
            torch.cuda.synchronize()
    except RuntimeError as e:
        print(f"[bench] reference attention unavailable: {e}", file=sys.stderr, flush=True)
        return None
    ms = e0.elapsed_time(e1) / reps
    flops = useful_flops(seq * (seq + 1) // 2, d, heads)
    del q, k, v, o
    return {"op": "torch scaled_dot_product_attention, flash backend, bf16, causal", "shape":
            {"batch": 1, "heads": heads, "seq": seq, "d_h": d}, "ms": ms, "value": flops / (ms * 1e-3) / 1e12,
            "unit": "TFLOP/s", "frac_of_peak": flops / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS}


def measure_decode(name: str = "decode-31k-gqa64", reps: int = 20) -> dict:
    """Time ringattn_decode_partial on one resident shard of a decode workload
    (HIP events around the call's kernels, inside the library) and report the
    achieved GB/s of its algorithmic bytes against 8 TB/s."""
    import torch

    import ring_attention_block_step_amd as ra
    import workloads as wl

    w = wl.DECODE_WORKLOADS[name]
    q = wl.decode_query(w).cuda()
    k, v = (t.cuda() for t in wl.decode_shard(w, w.P - 1))
    m = torch.empty(w.Hq, w.n_q, device="cuda")
    z = torch.empty_like(m)
    y = torch.empty(w.n_q, w.Hq, w.d, device="cuda")
    for _ in range(3):
        ra.decode_partial(q, k, v, m=m, z=z, y=y)
    torch.cuda.synchronize()
    ra.timing_collect_decode()
    ra.timing_enable(True)
    for _ in range(reps):
        ra.decode_partial(q, k, v, m=m, z=z, y=y)
    torch.cuda.synchronize()
    ra.timing_enable(False)
    t = ra.timing_collect_decode()
    avg_ms = t["decode_ms"] / max(1, t["decode_calls"])
    nbytes = decode_bytes(w.n_q, w.n_keys, w.Hq, w.Hkv, w.d)
    gbs = nbytes / (avg_ms * 1e-3) / 1e9
    return {"kernel": "decode_chunk_kernel<128>+decode_combine_kernel<128>", "workload": name,
            "shape": {"n_q": w.n_q, "n_keys": w.n_keys, "Hq": w.Hq, "Hkv": w.Hkv, "d_h": w.d},
            "bytes_per_call": nbytes, "avg_call_ms": avg_ms, "achieved": gbs, "peak": PEAK_HBM_GBS,
            "unit": "GB/s", "frac": gbs / PEAK_HBM_GBS, "calls": t["decode_calls"]}


def backward_useful_flops(pairs: int, d: int, heads: int) -> float:
    """The backward of attention with recomputed scores: S = Q K^T again, then
    dV = P^T dO, dP = dO V^T, dQ = dS K, dK = dS^T Q: five contractions of
    2*d FLOPs per allowed pair and head, 10*d (2.5x the forward's)."""
    return 10.0 * d * pairs * heads


def measure_backward(name: str = "32k-contiguous-causal", reps: int = 3, constant_inputs: bool = False) -> dict:
    """Time ringattn_backward for the workload's rank (inputs: the GPU
    forward's O and LSE, a seeded upstream gradient) and report useful
    TFLOP/s per call and per step-kernel time against the bf16 peak, with the
    engine clock.  constant_inputs: also time the same calls on operands that
    do not toggle (Q = K = 0, V = 1, dO = 1), a clock/power diagnostic."""
    import torch

    import ring_attention_block_step_amd as ra
    import workloads as wl

    w = wl.WORKLOADS[name]
    rank = w.ranks[-1]
    k_glob, v_glob = wl.global_kv(w)
    idx = ra.shard_index(w.N, w.P, w.layout, rank)
    q = wl.query_rows(w, idx.numpy()).cuda()
    do = wl.token_rows(w.seed, "do", idx.numpy(), w.Hq, w.d, "normal", 1.0, w.torch_dtype).cuda()
    kp = ra.pack_shards(k_glob, w.P, w.layout).cuda()
    vp = ra.pack_shards(v_glob, w.P, w.layout).cuda()
    del k_glob, v_glob
    out, lse = ra.forward(q, kp, vp, P=w.P, rank=rank, causal=w.causal, layout=w.layout)
    dq = torch.empty(q.shape, dtype=torch.float32, device="cuda")
    dk = torch.zeros(kp.shape, dtype=torch.float32, device="cuda")
    dv = torch.zeros(kp.shape, dtype=torch.float32, device="cuda")
    # Warm-up: at least 2 calls and 150 ms of them (the first ~0.1 s of work
    # after an idle spell runs slow: a 32k call takes ~8 ms at first and
    # ~6.7 ms from the fifth on); shares of a few ms per call then time 10.
    t_warm = time.perf_counter()
    calls = 0
    while calls < 2 or time.perf_counter() - t_warm < 0.15:
        ra.backward(q, kp, vp, out, lse, do, P=w.P, rank=rank, causal=w.causal, layout=w.layout, dq=dq, dk=dk,
                    dv=dv)
        torch.cuda.synchronize()
        calls += 1
    if w.N <= 32768:
        reps = max(reps, 10)
    ra.timing_collect_backward()
    ra.timing_enable(True)
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    clock = ClockSampler()
    with clock:
        t0.record()
        for _ in range(reps):
            ra.backward(q, kp, vp, out, lse, do, P=w.P, rank=rank, causal=w.causal, layout=w.layout, dq=dq, dk=dk,
                        dv=dv)
        t1.record()
        torch.cuda.synchronize()
    ra.timing_enable(False)
    t = ra.timing_collect_backward()
    ms = t0.elapsed_time(t1) / reps
    flops = backward_useful_flops(useful_pairs(w.layout, rank, w.P, w.b, w.causal), w.d, w.Hq)
    kern_ms = t["step_ms"] / reps
    sclk = clock.summary()
    const = None
    if constant_inputs:
        zq, zk, ov, od = torch.zeros_like(q), torch.zeros_like(kp), torch.ones_like(vp), torch.ones_like(do)
        cout, clse = ra.forward(zq, zk, ov, P=w.P, rank=rank, causal=w.causal, layout=w.layout)
        for _ in range(2):
            ra.backward(zq, zk, ov, cout, clse, od, P=w.P, rank=rank, causal=w.causal, layout=w.layout, dq=dq,
                        dk=dk, dv=dv)
        torch.cuda.synchronize()
        cclock = ClockSampler()
        with cclock:
            t0.record()
            for _ in range(reps):
                ra.backward(zq, zk, ov, cout, clse, od, P=w.P, rank=rank, causal=w.causal, layout=w.layout, dq=dq,
                            dk=dk, dv=dv)
            t1.record()
            torch.cuda.synchronize()
        cms = t0.elapsed_time(t1) / reps
        cs = cclock.summary()
        const = {"inputs": "Q = K = 0, V = 1, dO = 1", "calls": reps, "ms_per_call": cms,
                 "value": flops / (cms * 1e-3) / 1e12, "unit": "TFLOP/s",
                 "frac_of_bf16_peak": flops / (cms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
                 "sclk_mean_mhz": cs["mean_mhz"] if cs else None,
                 "note": "same calls on non-toggling operands: the clock the power limit allows rises; not the metric"}
    return {"workload": name, "rank": rank, "useful_flops": flops, "ms_per_call": ms,
            "value": flops / (ms * 1e-3) / 1e12, "unit": "TFLOP/s",
            "kernels": "bwd_visit_kernel<128> (dK/dV and dQ workgroups)", "kernel_ms_per_call": kern_ms,
            "achieved": flops / (kern_ms * 1e-3) / 1e12, "peak": PEAK_BF16_TFLOPS,
            "frac": flops / (kern_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, "visits_per_call": t["step_launches"] / reps,
            "calls": reps, "sclk_mean_mhz": sclk["mean_mhz"] if sclk else None,
            "same_calls_on_constant_inputs": const,
            "note": "useful = 5 contractions per allowed pair; the kernels run 7 (the dQ workgroups recompute S, dP)"}


def measure_constant_inputs(w, rank: int, q, k, v, flops: float, reps: int = 5) -> dict:
    """The headline launches again on constant operands (Q = K = 0, V = 1):
    the same instruction stream (every score 0, every probability 1, the same
    tiles, hop copies and epilogue), but matrix-core operands that do not
    toggle.  The chip then holds a much higher engine clock than on the
    workload's random operands, which separates what the kernel's schedule
    sustains from what the power limit allows.  Context, not the metric."""
    import torch

    import ring_attention_block_step_amd as ra

    zq, zk, ov = torch.zeros_like(q), torch.zeros_like(k), torch.ones_like(v)
    out = torch.empty_like(q)
    lse = torch.empty((w.Hq, w.b), dtype=torch.float32, device=q.device)

    def run():
        ra.forward(zq, zk, ov, P=w.P, rank=rank, causal=w.causal, layout=w.layout, out=out, lse=lse)

    for _ in range(2):
        run()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    clock = ClockSampler()
    with clock:
        e0.record()
        for _ in range(reps):
            run()
        e1.record()
        torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    sclk = clock.summary()
    ok = bool(torch.all(out == 1).item())
    del zq, zk, ov, out, lse
    value = flops / (ms * 1e-3) / 1e12
    return {"inputs": "Q = K = 0, V = 1 (every probability 1, O = 1)", "output_is_one": ok, "calls": reps,
            "ms_per_call": ms, "value": value, "unit": "TFLOP/s", "frac_of_bf16_peak": value / PEAK_BF16_TFLOPS,
            "sclk_mean_mhz": sclk["mean_mhz"] if sclk else None,
            "note": "same launches on non-toggling operands: the clock the power limit allows rises; not the metric"}


def copy_calibration(nbytes: int, reps: int = 3) -> None:
    """A plain device copy of known size (torch's copy kernel), for scaling the
    FETCH_SIZE / WRITE_SIZE counters of other kernels."""
    import torch

    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": nbytes, "reps": reps}), flush=True)


# ---------------------------------------------------------------------------
# Main.
# ---------------------------------------------------------------------------

class ClockSampler:
    """The engine clock the kernel driver reports while the timed region runs:
    a background thread reads the current level of pp_dpm_sclk in sysfs every
    `period` seconds.  Used only when the machine shows exactly one such file (one
    GPU); otherwise, or on any read error, the summary is None."""

    PUBLISHED_MHZ = 2400.0

    def __init__(self, period: float = 0.01):
        import glob

        self.paths = sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk"))
        self.period = period
        self.samples = []
        self._stop = None
        self._thread = None

    def _read(self):
        import re

        with open(self.paths[0]) as f:
            for line in f:
                m = re.search(r"(\d+)\s*Mhz\s*\*", line)
                if m:
                    return float(m.group(1))
        return None

    def __enter__(self):
        import threading

        if len(self.paths) != 1:
            return self
        self._stop = threading.Event()

        def loop():
            while not self._stop.is_set():
                try:
                    v = self._read()
                except OSError:
                    return
                if v is not None:
                    self.samples.append(v)
                self._stop.wait(self.period)

        self._thread = threading.Thread(target=loop, daemon=True)
        self._thread.start()
        return self

    def __exit__(self, *exc):
        if self._thread is not None:
            self._stop.set()
            self._thread.join(timeout=1.0)
        return False

    def summary(self):
        if not self.samples:
            return None
        v = self.samples
        return {"mean_mhz": sum(v) / len(v), "min_mhz": min(v), "max_mhz": max(v), "samples": len(v),
                "source": self.paths[0] + " (current level)", "published_mhz": self.PUBLISHED_MHZ}


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="1m-contiguous-causal")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-merge", action="store_true", help="skip the merge-kernel measurement")
    ap.add_argument("--no-gemm-ref", action="store_true",
                    help="skip the vendor bf16 GEMM and attention reference measurements")
    ap.add_argument("--no-workloads", action="store_true", help="skip the forward on the other named workloads")
    ap.add_argument("--no-decode", action="store_true", help="skip the decode-kernel measurement")
    ap.add_argument("--no-constant-inputs", action="store_true",
                    help="skip the headline launches on constant operands (a clock/power diagnostic)")
    ap.add_argument("--decode-workload", default="decode-31k-gqa64",
                    help="decode workload of the decode-kernel measurement")
    ap.add_argument("--decode-only", action="store_true",
                    help="only run the decode-kernel measurement and print its JSON object")
    ap.add_argument("--no-backward", action="store_true", help="skip the backward measurement")
    ap.add_argument("--backward-workload", default="32k-contiguous-causal",
                    help="workload of the backward measurement")
    ap.add_argument("--backward-only", action="store_true",
                    help="only run the backward measurement and print its JSON object")
    ap.add_argument("--merge-only", action="store_true",
                    help="only run the merge-kernel measurement and print its JSON object")
    ap.add_argument("--hop-mode", default="fused", choices=("fused", "serial", "streams"),
                    help="schedule of the ring's hop copies (ringattn_set_hop_mode)")
    ap.add_argument("--hop-compare", action="store_true",
                    help="only time the forward of --workload under each hop schedule and print a JSON object")
    ap.add_argument("--copy-bytes", type=int, default=0,
                    help="only run a plain device copy of this many bytes (counter calibration)")
    args = ap.parse_args(argv)

    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported: the path is one "
              "device's share of the ring, and every GPU of a ring runs the same share", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import ring_attention_block_step_amd as ra
    import workloads as wl

    if not torch.cuda.is_available():
        print("bench.py needs a HIP device", file=sys.stderr)
        return 3
    ra.set_hop_mode(args.hop_mode)
    if args.decode_only:
        print(json.dumps(measure_decode(args.decode_workload)), flush=True)
        return 0
    if args.backward_only:
        print(json.dumps(measure_backward(args.backward_workload, reps=max(1, args.steps))), flush=True)
        return 0
    if args.merge_only:
        print(json.dumps(measure_merge()), flush=True)
        return 0
    if args.copy_bytes:
        copy_calibration(args.copy_bytes)
        return 0
    if args.hop_compare:
        print(json.dumps(compare_hop_modes(args.workload)), flush=True)
        return 0
    w = wl.WORKLOADS[args.workload]
    rank = w.ranks[-1]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    t_gen = time.perf_counter()
    k_glob, v_glob = wl.global_kv(w)
    idx = ra.shard_index(w.N, w.P, w.layout, rank)
    q = wl.query_rows(w, idx.numpy()).to(dev)
    k = ra.pack_shards(k_glob, w.P, w.layout).to(dev)
    v = ra.pack_shards(v_glob, w.P, w.layout).to(dev)
    out = torch.empty_like(q)
    lse = torch.empty((w.Hq, w.b), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()
    print(f"[bench] inputs ready in {time.perf_counter() - t_gen:.1f} s: {w.note}", file=sys.stderr, flush=True)

    def run():
        ra.forward(q, k, v, P=w.P, rank=rank, causal=w.causal, layout=w.layout, out=out, lse=lse)

    for _ in range(args.warmup):
        run()
    torch.cuda.synchronize()

    ra.timing_collect()
    ra.timing_enable(True)
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    clock = ClockSampler()
    t0 = time.perf_counter()
    with clock:
        start.record()
        for _ in range(args.steps):
            run()
        stop.record()
        torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    sclk = clock.summary()
    ra.timing_enable(False)
    kt = ra.timing_collect()
    ms_per_step = start.elapsed_time(stop) / args.steps
    print(f"[bench] {args.steps} steps: {ms_per_step:.3f} ms/step (host wall {wall:.3f} s)", file=sys.stderr,
          flush=True)

    pairs = useful_pairs(w.layout, rank, w.P, w.b, w.causal)
    flops = useful_flops(pairs, w.d, w.Hq)
    value = flops / (ms_per_step * 1e-3) / 1e12
    launches = kt["step_launches"]
    avg_launch_ms = kt["step_ms"] / max(1, launches)
    flops_per_launch = flops * args.steps / max(1, launches)
    achieved = flops_per_launch / (avg_launch_ms * 1e-3) / 1e12 if launches else None
    roofline = {
        "bound": "mfma",
        "achieved": achieved,
        "peak": PEAK_BF16_TFLOPS,
        "unit": "TFLOP/s",
        "frac": (achieved / PEAK_BF16_TFLOPS) if achieved else None,
        "traffic": measured_traffic(w.name),
        "kernel": "step_bf16_kernel<128>" if w.dtype == "bf16" else "step_f32_kernel",
        "avg_launch_ms": avg_launch_ms,
        "launches": launches,
        "flops_per_launch": flops_per_launch,
    }

    const_run = None
    if not args.no_constant_inputs and w.dtype == "bf16":
        const_run = measure_constant_inputs(w, rank, q, k, v, flops)
    merge = None if args.no_merge else measure_merge()
    gemm = None if args.no_gemm_ref else measure_reference_gemm()
    attn_ref = None if args.no_gemm_ref else measure_reference_attention()
    others = None if args.no_workloads else measure_workloads()
    decode = None if args.no_decode else measure_decode(args.decode_workload)
    backward = None if args.no_backward else measure_backward(args.backward_workload, reps=10,
                                                              constant_inputs=not args.no_constant_inputs)
    backward_other = None
    if not args.no_backward and not args.no_workloads:
        backward_other = [measure_backward(n, reps=2) for n in BACKWARD_OTHER_WORKLOADS if n != args.backward_workload]

    cpu, parity = None, None
    if not args.no_cpu_baseline:
        gpu_out = out.float().cpu().numpy()
        cpu, parity = cpu_baseline(w, rank, k_glob, v_glob, args.cpu_seconds, gpu_out)

    line = {
        "metric": "useful attention TFLOP/s per GPU (mask-aware) and % of bf16 MFMA peak",
        "value": value,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": "synthetic (seeded; Q,K,V as the workload states)",
        "config": {"workload": w.name, "N": w.N, "P": w.P, "b": w.b, "rank": rank, "layout": w.layout,
                   "causal": w.causal, "Hq": w.Hq, "Hkv": w.Hkv, "d_h": w.d, "useful_flops": flops,
                   "hop_mode": args.hop_mode},
        "pct_of_bf16_peak": 100.0 * value / PEAK_BF16_TFLOPS,
        "sclk_during_timed_region": sclk,
        "pct_of_bf16_peak_at_measured_clock": (100.0 * value / (PEAK_BF16_TFLOPS * sclk["mean_mhz"] /
                                                                 ClockSampler.PUBLISHED_MHZ)) if sclk else None,
        "roofline": roofline,
        "same_launches_on_constant_inputs": const_run,
        "cpu_baseline": cpu,
        "parity_sample": parity,
        "other_workloads": others,
        "reference_gemm": gemm,
        "step_kernel_vs_reference_gemm": (achieved / gemm["value"]) if (gemm and achieved) else None,
        "reference_attention": attn_ref,
        "value_vs_reference_attention": (value / attn_ref["value"]) if attn_ref else None,
        "merge_kernel": merge,
        "decode_kernel": decode,
        "backward": backward,
        "backward_other_workloads": backward_other,
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
