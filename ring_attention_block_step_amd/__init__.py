"""One device's share of Ring Attention on MI355X (gfx950): the forward ring
step, the merge of partial triples, pass-Q decode and the backward ring.

Python binding of ``libringattn.so`` (C ABI: ``include/ringattn.h``).  It only
marshals arguments: it checks torch tensors, passes their device pointers and
the current HIP stream, and raises on a non-zero status.  Every step of the
computation runs in the library's HIP kernels; there is no CPU or PyTorch
fallback, and using any entry point without the built library raises.

Names follow the C ABI: ``forward`` (``ringattn_forward`` for bf16,
``ringattn_forward_f32`` for fp32), ``merge`` (``ringattn_merge``),
``decode_partial`` (``ringattn_decode_partial``), ``backward``
(``ringattn_backward``).
"""

from __future__ import annotations

import ctypes
import os

import torch

__all__ = ["forward", "backward", "merge", "decode_partial", "decode_partial_noalloc", "shard_index", "pack_shards", "lib", "RingAttnError",
           "timing_enable", "timing_collect", "timing_collect_decode", "timing_collect_backward", "set_serial_hops", "set_hop_mode", "HOP_MODES",
           "redo_count", "version", "SYMBOLS", "LIB_PATH"]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libringattn.so")
LAYOUTS = {"contiguous": 0, "striped": 1, "zigzag": 2}

# Every symbol include/ringattn.h declares.
SYMBOLS = ("ringattn_forward", "ringattn_forward_f32", "ringattn_backward", "ringattn_merge",
           "ringattn_decode_partial", "ringattn_decode_partial_noalloc", "ringattn_status_string", "ringattn_last_error", "ringattn_timing_enable",
           "ringattn_timing_collect", "ringattn_timing_collect_backward", "ringattn_timing_collect_decode",
           "ringattn_redo_count", "ringattn_set_hop_mode", "ringattn_set_serial_hops", "ringattn_version")

_lib = None


class RingAttnError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(message)
        self.status = status


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run `python -m ring_attention_block_step_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, f32p = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_void_p
    fwd = [vp, vp, vp, vp, f32p, i64, i32, i32, i32, i32, i32, i32, i32, vp]
    L.ringattn_forward.argtypes = fwd
    L.ringattn_forward.restype = i32
    L.ringattn_forward_f32.argtypes = fwd
    L.ringattn_forward_f32.restype = i32
    L.ringattn_merge.argtypes = [vp, vp, vp, i32, i64, i32, i32, vp, i32, f32p, vp]
    L.ringattn_merge.restype = i32
    L.ringattn_backward.argtypes = [vp, vp, vp, vp, f32p, vp, f32p, f32p, f32p, i64, i32, i32, i32, i32, i32, i32,
                                    i32, vp]
    L.ringattn_backward.restype = i32
    L.ringattn_timing_collect_backward.argtypes = [ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int64)]
    L.ringattn_timing_collect_backward.restype = i32
    L.ringattn_decode_partial.argtypes = [vp, vp, vp, i32, i64, i32, i32, i32, vp, vp, vp, vp]
    L.ringattn_decode_partial.restype = i32
    L.ringattn_decode_partial_noalloc.argtypes = [vp, vp, vp, i32, i64, i32, i32, i32, vp, vp, vp, vp]
    L.ringattn_decode_partial_noalloc.restype = i32
    L.ringattn_status_string.argtypes = [i32]
    L.ringattn_status_string.restype = ctypes.c_char_p
    L.ringattn_last_error.argtypes = []
    L.ringattn_last_error.restype = ctypes.c_char_p
    L.ringattn_timing_enable.argtypes = [i32]
    L.ringattn_timing_enable.restype = i32
    L.ringattn_timing_collect.argtypes = [ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int64),
                                          ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int64)]
    L.ringattn_timing_collect.restype = i32
    L.ringattn_timing_collect_decode.argtypes = [ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int64)]
    L.ringattn_timing_collect_decode.restype = i32
    L.ringattn_redo_count.argtypes = [ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(ctypes.c_int64)]
    L.ringattn_redo_count.restype = i32
    L.ringattn_set_serial_hops.argtypes = [i32]
    L.ringattn_set_serial_hops.restype = i32
    L.ringattn_set_hop_mode.argtypes = [i32]
    L.ringattn_set_hop_mode.restype = i32
    L.ringattn_version.argtypes = []
    L.ringattn_version.restype = ctypes.c_char_p
    _lib = L
    return L


def _check(rc: int) -> None:
    if rc != 0:
        L = lib()
        raise RingAttnError(rc, f"{L.ringattn_status_string(rc).decode()}: {L.ringattn_last_error().decode()}")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(dev: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _need(cond: bool, msg: str) -> None:
    if not cond:
        raise ValueError(msg)


# ---------------------------------------------------------------------------
# Caller-side data arrangement (not part of the step; plain torch indexing).
# ---------------------------------------------------------------------------

def shard_index(N: int, P: int, layout: str, r: int) -> torch.Tensor:
    """Global token indices held by shard r, in its local row order."""
    _need(N % P == 0, "N must be a multiple of P")
    b = N // P
    grid = torch.arange(N, dtype=torch.int64)
    if layout == "contiguous":
        return grid.view(P, b)[r].clone()
    if layout == "striped":
        return grid.view(b, P)[:, r].clone()
    if layout == "zigzag":
        _need(N % (2 * P) == 0, "zigzag needs N to be a multiple of 2P")
        chunks = grid.view(2 * P, b // 2)
        return torch.cat([chunks[r], chunks[2 * P - 1 - r]])
    raise ValueError(f"unknown layout {layout!r}")


def pack_shards(x: torch.Tensor, P: int, layout: str) -> torch.Tensor:
    """[N, ...] in global token order -> [P, N/P, ...] shard-major, contiguous."""
    N = x.shape[0]
    _need(N % P == 0, "N must be a multiple of P")
    b = N // P
    if layout == "contiguous":
        return x.reshape(P, b, *x.shape[1:]).contiguous()
    if layout == "striped":
        return x.reshape(b, P, *x.shape[1:]).transpose(0, 1).contiguous()
    if layout == "zigzag":
        _need(N % (2 * P) == 0, "zigzag needs N to be a multiple of 2P")
        chunks = x.reshape(2 * P, b // 2, *x.shape[1:])
        early, late = chunks[:P], chunks[P:].flip(0)   # shard r: chunk r, then chunk 2P-1-r
        return torch.stack([early, late], dim=1).reshape(P, b, *x.shape[1:]).contiguous()
    raise ValueError(f"unknown layout {layout!r}")


# ---------------------------------------------------------------------------
# Entry points.
# ---------------------------------------------------------------------------

def forward(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, *, P: int, rank: int, causal: bool,
            layout: str = "contiguous", out: torch.Tensor | None = None, lse: torch.Tensor | None = None,
            want_lse: bool = True):
    """Rank ``rank``'s share of the ring.

    q: [b, Hq, d] and k, v: [P, b, Hkv, d] on one HIP device, all bf16 or all
    fp32, contiguous.  Returns (out [b, Hq, d] in the input dtype, lse [Hq, b]
    fp32 natural log, or None when want_lse is False and no lse is given).
    Asynchronous on the current stream of q's device.
    """
    L = lib()
    _need(q.is_cuda and k.is_cuda and v.is_cuda, "q, k, v must be device tensors")
    _need(q.device == k.device == v.device, "q, k, v must be on one device")
    _need(q.dtype == k.dtype == v.dtype and q.dtype in (torch.bfloat16, torch.float32),
          "q, k, v must all be bfloat16 or all float32")
    _need(q.is_contiguous() and k.is_contiguous() and v.is_contiguous(), "q, k, v must be contiguous")
    _need(q.dim() == 3 and k.dim() == 4 and v.shape == k.shape, "q [b, Hq, d], k and v [P, b, Hkv, d]")
    b, Hq, d = q.shape
    _need(k.shape[0] == P and k.shape[1] == b and k.shape[3] == d, "k, v must be [P, b, Hkv, d] matching q")
    Hkv = k.shape[2]
    _need(layout in LAYOUTS, f"layout must be one of {sorted(LAYOUTS)}")
    if out is None:
        out = torch.empty_like(q)
    _need(out.shape == q.shape and out.dtype == q.dtype and out.is_contiguous() and out.device == q.device,
          "out must match q")
    if lse is None and want_lse:
        lse = torch.empty((Hq, b), dtype=torch.float32, device=q.device)
    if lse is not None:
        _need(lse.shape == (Hq, b) and lse.dtype == torch.float32 and lse.is_contiguous()
              and lse.device == q.device, "lse must be float32 [Hq, b] on q's device")
    fn = L.ringattn_forward if q.dtype == torch.bfloat16 else L.ringattn_forward_f32
    with torch.cuda.device(q.device):
        _check(fn(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), P * b, P, rank, Hq, Hkv, d,
                  int(bool(causal)), LAYOUTS[layout], _stream(q.device)))
    return out, lse


def backward(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, out: torch.Tensor, lse: torch.Tensor,
             dout: torch.Tensor, *, P: int, rank: int, causal: bool, layout: str = "contiguous",
             dk: torch.Tensor | None = None, dv: torch.Tensor | None = None, dq: torch.Tensor | None = None):
    """Rank ``rank``'s share of the backward ring.

    q, out, dout: [b, Hq, d] bf16; lse: [Hq, b] fp32 (the forward's); k, v:
    [P, b, Hkv, d] bf16.  Returns (dq [b, Hq, d], dk, dv [P, b, Hkv, d]), all
    fp32.  dk and dv are ADDED TO when given (zeros are made otherwise), so
    passing the same tensors for every rank accumulates the full gradients.
    Asynchronous on the current stream of q's device.
    """
    L = lib()
    ts = (q, k, v, out, dout)
    _need(all(t.is_cuda and t.device == q.device for t in ts + (lse,)), "all tensors must be on q's device")
    _need(all(t.dtype == torch.bfloat16 for t in ts), "q, k, v, out, dout must be bfloat16")
    _need(lse.dtype == torch.float32, "lse must be float32")
    _need(all(t.is_contiguous() for t in ts + (lse,)), "tensors must be contiguous")
    _need(q.dim() == 3 and k.dim() == 4 and v.shape == k.shape and out.shape == q.shape and dout.shape == q.shape,
          "q, out, dout [b, Hq, d]; k, v [P, b, Hkv, d]")
    b, Hq, d = q.shape
    _need(k.shape[0] == P and k.shape[1] == b and k.shape[3] == d, "k, v must be [P, b, Hkv, d] matching q")
    _need(tuple(lse.shape) == (Hq, b), "lse must be [Hq, b]")
    _need(layout in LAYOUTS, f"layout must be one of {sorted(LAYOUTS)}")
    if dq is None:
        dq = torch.empty((b, Hq, d), dtype=torch.float32, device=q.device)
    if dk is None:
        dk = torch.zeros(k.shape, dtype=torch.float32, device=q.device)
    if dv is None:
        dv = torch.zeros(k.shape, dtype=torch.float32, device=q.device)
    _need(dq.shape == q.shape and dq.dtype == torch.float32 and dq.is_contiguous(), "dq must be float32 [b, Hq, d]")
    for t, name in ((dk, "dk"), (dv, "dv")):
        _need(t.shape == k.shape and t.dtype == torch.float32 and t.is_contiguous() and t.device == q.device,
              f"{name} must be float32 [P, b, Hkv, d] on q's device")
    with torch.cuda.device(q.device):
        _check(L.ringattn_backward(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _ptr(dout), _ptr(dq), _ptr(dk),
                                   _ptr(dv), P * b, P, rank, Hq, k.shape[2], d, int(bool(causal)), LAYOUTS[layout],
                                   _stream(q.device)))
    return dq, dk, dv


def merge(m: torch.Tensor, z: torch.Tensor, y: torch.Tensor, *, out_dtype=torch.bfloat16,
          out: torch.Tensor | None = None, lse: torch.Tensor | None = None, want_lse: bool = True):
    """Combine partial triples: m, z [n, Hq, rows], y [n, rows, Hq, d], fp32.

    Returns (out [rows, Hq, d] in out_dtype, lse [Hq, rows] fp32 or None).
    """
    L = lib()
    _need(m.is_cuda and z.is_cuda and y.is_cuda and m.device == z.device == y.device,
          "m, z, y must be on one device")
    _need(m.dtype == z.dtype == y.dtype == torch.float32, "m, z, y must be float32")
    _need(m.is_contiguous() and z.is_contiguous() and y.is_contiguous(), "m, z, y must be contiguous")
    _need(m.dim() == 3 and z.shape == m.shape and y.dim() == 4, "m, z [n, Hq, rows]; y [n, rows, Hq, d]")
    n, Hq, rows = m.shape
    _need(y.shape[0] == n and y.shape[1] == rows and y.shape[2] == Hq, "y must be [n, rows, Hq, d]")
    d = y.shape[3]
    _need(out_dtype in (torch.bfloat16, torch.float32), "out_dtype must be bfloat16 or float32")
    if out is None:
        out = torch.empty((rows, Hq, d), dtype=out_dtype, device=m.device)
    _need(out.shape == (rows, Hq, d) and out.dtype == out_dtype and out.is_contiguous()
          and out.device == m.device, "out must be [rows, Hq, d] of out_dtype")
    if lse is None and want_lse:
        lse = torch.empty((Hq, rows), dtype=torch.float32, device=m.device)
    if lse is not None:
        _need(lse.shape == (Hq, rows) and lse.dtype == torch.float32 and lse.is_contiguous()
              and lse.device == m.device, "lse must be float32 [Hq, rows]")
    with torch.cuda.device(m.device):
        _check(L.ringattn_merge(_ptr(m), _ptr(z), _ptr(y), n, rows, Hq, d, _ptr(out),
                                0 if out_dtype == torch.bfloat16 else 1, _ptr(lse), _stream(m.device)))
    return out, lse


def decode_partial(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, *, m: torch.Tensor | None = None,
                   z: torch.Tensor | None = None, y: torch.Tensor | None = None, no_alloc: bool = False):
    """Partial (m, z, y) of new query rows q [n_q, Hq, d] against a resident
    shard k, v [n_keys, Hkv, d], all bf16 on one device (n_keys may be 0).

    Returns m, z [Hq, n_q] (natural log) and y [n_q, Hq, d], fp32; pass views
    of part p of merge's inputs ([P, Hq, n_q], [P, n_q, Hq, d]) to fill them
    in place.  Asynchronous on the current stream of q's device.  no_alloc:
    call ringattn_decode_partial_noalloc (the library's static scratch).
    """
    L = lib()
    _need(q.is_cuda and k.is_cuda and v.is_cuda and q.device == k.device == v.device,
          "q, k, v must be device tensors on one device")
    _need(q.dtype == k.dtype == v.dtype == torch.bfloat16, "q, k, v must be bfloat16")
    _need(q.is_contiguous() and k.is_contiguous() and v.is_contiguous(), "q, k, v must be contiguous")
    _need(q.dim() == 3 and k.dim() == 3 and v.shape == k.shape, "q [n_q, Hq, d], k and v [n_keys, Hkv, d]")
    n_q, Hq, d = q.shape
    n_keys, Hkv = k.shape[0], k.shape[1]
    _need(k.shape[2] == d, "k, v must have q's d")
    if m is None:
        m = torch.empty((Hq, n_q), dtype=torch.float32, device=q.device)
    if z is None:
        z = torch.empty((Hq, n_q), dtype=torch.float32, device=q.device)
    if y is None:
        y = torch.empty((n_q, Hq, d), dtype=torch.float32, device=q.device)
    for t, shape, name in ((m, (Hq, n_q), "m"), (z, (Hq, n_q), "z"), (y, (n_q, Hq, d), "y")):
        _need(tuple(t.shape) == shape and t.dtype == torch.float32 and t.is_contiguous() and t.device == q.device,
              f"{name} must be float32 {list(shape)} on q's device")
    with torch.cuda.device(q.device):
        fn = L.ringattn_decode_partial_noalloc if no_alloc else L.ringattn_decode_partial
        _check(fn(_ptr(q), _ptr(k) if n_keys else None, _ptr(v) if n_keys else None,
                  n_q, n_keys, Hq, Hkv, d, _ptr(m), _ptr(z), _ptr(y), _stream(q.device)))
    return m, z, y


def decode_partial_noalloc(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, *, m: torch.Tensor | None = None,
                           z: torch.Tensor | None = None, y: torch.Tensor | None = None):
    """decode_partial through ringattn_decode_partial_noalloc: the library
    allocates nothing (its chunk partials use a static 32 MiB device buffer;
    calls that overlap on one device race).  Outputs made here when not given
    are the caller's allocations."""
    return decode_partial(q, k, v, m=m, z=z, y=y, no_alloc=True)


def timing_enable(flag: bool = True) -> None:
    _check(lib().ringattn_timing_enable(int(bool(flag))))


def timing_collect() -> dict:
    """Summed kernel durations (ms) and launch counts since the last collect."""
    sm, mm = ctypes.c_double(), ctypes.c_double()
    sn, mn = ctypes.c_int64(), ctypes.c_int64()
    _check(lib().ringattn_timing_collect(ctypes.byref(sm), ctypes.byref(sn), ctypes.byref(mm), ctypes.byref(mn)))
    return {"step_ms": sm.value, "step_launches": sn.value, "merge_ms": mm.value, "merge_launches": mn.value}


def timing_collect_backward() -> dict:
    """Summed backward step-kernel durations (ms) and visit count since the last collect."""
    ms, n = ctypes.c_double(), ctypes.c_int64()
    _check(lib().ringattn_timing_collect_backward(ctypes.byref(ms), ctypes.byref(n)))
    return {"step_ms": ms.value, "step_launches": n.value}


def timing_collect_decode() -> dict:
    """Summed decode kernel durations (ms) and call count since the last collect."""
    ms, n = ctypes.c_double(), ctypes.c_int64()
    _check(lib().ringattn_timing_collect_decode(ctypes.byref(ms), ctypes.byref(n)))
    return {"decode_ms": ms.value, "decode_calls": n.value}


def redo_count() -> dict:
    """Step-kernel workgroups that redid their tiles on the exact path since the
    last call (all of them, and those that had been folding the carried state
    in late); waits for the current device and clears the counts."""
    a, b = ctypes.c_int64(), ctypes.c_int64()
    _check(lib().ringattn_redo_count(ctypes.byref(a), ctypes.byref(b)))
    return {"redone": a.value, "redone_late_fold": b.value}


HOP_MODES = {"fused": 0, "serial": 1, "streams": 2}


def set_hop_mode(mode: str) -> None:
    """Schedule of the ring's hop copies for later calls: "fused" (the step
    launch of visit i copies the block of visit i+1; the default), "serial"
    (copy kernels on the caller's stream) or "streams" (copy kernels on the
    library's second stream, ordered by events)."""
    _check(lib().ringattn_set_hop_mode(HOP_MODES[mode]))


def set_serial_hops(flag: bool) -> None:
    """True: hop copies serialised on the caller's stream; False: the default
    fused schedule."""
    _check(lib().ringattn_set_serial_hops(int(bool(flag))))


def version() -> str:
    return lib().ringattn_version().decode()
