"""The C ABI without a GPU: the library loads, exports every declared symbol, and
rejects bad arguments before making any HIP call."""

import ctypes
import os
import re
import subprocess

import pytest

import ring_attention_block_step_amd as ra

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ringattn.h")

FAKE = ctypes.c_void_p(0x10000)        # aligned, never dereferenced on these paths
MISALIGNED = ctypes.c_void_p(0x10008)


def _lib():
    if not os.path.exists(ra.LIB_PATH):
        pytest.skip("library not built (run __graft_entry__.build())")
    return ra.lib()


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"\b(ringattn_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_binding_symbols():
    assert _declared() == sorted(ra.SYMBOLS)


def test_library_exports_every_declared_symbol():
    L = _lib()
    for name in _declared():
        assert hasattr(L, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", ra.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\b(ringattn_[a-z0-9_]+)\b", out))
    assert set(_declared()) <= exported


def test_version_and_status_strings():
    L = _lib()
    assert b"gfx950" in L.ringattn_version()
    assert L.ringattn_status_string(0) == b"ok"
    assert L.ringattn_status_string(1) == b"invalid argument"
    assert L.ringattn_status_string(2) == b"unsupported"
    assert L.ringattn_status_string(3) == b"HIP runtime error"


def _fwd(fn, **kw):
    args = dict(q=FAKE, k=FAKE, v=FAKE, out=FAKE, lse=None, N=1024, P=4, rank=0, Hq=4, Hkv=2, d=128,
                causal=1, layout=0, stream=None)
    args.update(kw)
    return fn(args["q"], args["k"], args["v"], args["out"], args["lse"], args["N"], args["P"], args["rank"],
              args["Hq"], args["Hkv"], args["d"], args["causal"], args["layout"], args["stream"])


@pytest.mark.parametrize("entry", ["ringattn_forward", "ringattn_forward_f32"])
@pytest.mark.parametrize("kw,status,needle", [
    (dict(q=None), 1, "non-null"),
    (dict(out=None), 1, "non-null"),
    (dict(k=MISALIGNED), 1, "aligned"),
    (dict(lse=MISALIGNED), 1, "aligned"),
    (dict(P=0), 1, "P must be"),
    (dict(N=3, P=4), 1, "N must be >= P"),
    (dict(N=1023), 1, "multiple of P"),
    (dict(rank=4), 1, "rank"),
    (dict(rank=-1), 1, "rank"),
    (dict(Hq=3, Hkv=2), 1, "Hq"),
    (dict(Hkv=0), 1, "Hq"),
    (dict(causal=2), 1, "causal"),
    (dict(layout=3), 1, "layout"),
    (dict(layout=-1), 1, "layout"),
    (dict(layout=2, N=1028), 1, "multiple of 2P"),
    (dict(d=96), 2, "d_h"),
    (dict(d=256), 2, "d_h"),
    (dict(N=1 << 31, P=4, Hq=4, Hkv=2), 2, "too large"),
    (dict(N=4 << 20, P=4, Hq=64, Hkv=8), 2, "too large"),
    (dict(N=1024, P=4, Hq=1 << 17, Hkv=1 << 17), 2, "key/value heads"),
])
def test_forward_rejects_bad_arguments(entry, kw, status, needle):
    L = _lib()
    rc = _fwd(getattr(L, entry), **kw)
    assert rc == status
    assert needle in L.ringattn_last_error().decode()


def test_merge_rejects_bad_arguments_and_accepts_empty():
    L = _lib()
    m = L.ringattn_merge
    assert m(None, FAKE, FAKE, 2, 10, 4, 128, FAKE, 0, None, None) == 1
    assert m(FAKE, FAKE, FAKE, 0, 10, 4, 128, FAKE, 0, None, None) == 1
    assert m(FAKE, FAKE, FAKE, 2, -1, 4, 128, FAKE, 0, None, None) == 1
    assert m(FAKE, FAKE, FAKE, 2, 10, 0, 128, FAKE, 0, None, None) == 1
    assert m(FAKE, FAKE, FAKE, 2, 10, 4, 128, FAKE, 2, None, None) == 1
    assert m(FAKE, FAKE, MISALIGNED, 2, 10, 4, 128, FAKE, 0, None, None) == 1
    assert m(FAKE, FAKE, FAKE, 2, 10, 4, 32, FAKE, 0, None, None) == 2
    assert m(FAKE, FAKE, FAKE, 2, 1 << 29, 4, 128, FAKE, 0, None, None) == 2
    assert "too many rows" in L.ringattn_last_error().decode()
    # zero rows: valid, nothing to do, no HIP call
    assert m(FAKE, FAKE, FAKE, 2, 0, 4, 128, FAKE, 0, None, None) == 0


def test_decode_rejects_bad_arguments():
    L = _lib()
    d = L.ringattn_decode_partial
    # q, k, v, n_q, n_keys, Hq, Hkv, d_h, m, z, y, stream
    assert d(None, FAKE, FAKE, 1, 10, 4, 1, 128, FAKE, FAKE, FAKE, None) == 1
    assert d(FAKE, None, FAKE, 1, 10, 4, 1, 128, FAKE, FAKE, FAKE, None) == 1
    assert d(FAKE, FAKE, FAKE, 1, 10, 4, 1, 128, None, FAKE, FAKE, None) == 1
    assert d(MISALIGNED, FAKE, FAKE, 1, 10, 4, 1, 128, FAKE, FAKE, FAKE, None) == 1
    assert d(FAKE, FAKE, FAKE, 1, 10, 4, 1, 128, ctypes.c_void_p(0x10002), FAKE, FAKE, None) == 1
    assert d(FAKE, FAKE, FAKE, 1, 10, 4, 1, 128, FAKE, FAKE, MISALIGNED, None) == 1
    assert d(FAKE, FAKE, FAKE, 0, 10, 4, 1, 128, FAKE, FAKE, FAKE, None) == 1
    assert d(FAKE, FAKE, FAKE, 1, -1, 4, 1, 128, FAKE, FAKE, FAKE, None) == 1
    assert d(FAKE, FAKE, FAKE, 1, 10, 6, 4, 128, FAKE, FAKE, FAKE, None) == 1
    assert "Hq" in L.ringattn_last_error().decode()
    assert d(FAKE, FAKE, FAKE, 1, 10, 4, 1, 96, FAKE, FAKE, FAKE, None) == 2
    assert "d_h" in L.ringattn_last_error().decode()
    assert d(FAKE, FAKE, FAKE, 1 << 20, 10, 1, 1, 128, FAKE, FAKE, FAKE, None) == 2
    assert "too large" in L.ringattn_last_error().decode()


def test_decode_noalloc_rejects_bad_arguments_and_calls_beyond_its_scratch():
    """The allocation-free decode checks its arguments like the decode entry
    point and refuses a call whose chunk partials exceed its 32 MiB static
    buffer, before any HIP call: ceil(1e6 / 256) chunks x 8 key/value heads x
    8 rows x (128 + 2) floats is about 130 MB."""
    L = _lib()
    d = L.ringattn_decode_partial_noalloc
    assert d(None, FAKE, FAKE, 1, 10, 4, 1, 128, FAKE, FAKE, FAKE, None) == 1
    assert d(FAKE, FAKE, FAKE, 1, 10, 6, 4, 128, FAKE, FAKE, FAKE, None) == 1
    assert d(FAKE, FAKE, FAKE, 1, 10, 4, 1, 96, FAKE, FAKE, FAKE, None) == 2
    assert d(FAKE, FAKE, FAKE, 1, 10 ** 6, 64, 8, 128, FAKE, FAKE, FAKE, None) == 2
    assert "scratch" in L.ringattn_last_error().decode()


def test_backward_rejects_bad_arguments():
    L = _lib()
    f32 = ctypes.POINTER(ctypes.c_float)
    fk = ctypes.cast(FAKE, f32)
    fm = ctypes.cast(MISALIGNED, f32)

    def bwd(**kw):
        g = dict(q=FAKE, k=FAKE, v=FAKE, out=FAKE, lse=fk, dout=FAKE, dq=fk, dk=fk, dv=fk, N=1024, P=4, rank=0,
                 Hq=4, Hkv=2, d=128, causal=1, layout=0)
        g.update(kw)
        return L.ringattn_backward(g["q"], g["k"], g["v"], g["out"], g["lse"], g["dout"], g["dq"], g["dk"],
                                   g["dv"], g["N"], g["P"], g["rank"], g["Hq"], g["Hkv"], g["d"], g["causal"],
                                   g["layout"], None)

    for kw, status, needle in [
        (dict(lse=None), 1, "non-null"),
        (dict(dout=None), 1, "non-null"),
        (dict(dk=None), 1, "non-null"),
        (dict(dq=fm), 1, "aligned"),
        (dict(dout=MISALIGNED), 1, "aligned"),
        (dict(q=None), 1, "non-null"),
        (dict(P=0), 1, "P must be"),
        (dict(rank=4), 1, "rank"),
        (dict(Hq=3), 1, "Hq"),
        (dict(layout=2, N=1028), 1, "multiple of 2P"),
        (dict(d=96), 2, "d_h"),
        (dict(N=1 << 31), 2, "too large"),
    ]:
        assert bwd(**kw) == status, kw
        assert needle in L.ringattn_last_error().decode(), (kw, L.ringattn_last_error())


def test_timing_collect_empty():
    _lib()
    ra.timing_enable(False)
    assert ra.timing_collect() == {"step_ms": 0.0, "step_launches": 0, "merge_ms": 0.0, "merge_launches": 0}


def test_hop_mode_accepts_the_three_schedules_and_rejects_others():
    L = _lib()
    for mode in (3, -1, 100):
        assert L.ringattn_set_hop_mode(mode) == 1
        assert "hop mode" in L.ringattn_last_error().decode()
    for name in ("serial", "streams", "fused"):
        ra.set_hop_mode(name)
    assert L.ringattn_set_serial_hops(1) == 0 and L.ringattn_set_serial_hops(0) == 0


def test_binding_raises_on_error_status():
    L = _lib()
    rc = _fwd(L.ringattn_forward, P=0)
    with pytest.raises(ra.RingAttnError) as ei:
        ra._check(rc)
    assert ei.value.status == 1


def test_shard_helpers_match_layout_definitions():
    import torch
    N, P = 24, 4
    b = N // P
    for r in range(P):
        assert ra.shard_index(N, P, "contiguous", r).tolist() == list(range(r * b, r * b + b))
        assert ra.shard_index(N, P, "striped", r).tolist() == [j * P + r for j in range(b)]
        c = b // 2
        assert ra.shard_index(N, P, "zigzag", r).tolist() == \
            list(range(r * c, r * c + c)) + list(range((2 * P - 1 - r) * c, (2 * P - r) * c))
    x = torch.arange(N * 3).view(N, 3)
    for layout in ("contiguous", "striped", "zigzag"):
        packed = ra.pack_shards(x, P, layout)
        for r in range(P):
            assert torch.equal(packed[r], x[ra.shard_index(N, P, layout, r)])


def test_bench_clock_sampler_reads_the_current_level(tmp_path):
    """The bench's clock sampler takes the level marked '*' of a pp_dpm_sclk
    file and summarises what it read while its block ran."""
    import time

    import bench

    f = tmp_path / "pp_dpm_sclk"
    f.write_text("S: 1620Mhz *\n0: 500Mhz\n1: 2400Mhz\n")
    c = bench.ClockSampler(period=0.005)
    c.paths = [str(f)]
    with c:
        time.sleep(0.05)
    s = c.summary()
    assert s is not None and s["mean_mhz"] == 1620.0 and s["samples"] >= 2
    f.write_text("0: 500Mhz\n1: 2400Mhz *\n")
    assert c._read() == 2400.0
    none = bench.ClockSampler()
    none.paths = []
    with none:
        pass
    assert none.summary() is None


def test_bench_traffic_is_null_for_another_kernel_source(monkeypatch):
    """The bench reports `traffic` from a committed counter record only while
    the kernel source it was taken on is unchanged."""
    import json

    import bench

    with open(bench.MERGE_TRAFFIC_FILE) as f:
        rec = json.load(f)
    monkeypatch.setattr(bench, "source_digest", lambda path=None: rec["merge_source_sha256_16"])
    assert bench.measured_merge_traffic() == rec["bytes_per_launch"]
    monkeypatch.setattr(bench, "source_digest", lambda path=None: "0" * 16)
    assert bench.measured_merge_traffic() is None
    assert bench.measured_traffic("1m-contiguous-causal") is None
