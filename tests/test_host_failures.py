"""Failure handling of the C ABI on the host, without a GPU.

- A call with valid arguments on a host that has no GPU fails at its first HIP
  runtime call and reports RINGATTN_EHIP with a message; nothing aborts.
- The driver's host code, built with AddressSanitizer (host side only), runs
  every entry point's argument validation and the no-GPU failure path without
  a memory error.

Both use aligned stand-in pointers that no path here dereferences, so they
only run where no GPU is present.
"""

from __future__ import annotations

import ctypes
import os
import subprocess

import pytest

import ring_attention_block_step_amd as ra
from ring_attention_block_step_amd import build as rbuild

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.dirname(os.path.abspath(__file__))

needs_no_gpu = pytest.mark.skipif(os.path.exists("/dev/kfd"),
                                  reason="a GPU is present: the stand-in pointers would reach a kernel")

FAKE = ctypes.c_void_p(0x10000)


def _lib():
    if not os.path.exists(ra.LIB_PATH):
        pytest.skip("library not built (run __graft_entry__.build())")
    return ra.lib()


@needs_no_gpu
def test_valid_calls_without_a_gpu_return_ehip_with_a_message():
    L = _lib()
    F = FAKE
    calls = {
        "forward": lambda: L.ringattn_forward(F, F, F, F, F, 1024, 4, 3, 4, 2, 128, 1, 0, None),
        "forward_f32": lambda: L.ringattn_forward_f32(F, F, F, F, None, 1024, 4, 0, 4, 2, 64, 0, 1, None),
        "backward": lambda: L.ringattn_backward(F, F, F, F, F, F, F, F, F, 1024, 4, 1, 4, 2, 128, 1, 2, None),
        "merge": lambda: L.ringattn_merge(F, F, F, 2, 10, 4, 128, F, 0, F, None),
        "decode_partial": lambda: L.ringattn_decode_partial(F, F, F, 1, 1000, 8, 2, 128, F, F, F, None),
    }
    for name, call in calls.items():
        rc = call()
        msg = L.ringattn_last_error().decode()
        assert rc == 3, (name, rc, msg)
        assert "failed" in msg and len(msg) > 10, (name, msg)
    with pytest.raises(ra.RingAttnError) as ei:
        ra.redo_count()
    assert ei.value.status == 3


def _tool(path):
    return path if os.path.exists(path) else None


@needs_no_gpu
def test_host_address_sanitizer_build_of_the_argument_checks(tmp_path):
    """Build the driver's host code with AddressSanitizer, link it with the
    library's other objects and a small C++ driver program, and run every
    entry point's validation plus the no-GPU failure path."""
    clangxx = _tool("/opt/rocm/llvm/bin/clang++")
    objdir = os.path.join(ROOT, "_build", "obj")
    others = [os.path.join(objdir, s.replace(".hip", ".o")) for s in rbuild.SOURCES if s != "driver.hip"]
    if clangxx is None or not all(os.path.exists(o) for o in others):
        pytest.skip("needs the ROCm clang and the library's objects (run __graft_entry__.build())")
    hipcc = rbuild.hipcc()
    drv = tmp_path / "driver_asan.o"
    main = tmp_path / "main_asan.o"
    exe = tmp_path / "asan_check"
    common = ["-O1", "-g", "-std=c++20", "-fPIC", "-I", os.path.join(ROOT, "include")]
    # Host code only: every sanitizer flag goes to the host pass.
    subprocess.run([hipcc, *common, f"--offload-arch={rbuild.ARCH}", "-Xarch_host", "-fsanitize=address",
                    "-Xarch_host", "-fno-omit-frame-pointer", "-c",
                    os.path.join(rbuild.CSRC, "driver.hip"), "-o", str(drv)], check=True, capture_output=True)
    subprocess.run([clangxx, *common, "-fsanitize=address", "-fno-omit-frame-pointer", "-c",
                    os.path.join(HERE, "host_asan_main.cpp"), "-o", str(main)], check=True, capture_output=True)
    subprocess.run([clangxx, "-fsanitize=address", str(main), str(drv), *others, "-L/opt/rocm/lib",
                    "-Wl,-rpath,/opt/rocm/lib", "-lamdhip64", "-o", str(exe)], check=True, capture_output=True)
    # The environment may preload a library ahead of the sanitizer's runtime,
    # which is harmless here: the instrumented code is the executable's own.
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:exitcode=99:verify_asan_link_order=0")
    res = subprocess.run([str(exe), "--no-gpu"], capture_output=True, text=True, env=env, timeout=120)
    print(res.stdout[-3000:])
    assert "AddressSanitizer" not in res.stderr, res.stderr[-3000:]
    assert res.returncode == 0, (res.returncode, res.stdout[-2000:], res.stderr[-2000:])
    assert "ALL OK" in res.stdout
