"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer
(CPU only).

A second build of libipttt.so instruments every host path -- argument
validation, workspace layouts, the host segment table, the packing of
document starts into launch arguments -- and the host ABI tests run against it
in a child process with the ASan runtime preloaded.  Any out-of-bounds access,
use of freed memory, signed overflow, misaligned or null dereference aborts the
child (halt_on_error), which fails this test.  Device code is built as usual
and never runs here.
"""
import os
import subprocess
import sys
import textwrap

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

from test_weight_mlp_amd import build as b  # noqa: E402

pytestmark = [pytest.mark.slow,
              pytest.mark.skipif(torch.cuda.is_available(),
                                 reason="host-only check: the launch set-up is driven with no device present")]

SOURCES = [os.path.join(b.CSRC, f) for f in os.listdir(b.CSRC)] + [os.path.join(ROOT, "include", "ipttt.h")]


@pytest.fixture(scope="module")
def sanitized():
    lib = b.SAN_LIB
    newest = max(os.path.getmtime(p) for p in SOURCES)
    if not os.path.exists(lib) or os.path.getmtime(lib) < newest:
        b.build(jobs=min(8, os.cpu_count() or 1), sanitize=True)
    syms = subprocess.run(["nm", "-D", lib], capture_output=True, text=True).stdout
    assert "__asan_report" in syms and "__ubsan_handle" in syms, "host code is not instrumented"
    env = dict(os.environ, LD_PRELOAD=b.sanitizer_runtime(), IPTTT_LIBRARY=lib,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    return lib, env


def _run(env, args, timeout=600):
    res = subprocess.run([sys.executable] + args, cwd=ROOT, env=env, capture_output=True, text=True,
                         timeout=timeout)
    report = res.stdout[-3000:] + res.stderr[-6000:]
    assert "ERROR: AddressSanitizer" not in report and "runtime error:" not in report, report
    assert res.returncode == 0, report
    return res.stdout


def test_host_abi_tests_clean_under_asan_and_ubsan(sanitized):
    lib, env = sanitized
    out = _run(env, ["-m", "pytest", "-q", "-p", "no:cacheprovider", "tests/test_abi_host.py"])
    assert " passed" in out and "failed" not in out


def test_launch_setup_paths_clean_under_asan_and_ubsan(sanitized):
    """Entry points that pass validation and reach the launch set-up: the
    document starts are packed into launch arguments in batches (more starts
    than one batch holds, continuing rows), the workspace is carved, and the
    first launch fails for want of a device, which the call reports."""
    lib, env = sanitized
    script = textwrap.dedent(f"""
        import ctypes, numpy as np
        import test_weight_mlp_amd as ip
        assert ip.library_path == {lib!r}
        lib = ip.library()
        maps = open("/proc/self/maps").read()
        assert {lib!r} in maps and "libclang_rt.asan" in maps
        v = ctypes.c_void_p
        rng = np.random.default_rng(5)
        T, rows = 4096, 3
        starts = np.sort(rng.choice(np.arange(1, rows * T), 1000, replace=False)).astype(np.int64)
        for cont in (None, [1, 0, 1]):
            p = ip.Problem(rows, T, 64, 128, 64, ip.IPTTT_BF16, starts, continues=cont)
            ws = ip.ipttt_workspace_bytes(p)
            bws = ip.ipttt_backward_workspace_bytes(p)
            HIP = 7
            assert lib.ipttt_segments_device(p.ref, v(256), v(256), None) == HIP
            assert lib.ipttt_target(p.ref, v(256), v(256), v(256), v(256), v(256), ws, None) == HIP
            assert lib.ipttt_chunk_delta(p.ref, v(256), v(256), 1e-3, 1e-5, v(256), None, v(256), ws, None) == HIP
            assert lib.ipttt_scan_apply(p.ref, v(256), v(256), v(256), v(256), 1e-3, v(256), v(256), ws,
                                        None) == HIP
            assert lib.ipttt_scan_apply_backward(p.ref, v(256), v(256), v(256), 1e-3, 1e-5, v(256), v(256),
                                                 v(256), v(256), v(256), bws, None) == HIP
            tbl = ip.ipttt_segment_table(p)
            assert tbl.shape == (rows, T // 64, 3)
        print("launch set-up paths ok")
    """)
    out = _run(env, ["-c", script])
    assert "launch set-up paths ok" in out
