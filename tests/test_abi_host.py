"""Host-side checks of the C ABI (no GPU): the library loads, exports every
symbol the header declares, rejects bad arguments before launching anything,
and its host segment table equals the oracle's independently derived one."""
import ctypes
import os
import re

import numpy as np
import pytest
import torch

import oracle
import test_weight_mlp_amd as ip
from test_weight_mlp_amd import inputs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

pytestmark = pytest.mark.skipif(not os.path.exists(ip.library_path),
                                reason="libipttt.so not built")


def _header_functions():
    text = open(os.path.join(ROOT, "include", "ipttt.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ipttt_[a-z_0-9]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    names = _header_functions()
    assert len(names) >= 10
    lib = ctypes.CDLL(ip.library_path)
    for n in names:
        assert hasattr(lib, n), n
    assert ip.ipttt_abi_version() == 10


def test_status_strings_cover_all_codes():
    lib = ip.library()
    for code in range(0, 10):
        assert lib.ipttt_status_string(code).decode() not in ("", "unknown status")
    assert lib.ipttt_status_string(99).decode() == "unknown status"


@pytest.mark.parametrize("kw,code", [
    (dict(rows=0), 2), (dict(seq_len=0), 2), (dict(d_model=12), 2), (dict(d_ff=4100 + 2), 2),
    (dict(chunk=0), 2), (dict(dtype=7), 3), (dict(d_model=1 << 21), 2),
    (dict(rows=1 << 20, seq_len=1 << 12), 2),
    # rows, and (row, chunk) pairs, ride in a launch grid's y dimension
    (dict(rows=65536, seq_len=1, chunk=1), 2), (dict(rows=1, seq_len=65536, chunk=1), 2),
    (dict(rows=4, seq_len=16384 * 4, chunk=4), 2),
    (dict(doc_starts=[5, 5]), 5), (dict(doc_starts=[9, 3]), 5), (dict(doc_starts=[-1]), 5),
    (dict(doc_starts=[64]), 5),
])
def test_validation_rejects(kw, code):
    base = dict(rows=2, seq_len=32, d_model=16, d_ff=32, chunk=8, dtype=ip.IPTTT_BF16)
    base.update(kw)
    p = ip.Problem(**base)
    assert ip.ipttt_validate(p) == code
    assert ip.ipttt_workspace_bytes(p) == 0


def test_validation_accepts_edge_cases():
    for kw in (dict(chunk=1000), dict(chunk=1), dict(doc_starts=[0, 32, 63]), dict(seq_len=1),
               dict(rows=65535, seq_len=1), dict(rows=1, seq_len=65535, chunk=1),
               dict(rows=5, seq_len=13107 * 4, chunk=4)):
        base = dict(rows=2, seq_len=32, d_model=16, d_ff=32, chunk=8, dtype=ip.IPTTT_F32)
        base.update(kw)
        assert ip.ipttt_validate(ip.Problem(**base)) == 0


def test_null_and_alignment_errors_before_any_launch():
    """Bad pointers come back as status codes; nothing touches a device (this
    runs on a host without a GPU)."""
    lib = ip.library()
    p = ip.Problem(1, 32, 16, 32, 8, ip.IPTTT_BF16)
    v = ctypes.c_void_p
    assert lib.ipttt_z(p.ref, None, v(256), v(256), v(256), None) == 1
    assert lib.ipttt_z(p.ref, v(258), v(256), v(256), v(256), None) == 4
    assert lib.ipttt_z(None, v(256), v(256), v(256), v(256), None) == 1
    ws = ip.ipttt_workspace_bytes(p)
    assert lib.ipttt_target(p.ref, v(256), v(256), v(256), v(256), v(256), ws - 1, None) == 6
    assert lib.ipttt_target(p.ref, v(256), v(256), v(256), v(256), None, ws, None) == 6
    assert lib.ipttt_target(p.ref, v(256), v(256), v(256), v(256), v(272), ws, None) == 4
    nan = float("nan")
    assert lib.ipttt_chunk_delta(p.ref, v(256), v(256), nan, 0.0, v(256), None, v(256), ws,
                                 None) == 8
    assert lib.ipttt_chunk_delta(p.ref, v(256), v(256), 1e-3, 0.0, None, None, v(256), ws,
                                 None) == 1
    assert lib.ipttt_chunk_delta(p.ref, v(256), v(256), 1e-3, 0.0, v(256), v(264), v(256), ws,
                                 None) == 4
    assert lib.ipttt_scan_apply(p.ref, v(256), v(256), v(256), v(256), float("inf"), v(256),
                                v(256), ws, None) == 8
    assert lib.ipttt_scan_apply(p.ref, v(256), None, v(256), v(256), 1e-3, v(256), v(256), ws,
                                None) == 1
    assert lib.ipttt_segments_device(p.ref, None, None, None) == 1
    # the carried state: aligned, and S_out either S_in itself or disjoint
    sc = lib.ipttt_scan_apply_carry
    assert sc(p.ref, v(256), v(256), v(256), v(256), 1e-3, v(260), None, v(256), v(256), ws, None) == 4
    assert sc(p.ref, v(256), v(256), v(256), v(256), 1e-3, None, v(264), v(256), v(256), ws, None) == 4
    sbytes = 1 * 16 * 32 * 4
    assert sc(p.ref, v(4096), v(4096), v(4096), v(4096), 1e-3, v(1 << 20), v((1 << 20) + sbytes - 16),
              v(4096), v(4096), ws, None) == 8
    assert sc(p.ref, v(256), v(256), v(256), v(256), float("nan"), None, None, v(256), v(256), ws,
              None) == 8
    assert sc(p.ref, v(256), v(256), None, v(256), 1e-3, None, None, v(256), v(256), ws, None) == 1


def test_workspace_is_dominated_by_per_chunk_weights():
    """64 per-chunk bf16 weights plus W_down in the same fragment layout, the
    scaled V_hat operand of the scan, and a little for the segment
    descriptors."""
    p = ip.Problem(1, 32768, 2560, 9728, 512, ip.IPTTT_BF16)
    ws = ip.ipttt_workspace_bytes(p)
    need = 65 * 2560 * 9728 * 2 + 32768 * 2560 * 2
    assert need <= ws < need + (1 << 20)


def test_workspace_holds_one_pass_of_rows():
    """The 8-wave scan and apply run in passes of whole rows whose per-chunk
    weights fit 4 GiB: the 8 x 32k packed workload (3.19 GB of weights per
    row) needs one row's worth, under 4 GB; rows that fit together share one
    pass."""
    packed = ip.Problem(8, 32768, 2560, 9728, 512, ip.IPTTT_BF16)
    one_row = 64 * 2560 * 9728 * 2 + 2560 * 9728 * 2 + 32768 * 2560 * 2
    ws = ip.ipttt_workspace_bytes(packed)
    assert one_row <= ws < one_row + 8 * (1 << 20) and ws < 4 * 10 ** 9
    small = ip.Problem(4, 8192, 1024, 4096, 512, ip.IPTTT_BF16)
    assert ip.ipttt_workspace_bytes(small) >= 4 * 16 * 1024 * 4096 * 2 + 4 * 8192 * 1024 * 2
    # the saved state still holds every row's weights
    assert ip.ipttt_saved_bytes(packed) == 8 * 64 * 2560 * 9728 * 2 + 2560 * 9728 * 2


def test_workspace_of_a_long_row_holds_one_window_of_chunks(monkeypatch):
    """A row whose per-chunk weights exceed the 4 GiB pass budget runs in
    windows of its chunks, each handing the fp32 state to the next: the
    workspace stays within the budget at 128k and 256k tokens and does not grow
    with the row's length; the budget can be set with IPTTT_PASS_BYTES."""
    monkeypatch.delenv("IPTTT_PASS_BYTES", raising=False)
    wd, st = 2560 * 9728 * 2, 2560 * 9728 * 4
    sizes = []
    for T in (131072, 262144, 524288):
        p = ip.Problem(1, T, 2560, 9728, 1024, ip.IPTTT_BF16)
        ws = ip.ipttt_workspace_bytes(p)
        # at least one window: one chunk's weights, its V_s, W_down's fragments, the state
        assert wd + 1024 * 2560 * 2 + wd + st <= ws <= 4 * 2 ** 30 + (8 << 20)
        sizes.append(ws)
    assert max(sizes) - min(sizes) < (8 << 20)
    p = ip.Problem(1, 131072, 2560, 9728, 1024, ip.IPTTT_BF16)
    monkeypatch.setenv("IPTTT_PASS_BYTES", str(wd + st + 3 * (wd + 1024 * 2560 * 2)))
    small = ip.ipttt_workspace_bytes(p)
    assert small < sizes[0]
    # a value that is not a positive decimal leaves the default
    monkeypatch.setenv("IPTTT_PASS_BYTES", "4GiB")
    assert ip.ipttt_workspace_bytes(p) == sizes[0]
    monkeypatch.setenv("IPTTT_PASS_BYTES", "0")
    assert ip.ipttt_workspace_bytes(p) == sizes[0]


def _random_starts(rng, rows, T, n):
    s = rng.choice(rows * T, size=min(n, rows * T), replace=False)
    return np.sort(s)


@pytest.mark.parametrize("seed", range(40))
def test_p13_host_segment_table_equals_oracle(seed):
    rng = np.random.default_rng(seed)
    rows = int(rng.integers(1, 4))
    T = int(rng.integers(1, 90))
    C = int(rng.integers(1, 40))
    starts = _random_starts(rng, rows, T, int(rng.integers(0, 12)))
    p = ip.Problem(rows, T, 8, 8, C, ip.IPTTT_F32, starts)
    assert ip.ipttt_validate(p) == 0
    got = ip.ipttt_segment_table(p)
    ref = oracle.segment_table(rows, T, C, starts)
    assert np.array_equal(got, ref.astype(np.int32))


def test_p13_host_segment_table_packed_4b_workload():
    cfg = inputs.CONFIGS["4b_packed"]
    starts = inputs.loguniform_doc_starts(cfg.rows, cfg.seq_len, cfg.chunk, seed=7)
    assert len(starts) > 8 and np.all(starts % cfg.chunk != 0)
    p = ip.Problem(cfg.rows, cfg.seq_len, 8, 8, cfg.chunk, ip.IPTTT_BF16, starts)
    got = ip.ipttt_segment_table(p)
    ref = oracle.segment_table(cfg.rows, cfg.seq_len, cfg.chunk, starts)
    assert np.array_equal(got, ref.astype(np.int32))


@pytest.mark.parametrize("seed", range(20))
def test_host_segment_table_with_continuing_rows_equals_oracle(seed):
    """Rows flagged as continuing a document of the previous call have no
    start at their first token (unless one is listed there)."""
    rng = np.random.default_rng(100 + seed)
    rows = int(rng.integers(1, 5))
    T = int(rng.integers(1, 90))
    C = int(rng.integers(1, 40))
    starts = _random_starts(rng, rows, T, int(rng.integers(0, 10)))
    cont = rng.integers(0, 2, rows).astype(np.uint8)
    p = ip.Problem(rows, T, 8, 8, C, ip.IPTTT_F32, starts, continues=cont)
    got = ip.ipttt_segment_table(p)
    ref = oracle.segment_table(rows, T, C, starts, continues=cont)
    assert np.array_equal(got, ref.astype(np.int32))


def test_continues_needs_one_flag_per_row():
    with pytest.raises(ValueError):
        ip.Problem(2, 32, 16, 32, 8, ip.IPTTT_BF16, continues=[1])


def test_p13_host_segment_table_golden(golden_dir):
    import json
    with open(os.path.join(golden_dir, "segment_tables.json")) as fh:
        g = json.load(fh)
    for case in g["cases"]:
        p = ip.Problem(case["rows"], case["T"], 8, 8, case["C"], ip.IPTTT_F32, case["doc_starts"])
        assert ip.ipttt_segment_table(p).tolist() == case["table"], case["name"]


def test_target_mode_validation():
    for t in (ip.IPTTT_TARGET_LM, ip.IPTTT_TARGET_NO_CONV, ip.IPTTT_TARGET_NO_PROJ):
        assert ip.ipttt_validate(ip.Problem(1, 32, 16, 32, 8, ip.IPTTT_BF16, target=t)) == 0
    for t in (-1, 3, 7):
        assert ip.ipttt_validate(ip.Problem(1, 32, 16, 32, 8, ip.IPTTT_BF16, target=t)) == 8
    # the unused weight of each mode may be NULL; the others may not
    lib = ip.library()
    v = ctypes.c_void_p
    p = ip.Problem(1, 32, 16, 32, 8, ip.IPTTT_BF16, target=ip.IPTTT_TARGET_LM)
    ws = ip.ipttt_workspace_bytes(p)
    assert lib.ipttt_target(p.ref, v(256), None, v(256), v(256), v(256), ws, None) == 1
    assert lib.ipttt_target(p.ref, v(256), v(256), None, v(256), v(256), ws, None) == 1
    p = ip.Problem(1, 32, 16, 32, 8, ip.IPTTT_BF16, target=ip.IPTTT_TARGET_NO_CONV)
    assert lib.ipttt_target(p.ref, v(256), v(256), None, v(256), v(256), ws, None) == 1
    p = ip.Problem(1, 32, 16, 32, 8, ip.IPTTT_BF16, target=ip.IPTTT_TARGET_NO_PROJ)
    assert lib.ipttt_target(p.ref, v(256), None, v(256), v(256), v(256), ws, None) == 1


def test_backward_argument_errors_before_any_launch():
    lib = ip.library()
    p = ip.Problem(1, 32, 16, 32, 8, ip.IPTTT_BF16)
    v = ctypes.c_void_p
    ws = ip.ipttt_backward_workspace_bytes(p)
    assert ws > ip.ipttt_workspace_bytes(p) > 0
    sab = lib.ipttt_scan_apply_backward
    assert sab(p.ref, v(256), v(256), v(256), 1e-3, 0.0, v(256), v(256), v(256), v(256), v(256), ws - 1,
               None) == 6
    assert sab(p.ref, v(256), v(256), v(256), 1e-3, 0.0, v(256), v(256), v(256), v(256), v(264), ws,
               None) == 4
    assert sab(p.ref, v(256), None, v(256), 1e-3, 0.0, v(256), v(256), v(256), v(256), v(256), ws, None) == 1
    assert sab(p.ref, v(256), v(256), v(256), float("inf"), 0.0, v(256), v(256), v(256), v(256), v(256), ws,
               None) == 8
    assert sab(p.ref, v(256), v(256), v(256), 1e-3, 0.0, v(256), v(258), v(256), v(256), v(256), ws,
               None) == 4
    tb = lib.ipttt_target_backward
    assert tb(p.ref, v(256), v(256), v(256), v(256), v(256), None, v(256), v(256), ws, None) == 1
    pn = ip.Problem(1, 32, 16, 32, 8, ip.IPTTT_BF16, target=ip.IPTTT_TARGET_NO_CONV)
    assert tb(pn.ref, v(256), None, v(256), v(256), None, None, v(256), v(256), ws, None) == 1
    zb = lib.ipttt_z_backward
    assert zb(p.ref, v(256), v(256), v(256), v(256), v(256), v(256), None, v(256), ws, None) == 1
    assert zb(p.ref, v(256), v(256), v(256), v(256), v(256), v(256), v(256), None, ws, None) == 6
    assert lib.ipttt_backward_workspace_bytes(None) == 0



def test_saved_state_sizes_and_argument_errors_before_any_launch():
    lib = ip.library()
    v = ctypes.c_void_p
    p = ip.Problem(1, 32, 64, 128, 8, ip.IPTTT_BF16)  # 4 chunks, the fast shapes
    need = ip.ipttt_saved_bytes(p)
    assert need == 4 * 64 * 128 * 2 + 64 * 128 * 2
    assert ip.ipttt_saved_bytes(ip.Problem(1, 32, 64, 128, 8, ip.IPTTT_F32)) == 0
    assert ip.ipttt_saved_bytes(ip.Problem(1, 32, 72, 128, 8, ip.IPTTT_BF16)) == 0
    assert lib.ipttt_saved_bytes(None) == 0
    ws = ip.ipttt_workspace_bytes(p)
    sv = lib.ipttt_scan_apply_save
    assert sv(p.ref, v(256), v(256), v(256), v(256), 1e-3, v(256), None, need, v(256), ws, None) == 1
    assert sv(p.ref, v(256), v(256), v(256), v(256), 1e-3, v(256), v(256), need - 1, v(256), ws, None) == 6
    assert sv(p.ref, v(256), v(256), v(256), v(256), 1e-3, v(256), v(272), need, v(256), ws, None) == 4
    bws = ip.ipttt_backward_workspace_bytes(p)
    sb = lib.ipttt_scan_apply_backward_saved
    args = lambda alpha, saved, n: (p.ref, v(256), v(256), v(256), 1e-3, 1e-5, alpha, saved, n, v(256), v(256),
                                    v(256), v(256), v(256), bws, None)
    assert sb(*args(None, v(256), need)) == 1
    assert sb(*args(v(258), v(256), need)) == 4
    assert sb(*args(v(256), v(256), need - 1)) == 6
    assert sb(*args(v(256), v(272), need)) == 4


def test_saved_gate_products_argument_errors_before_any_launch():
    lib = ip.library()
    v = ctypes.c_void_p
    p = ip.Problem(1, 32, 64, 128, 8, ip.IPTTT_BF16)
    zs = lib.ipttt_z_save
    assert zs(p.ref, v(256), v(256), v(256), v(256), None, None) == 1
    assert zs(p.ref, v(256), v(256), v(256), v(256), v(264), None) == 4
    bws = ip.ipttt_backward_workspace_bytes(p)
    zb = lib.ipttt_z_backward_saved
    assert zb(p.ref, v(256), v(256), v(256), None, v(256), v(256), v(256), v(256), v(256), bws, None) == 1
    assert zb(p.ref, v(256), v(256), v(256), v(264), v(256), v(256), v(256), v(256), v(256), bws, None) == 4
    assert zb(p.ref, v(256), v(256), v(256), v(256), v(256), v(256), v(256), v(256), v(256), bws - 1, None) == 6


def test_chunks_too_long_for_32_bit_offsets_take_the_general_kernels():
    """The 8-wave scan, reverse scan and backward products address the rows of
    one chunk through 32-bit buffer offsets; a chunk whose (C + 64) rows of
    max(d_model, d_ff) bf16 reach 2^31 bytes goes to the general kernels
    (64-bit indexing) instead, which save no chunk weights."""
    d, f = 64, 65536
    limit = ((1 << 31) - 1) // (2 * f) - 64    # longest chunk the 8-wave path takes
    ok = ip.Problem(1, limit, d, f, limit, ip.IPTTT_BF16)
    too_long = ip.Problem(1, limit + 1, d, f, limit + 1, ip.IPTTT_BF16)
    assert ip.ipttt_validate(ok) == 0 and ip.ipttt_validate(too_long) == 0
    assert ip.ipttt_saved_bytes(ok) == d * f * 2 + d * f * 2
    assert ip.ipttt_saved_bytes(too_long) == 0
    # the 4B shapes with the pages' chunk sizes stay on the 8-wave path
    for C in (512, 1024):
        assert ip.ipttt_saved_bytes(ip.Problem(1, 4 * C, 2560, 9728, C, ip.IPTTT_BF16)) > 0


@pytest.mark.skipif(__import__("torch").cuda.is_available(),
                    reason="drives the launch set-up with no device present")
def test_launch_hook_is_called_before_the_first_launch_and_can_be_removed():
    """With no device, each call gets as far as its first launch, which fails
    (IPTTT_ERR_HIP); the hook has seen that launch's name by then."""
    lib = ip.library()
    v = ctypes.c_void_p
    seen = []
    ip.ipttt_set_launch_hook(lambda name, stream: seen.append((name, stream)))
    try:
        p = ip.Problem(1, 64, 64, 128, 16, ip.IPTTT_BF16)
        assert lib.ipttt_z(p.ref, v(256), v(256), v(256), v(256), v(4096)) == 7
        ws = ip.ipttt_workspace_bytes(p)
        assert lib.ipttt_target(p.ref, v(256), v(256), v(256), v(256), v(256), ws, None) == 7
        assert seen == [("gated_z", 4096), ("segments", 0)]
    finally:
        ip.ipttt_set_launch_hook(None)
    assert lib.ipttt_z(p.ref, v(256), v(256), v(256), v(256), None) == 7
    assert len(seen) == 2


def test_prepared_segment_descriptors_go_together_and_are_aligned():
    """seg_table and seg_bytes: both NULL or both set; the table 4-byte aligned.
    Checked before anything is launched (the pointers are never dereferenced here)."""
    p = ip.Problem(2, 64, 16, 32, 16, ip.IPTTT_BF16)
    assert ip.ipttt_validate(p) == 0
    p._c.seg_table, p._c.seg_bytes = 4096, None
    assert ip.ipttt_validate(p) == 1  # IPTTT_ERR_NULL
    p._c.seg_table, p._c.seg_bytes = None, 4096
    assert ip.ipttt_validate(p) == 1
    p._c.seg_table, p._c.seg_bytes = 4098, 4096
    assert ip.ipttt_validate(p) == 4  # IPTTT_ERR_ALIGN
    p._c.seg_table, p._c.seg_bytes = 4096, 8193
    assert ip.ipttt_validate(p) == 0
    with pytest.raises(ValueError):
        p.use_segments(None, torch.empty(1, dtype=torch.uint8))
    # host tensors would hand the kernels host addresses: refused by the binding
    with pytest.raises(ValueError):
        p.use_segments(torch.zeros(2 * 4 * 3, dtype=torch.int32), torch.zeros(128, dtype=torch.uint8))
