"""In-Place TTT layer forward on AMD MI355X: Python binding of libipttt.so.

The functions below carry the names of the C ABI in ``include/ipttt.h`` and
only marshal arguments: torch tensors become device pointers, the current
torch stream becomes the HIP stream, and status codes become exceptions.
Every step of the layer runs in the library's HIP kernels; there is no other
code path.  The library is built in-tree by ``python -m test_weight_mlp_amd.build``
(or ``__graft_entry__.build()``); importing this module does not load it,
the first call does, and raises if it is missing.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import numpy as np
import torch

__all__ = [
    "IPTTT_F32", "IPTTT_BF16", "IPTTT_TARGET_LM", "IPTTT_TARGET_NO_CONV", "IPTTT_TARGET_NO_PROJ",
    "IptttError", "Problem", "library", "library_path",
    "ipttt_abi_version", "ipttt_validate", "ipttt_workspace_bytes", "ipttt_segment_table",
    "ipttt_segments_device", "ipttt_z", "ipttt_target", "ipttt_chunk_delta", "ipttt_scan_apply",
    "ipttt_scan_apply_carry", "Buffers", "allocate", "forward",
    "ipttt_backward_workspace_bytes", "ipttt_scan_apply_backward", "ipttt_target_backward",
    "ipttt_z_backward", "Grads", "backward", "ipttt_saved_bytes", "ipttt_scan_apply_save",
    "ipttt_scan_apply_backward_saved", "ipttt_z_save", "ipttt_z_backward_saved", "ipttt_chunk_delta_noalloc",
    "IPTTT_NOALLOC_SCRATCH_BYTES", "ipttt_set_launch_hook",
]

IPTTT_F32 = 0
IPTTT_BF16 = 1
IPTTT_TARGET_LM = 0       # V_hat = Conv1D(X0) W_target
IPTTT_TARGET_NO_CONV = 1  # V_hat = X0 W_target
IPTTT_TARGET_NO_PROJ = 2  # V_hat = Conv1D(X0)
IPTTT_NOALLOC_SCRATCH_BYTES = 8 << 20  # static scratch of ipttt_chunk_delta_noalloc, per GPU

# IPTTT_LIBRARY selects another build of the same library (the host-sanitized
# copy that the CPU sanitizer test loads); the default is the in-tree build.
library_path = os.environ.get("IPTTT_LIBRARY") or os.path.join(os.path.dirname(os.path.abspath(__file__)),
                                                                "libipttt.so")
_lib = None


# void (*)(const char* kernel, void* stream, void* user)
LAUNCH_HOOK = ctypes.CFUNCTYPE(None, ctypes.c_char_p, ctypes.c_void_p, ctypes.c_void_p)
_hook_ref = None


def ipttt_set_launch_hook(fn) -> None:
    """Measurement aid: fn(kernel_name: str, stream: int) runs right before the
    library enqueues each kernel (None turns it off).  A profiler records a
    stream event there and times every kernel on its own stream."""
    global _hook_ref
    if fn is None:
        library().ipttt_set_launch_hook(LAUNCH_HOOK(), None)
        _hook_ref = None
        return
    cb = LAUNCH_HOOK(lambda name, stream, user: fn(name.decode(), stream or 0))
    library().ipttt_set_launch_hook(cb, None)
    _hook_ref = cb  # keep the trampoline alive while the library holds it


class IptttError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = library().ipttt_status_string(status).decode()
        super().__init__(f"{where}: status {status} ({msg})")


class _CProblem(ctypes.Structure):
    _fields_ = [
        ("rows", ctypes.c_int64), ("seq_len", ctypes.c_int64), ("d_model", ctypes.c_int64),
        ("d_ff", ctypes.c_int64), ("chunk", ctypes.c_int64), ("dtype", ctypes.c_int32),
        ("target", ctypes.c_int32), ("doc_starts", ctypes.POINTER(ctypes.c_int64)),
        ("n_doc_starts", ctypes.c_int64), ("continues", ctypes.POINTER(ctypes.c_uint8)),
        ("seg_table", ctypes.c_void_p), ("seg_bytes", ctypes.c_void_p),
    ]


def library() -> ctypes.CDLL:
    """Loads libipttt.so once; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(library_path):
            raise RuntimeError(f"{library_path} is missing: build it with "
                               "`python -m test_weight_mlp_amd.build`")
        lib = ctypes.CDLL(library_path)
        P = ctypes.POINTER(_CProblem)
        vp, f32, i32, sz = ctypes.c_void_p, ctypes.c_float, ctypes.c_int, ctypes.c_size_t
        sigs = {
            "ipttt_abi_version": (i32, []),
            "ipttt_status_string": (ctypes.c_char_p, [i32]),
            "ipttt_validate": (i32, [P]),
            "ipttt_workspace_bytes": (sz, [P]),
            "ipttt_segment_table": (i32, [P, vp]),
            "ipttt_segments_device": (i32, [P, vp, vp, vp]),
            "ipttt_z": (i32, [P, vp, vp, vp, vp, vp]),
            "ipttt_target": (i32, [P, vp, vp, vp, vp, vp, sz, vp]),
            "ipttt_chunk_delta": (i32, [P, vp, vp, f32, f32, vp, vp, vp, sz, vp]),
            "ipttt_chunk_delta_noalloc": (i32, [P, vp, vp, f32, f32, vp, vp]),
            "ipttt_set_launch_hook": (None, [LAUNCH_HOOK, vp]),
            "ipttt_scan_apply": (i32, [P, vp, vp, vp, vp, f32, vp, vp, sz, vp]),
            "ipttt_scan_apply_carry": (i32, [P, vp, vp, vp, vp, f32, vp, vp, vp, vp, sz, vp]),
            "ipttt_backward_workspace_bytes": (sz, [P]),
            "ipttt_scan_apply_backward": (i32, [P, vp, vp, vp, f32, f32, vp, vp, vp, vp, vp, sz, vp]),
            "ipttt_target_backward": (i32, [P, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]),
            "ipttt_z_backward": (i32, [P, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]),
            "ipttt_saved_bytes": (sz, [P]),
            "ipttt_z_save": (i32, [P, vp, vp, vp, vp, vp, vp]),
            "ipttt_z_backward_saved": (i32, [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]),
            "ipttt_scan_apply_save": (i32, [P, vp, vp, vp, vp, f32, vp, vp, sz, vp, sz, vp]),
            "ipttt_scan_apply_backward_saved": (i32, [P, vp, vp, vp, f32, f32, vp, vp, sz, vp, vp, vp, vp, vp,
                                                      sz, vp]),
        }
        for name, (res, args) in sigs.items():
            fn = getattr(lib, name)
            fn.restype, fn.argtypes = res, args
        _lib = lib
    return _lib


class Problem:
    """Sizes, dtype, document starts and continuing rows of one layer call
    (ipttt_problem)."""

    def __init__(self, rows: int, seq_len: int, d_model: int, d_ff: int, chunk: int,
                 dtype: int = IPTTT_BF16, doc_starts: Optional[Sequence[int]] = None,
                 target: int = IPTTT_TARGET_LM, continues: Optional[Sequence[int]] = None):
        self.rows, self.seq_len, self.d_model, self.d_ff = rows, seq_len, d_model, d_ff
        self.chunk, self.dtype, self.target = chunk, dtype, target
        self.doc_starts = np.ascontiguousarray(
            np.asarray([] if doc_starts is None else doc_starts, dtype=np.int64))
        ptr = (self.doc_starts.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))
               if self.doc_starts.size else None)
        self.continues = None
        cptr = None
        if continues is not None:
            self.continues = np.ascontiguousarray(np.asarray(continues, dtype=np.uint8))
            if self.continues.shape != (rows,):
                raise ValueError("continues needs one flag per row")
            cptr = self.continues.ctypes.data_as(ctypes.POINTER(ctypes.c_uint8))
        self._c = _CProblem(rows, seq_len, d_model, d_ff, chunk, dtype, target, ptr,
                            int(self.doc_starts.size), cptr, None, None)
        self._segments = None

    def use_segments(self, table: Optional[torch.Tensor], segs: Optional[torch.Tensor]) -> "Problem":
        """Has every call read these device descriptors (ipttt_problem.seg_table
        and seg_bytes, as ipttt_segments_device fills them for this problem)
        instead of building its own; None, None goes back to building them."""
        if (table is None) != (segs is None):
            raise ValueError("seg_table and seg_bytes go together")
        if table is not None:
            n_table, n_segs = self.rows * self.n_chunks * 3, self.tokens
            for t, dt, n, what in ((table, torch.int32, n_table, "seg_table"), (segs, torch.uint8, n_segs, "seg_bytes")):
                if t.device.type != "cuda" or t.dtype != dt or not t.is_contiguous() or t.numel() < n:
                    raise ValueError(f"{what} must be a contiguous {dt} device tensor of at least {n} elements")
        self._segments = None if table is None else (table, segs)
        self._c.seg_table = None if table is None else table.data_ptr()
        self._c.seg_bytes = None if segs is None else segs.data_ptr()
        return self

    def prepare_segments(self, device="cuda", stream=None) -> "Problem":
        """Builds the segment descriptors on the device once, for all later calls."""
        self.use_segments(None, None)
        table = torch.empty(self.rows * self.n_chunks * 3, dtype=torch.int32, device=device)
        segs = torch.empty(self.tokens, dtype=torch.uint8, device=device)
        ipttt_segments_device(self, table, segs, stream)
        return self.use_segments(table, segs)

    @property
    def ref(self):
        return ctypes.byref(self._c)

    @property
    def chunk_eff(self) -> int:
        return min(self.chunk, self.seq_len)

    @property
    def n_chunks(self) -> int:
        return -(-self.seq_len // self.chunk_eff)

    @property
    def tokens(self) -> int:
        return self.rows * self.seq_len

    @property
    def torch_dtype(self) -> torch.dtype:
        return torch.float32 if self.dtype == IPTTT_F32 else torch.bfloat16



def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors passed to the library must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _check(status: int, where: str):
    if status != 0:
        raise IptttError(status, where)


def ipttt_abi_version() -> int:
    return library().ipttt_abi_version()


def ipttt_validate(p: Problem) -> int:
    """Returns the status code (0 = valid) without raising."""
    return library().ipttt_validate(p.ref)


def ipttt_workspace_bytes(p: Problem) -> int:
    return int(library().ipttt_workspace_bytes(p.ref))


def ipttt_segment_table(p: Problem) -> np.ndarray:
    """Host segment table [rows, N, 3] (r0, l0, carry) as int32."""
    out = np.zeros((p.rows, p.n_chunks, 3), dtype=np.int32)
    _check(library().ipttt_segment_table(p.ref, out.ctypes.data_as(ctypes.c_void_p)),
           "ipttt_segment_table")
    return out


def ipttt_segments_device(p: Problem, table: Optional[torch.Tensor], segs: torch.Tensor,
                          stream=None):
    _check(library().ipttt_segments_device(p.ref, _ptr(table), _ptr(segs), _stream(stream)),
           "ipttt_segments_device")


def ipttt_z(p: Problem, H, W_gate, W_up, Z, stream=None):
    _check(library().ipttt_z(p.ref, _ptr(H), _ptr(W_gate), _ptr(W_up), _ptr(Z), _stream(stream)),
           "ipttt_z")


def ipttt_z_save(p: Problem, H, W_gate, W_up, Z, GU, stream=None):
    _check(library().ipttt_z_save(p.ref, _ptr(H), _ptr(W_gate), _ptr(W_up), _ptr(Z), _ptr(GU), _stream(stream)),
           "ipttt_z_save")


def ipttt_target(p: Problem, X0, conv_w, W_target, V, ws, stream=None):
    _check(library().ipttt_target(p.ref, _ptr(X0), _ptr(conv_w), _ptr(W_target), _ptr(V),
                                  _ptr(ws), ws.numel(), _stream(stream)), "ipttt_target")


def ipttt_chunk_delta(p: Problem, V, Z, eta: float, tau: float, alpha, dW, ws, stream=None):
    _check(library().ipttt_chunk_delta(p.ref, _ptr(V), _ptr(Z), eta, tau, _ptr(alpha), _ptr(dW),
                                       _ptr(ws), ws.numel(), _stream(stream)), "ipttt_chunk_delta")


def ipttt_chunk_delta_noalloc(p: Problem, V, Z, eta: float, tau: float, alpha, stream=None):
    _check(library().ipttt_chunk_delta_noalloc(p.ref, _ptr(V), _ptr(Z), eta, tau, _ptr(alpha), _stream(stream)),
           "ipttt_chunk_delta_noalloc")


def ipttt_scan_apply(p: Problem, Z, V, W_down, alpha, eta: float, O, ws, stream=None):
    _check(library().ipttt_scan_apply(p.ref, _ptr(Z), _ptr(V), _ptr(W_down), _ptr(alpha), eta,
                                      _ptr(O), _ptr(ws), ws.numel(), _stream(stream)),
           "ipttt_scan_apply")


def ipttt_scan_apply_carry(p: Problem, Z, V, W_down, alpha, eta: float, S_in, S_out, O, ws,
                           stream=None):
    _check(library().ipttt_scan_apply_carry(p.ref, _ptr(Z), _ptr(V), _ptr(W_down), _ptr(alpha), eta,
                                            _ptr(S_in), _ptr(S_out), _ptr(O), _ptr(ws), ws.numel(),
                                            _stream(stream)), "ipttt_scan_apply_carry")


def ipttt_saved_bytes(p: Problem) -> int:
    return int(library().ipttt_saved_bytes(p.ref))


def ipttt_scan_apply_save(p: Problem, Z, V, W_down, alpha, eta: float, O, saved, ws, stream=None):
    _check(library().ipttt_scan_apply_save(p.ref, _ptr(Z), _ptr(V), _ptr(W_down), _ptr(alpha), eta, _ptr(O),
                                           _ptr(saved), 0 if saved is None else saved.numel(), _ptr(ws),
                                           ws.numel(), _stream(stream)), "ipttt_scan_apply_save")


class Buffers:
    """Device buffers of one forward: outputs, intermediates and workspace;
    with ``save``, also what the backward can reuse: ``GU`` (the products
    before the gate) and ``saved`` (the chunk weights; None where the shape
    keeps none)."""

    def __init__(self, p: Problem, device="cuda", want_dW: bool = False, save: bool = False):
        dt = p.torch_dtype
        n, d, f = p.tokens, p.d_model, p.d_ff
        self.Z = torch.empty((n, f), dtype=dt, device=device)
        self.V = torch.empty((n, d), dtype=dt, device=device)
        self.alpha = torch.empty((p.rows, p.n_chunks), dtype=torch.float32, device=device)
        self.dW = (torch.empty((p.rows * p.n_chunks, d, f), dtype=torch.float32, device=device)
                   if want_dW else None)
        self.O = torch.empty((n, d), dtype=dt, device=device)
        self.ws = torch.empty(ipttt_workspace_bytes(p), dtype=torch.uint8, device=device)
        nsave = ipttt_saved_bytes(p) if save else 0
        self.saved = torch.empty(nsave, dtype=torch.uint8, device=device) if nsave > 0 else None
        self.GU = torch.empty((2, n, f), dtype=dt, device=device) if save else None


def allocate(p: Problem, device="cuda", want_dW: bool = False, save: bool = False) -> Buffers:
    return Buffers(p, device, want_dW, save)


def forward(p: Problem, H, X0, W_gate, W_up, W_down, conv_w, W_target, eta: float, tau: float,
            buf: Optional[Buffers] = None, stream=None, carry: bool = False, S_in=None,
            S_out=None) -> Buffers:
    """The whole layer: ipttt_z -> ipttt_target -> ipttt_chunk_delta -> ipttt_scan_apply,
    enqueued on one stream.  Returns the buffers (O, Z, V, alpha, ...).

    With ``carry`` (implied by S_in or S_out) the last step is
    ipttt_scan_apply_carry: S_in [rows, d, f] float32 (or None) is the state
    the rows flagged in ``p.continues`` start from, S_out receives the state of
    each row's open document at its end; S_out may be S_in.  Otherwise, when
    ``buf.saved`` is set (``allocate(..., save=True)``), the last step is
    ipttt_scan_apply_save, which leaves the state ``backward`` reuses there;
    with ``buf.GU`` set, the first step is ipttt_z_save."""
    if buf is None:
        buf = Buffers(p, H.device)
    if buf.GU is not None:
        ipttt_z_save(p, H, W_gate, W_up, buf.Z, buf.GU, stream)
    else:
        ipttt_z(p, H, W_gate, W_up, buf.Z, stream)
    ipttt_target(p, X0, conv_w, W_target, buf.V, buf.ws, stream)
    ipttt_chunk_delta(p, buf.V, buf.Z, eta, tau, buf.alpha, buf.dW, buf.ws, stream)
    if carry or S_in is not None or S_out is not None:
        ipttt_scan_apply_carry(p, buf.Z, buf.V, W_down, buf.alpha, eta, S_in, S_out, buf.O, buf.ws,
                               stream)
    elif buf.saved is not None:
        ipttt_scan_apply_save(p, buf.Z, buf.V, W_down, buf.alpha, eta, buf.O, buf.saved, buf.ws, stream)
    else:
        ipttt_scan_apply(p, buf.Z, buf.V, W_down, buf.alpha, eta, buf.O, buf.ws, stream)
    return buf


def ipttt_backward_workspace_bytes(p: Problem) -> int:
    return int(library().ipttt_backward_workspace_bytes(p.ref))


def ipttt_scan_apply_backward(p: Problem, Z, V, W_down, eta: float, tau: float, dO, dZ, dV, dW_down, ws,
                              stream=None):
    _check(library().ipttt_scan_apply_backward(p.ref, _ptr(Z), _ptr(V), _ptr(W_down), eta, tau, _ptr(dO),
                                               _ptr(dZ), _ptr(dV), _ptr(dW_down), _ptr(ws), ws.numel(),
                                               _stream(stream)), "ipttt_scan_apply_backward")


def ipttt_scan_apply_backward_saved(p: Problem, Z, V, W_down, eta: float, tau: float, alpha, saved, dO, dZ, dV,
                                    dW_down, ws, stream=None):
    _check(library().ipttt_scan_apply_backward_saved(
        p.ref, _ptr(Z), _ptr(V), _ptr(W_down), eta, tau, _ptr(alpha), _ptr(saved),
        0 if saved is None else saved.numel(), _ptr(dO), _ptr(dZ), _ptr(dV), _ptr(dW_down), _ptr(ws), ws.numel(),
        _stream(stream)), "ipttt_scan_apply_backward_saved")


def ipttt_target_backward(p: Problem, X0, conv_w, W_target, dV, dX0, dconv_w, dW_target, ws, stream=None):
    _check(library().ipttt_target_backward(p.ref, _ptr(X0), _ptr(conv_w), _ptr(W_target), _ptr(dV), _ptr(dX0),
                                           _ptr(dconv_w), _ptr(dW_target), _ptr(ws), ws.numel(),
                                           _stream(stream)), "ipttt_target_backward")


def ipttt_z_backward(p: Problem, H, W_gate, W_up, dZ, dH, dW_gate, dW_up, ws, stream=None):
    _check(library().ipttt_z_backward(p.ref, _ptr(H), _ptr(W_gate), _ptr(W_up), _ptr(dZ), _ptr(dH),
                                      _ptr(dW_gate), _ptr(dW_up), _ptr(ws), ws.numel(), _stream(stream)),
           "ipttt_z_backward")


def ipttt_z_backward_saved(p: Problem, H, W_gate, W_up, GU, dZ, dH, dW_gate, dW_up, ws, stream=None):
    _check(library().ipttt_z_backward_saved(p.ref, _ptr(H), _ptr(W_gate), _ptr(W_up), _ptr(GU), _ptr(dZ),
                                            _ptr(dH), _ptr(dW_gate), _ptr(dW_up), _ptr(ws), ws.numel(),
                                            _stream(stream)), "ipttt_z_backward_saved")


class Grads:
    """Device buffers of one backward: the input gradients, dZ, dV and the
    backward workspace."""

    def __init__(self, p: Problem, device="cuda"):
        dt = p.torch_dtype
        n, d, f = p.tokens, p.d_model, p.d_ff
        f32 = torch.float32
        self.dZ = torch.empty((n, f), dtype=dt, device=device)
        self.dV = torch.empty((n, d), dtype=dt, device=device)
        self.dH = torch.empty((n, d), dtype=dt, device=device)
        self.dX0 = torch.empty((n, d), dtype=dt, device=device)
        self.dW_gate = torch.empty((f, d), dtype=f32, device=device)
        self.dW_up = torch.empty((f, d), dtype=f32, device=device)
        self.dW_down = torch.empty((d, f), dtype=f32, device=device)
        self.dconv_w = (torch.empty((d, 5), dtype=f32, device=device)
                        if p.target != IPTTT_TARGET_NO_CONV else None)
        self.dW_target = (torch.empty((d, d), dtype=f32, device=device)
                          if p.target != IPTTT_TARGET_NO_PROJ else None)
        self.ws = torch.empty(ipttt_backward_workspace_bytes(p), dtype=torch.uint8, device=device)


def backward(p: Problem, buf: Buffers, H, X0, W_gate, W_up, W_down, conv_w, W_target, eta: float,
             tau: float, dO, grads: Optional[Grads] = None, stream=None) -> Grads:
    """The layer's backward after ``forward(p, ..., buf)``: ipttt_scan_apply_backward ->
    ipttt_target_backward -> ipttt_z_backward on one stream, from the forward's Z and V
    (and, when the forward saved them, its clip scales and chunk weights:
    ipttt_scan_apply_backward_saved; its G and U: ipttt_z_backward_saved)."""
    if grads is None:
        grads = Grads(p, H.device)
    g = grads
    if buf.saved is not None:
        ipttt_scan_apply_backward_saved(p, buf.Z, buf.V, W_down, eta, tau, buf.alpha, buf.saved, dO, g.dZ, g.dV,
                                        g.dW_down, g.ws, stream)
    else:
        ipttt_scan_apply_backward(p, buf.Z, buf.V, W_down, eta, tau, dO, g.dZ, g.dV, g.dW_down, g.ws, stream)
    ipttt_target_backward(p, X0, conv_w, W_target, g.dV, g.dX0, g.dconv_w, g.dW_target, g.ws, stream)
    if buf.GU is not None:
        ipttt_z_backward_saved(p, H, W_gate, W_up, buf.GU, g.dZ, g.dH, g.dW_gate, g.dW_up, g.ws, stream)
    else:
        ipttt_z_backward(p, H, W_gate, W_up, g.dZ, g.dH, g.dW_gate, g.dW_up, g.ws, stream)
    return g
