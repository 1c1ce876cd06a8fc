"""GPU tests of the degenerate cases of the method, on both kernel families.

The state a chunk applies is W_down plus the clipped deltas of its
document's earlier chunks (lijianxiong.blog "In-Place Test-Time Training",
工程实现: the exclusive prefix sum; iplexlaw.co.kr review, section 6: the
state resets at every document start).  At the edges of that definition:
- a row of one token, or a chunk grid with one chunk per row, applies W_down
  alone;
- one-token chunks update the state after every token;
- a document start at every token, or at every chunk start, leaves no delta
  that any later token of the same document could see.
Where no delta reaches any token, the outputs must equal those of a run with
eta = 0 bit for bit (the same kernels apply the same W_down) and the plain
gated MLP within tolerance; one-token chunks and one-token rows are compared
with the oracle's sequential loop.  Both kernel families run every case: the
general kernels (fp32, widths not multiples of 64) and the 8-wave kernels
(bf16, widths multiples of 64).
"""
import numpy as np
import pytest
import torch

import oracle
import test_weight_mlp_amd as ip
from test_weight_mlp_amd import inputs
from gpu_helpers import np64, rel, run_gpu, run_oracle, tol

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

FAMILIES = {
    "general_f32": inputs.CONFIGS["tiny_f32"].with_(name="degenerate_f32", d_model=72, d_ff=136, eta=5e-2,
                                                    tau=2e-2),
    "fast_bf16": inputs.CONFIGS["4b_32k"].with_(name="degenerate_bf16", d_model=128, d_ff=192, eta=1e-2,
                                                tau=1e-3),
}


def _run(cfg, docs, seed):
    x = inputs.make_inputs(cfg, seed, "cuda", doc_starts=docs)
    _, buf = run_gpu(cfg, x)
    return x, inputs.to_f64(x), buf


def _no_delta_reaches_a_token(cfg, docs, seed):
    x, x64, buf = _run(cfg, docs, seed)
    _, b0 = run_gpu(cfg, dict(x, eta=0.0))
    assert torch.equal(buf.O, b0.O)
    r = rel(np64(buf.O), oracle.plain_mlp(x64["H"], x64["W_gate"], x64["W_up"], x64["W_down"]))
    print(f"  [{cfg.name}] O rel to the plain MLP {r:.2e}", flush=True)
    assert r <= tol(cfg)


@pytest.mark.parametrize("family", list(FAMILIES))
def test_one_token_rows(family):
    cfg = FAMILIES[family].with_(rows=3, seq_len=1, chunk=4)
    _no_delta_reaches_a_token(cfg, None, 41)


@pytest.mark.parametrize("family", list(FAMILIES))
def test_one_chunk_longer_than_the_row(family):
    cfg = FAMILIES[family].with_(rows=2, seq_len=300, chunk=4096)
    _no_delta_reaches_a_token(cfg, [120, 300 + 7], 42)


@pytest.mark.parametrize("family", list(FAMILIES))
def test_a_document_at_every_token(family):
    """Every token but the row starts begins a document: 2 x 199 listed
    starts, more than one kernel-argument batch of the descriptor builder."""
    cfg = FAMILIES[family].with_(rows=2, seq_len=200, chunk=16)
    T = cfg.seq_len
    docs = [t for t in range(1, 2 * T) if t != T]
    _no_delta_reaches_a_token(cfg, docs, 43)


@pytest.mark.parametrize("family", list(FAMILIES))
def test_a_document_at_every_chunk_start(family):
    cfg = FAMILIES[family].with_(rows=2, seq_len=250, chunk=32)
    T, C = cfg.seq_len, cfg.chunk
    docs = [b * T + c for b in range(2) for c in range(C, T, C)]
    _no_delta_reaches_a_token(cfg, docs, 44)


@pytest.mark.parametrize("family", list(FAMILIES))
def test_one_token_chunks(family):
    """C = 1: the state is updated after every token (clipped), and every
    token applies the deltas of all earlier tokens of its document."""
    cfg = FAMILIES[family].with_(rows=2, seq_len=70, chunk=1)
    docs = [20, 70 + 35]
    x, x64, buf = _run(cfg, docs, 45)
    ref = run_oracle(cfg, x64)
    ra = rel(np64(buf.alpha).reshape(ref["alpha"].shape), ref["alpha"])
    ro = rel(np64(buf.O), ref["O"])
    # the fast-weight term alone: W_down = 0
    Wz = torch.zeros_like(x["W_down"])
    _, bz = run_gpu(cfg, x, W_down=Wz)
    refz = run_oracle(cfg, x64, W_down=np.zeros_like(x64["W_down"]))
    rz = rel(np64(bz.O), refz["O"])
    print(f"  [{cfg.name}] alpha rel {ra:.2e}, O rel {ro:.2e}, fast-weight term rel {rz:.2e}", flush=True)
    assert np.any(ref["alpha"] < 1.0)
    assert ra <= tol(cfg) and ro <= tol(cfg) and rz <= tol(cfg)


BACKWARD_CASES = {
    "one_token_rows": (dict(rows=3, seq_len=1, chunk=4), None),
    "one_token_chunks": (dict(rows=2, seq_len=70, chunk=1), [20, 70 + 35]),
    "a_document_at_every_token": (dict(rows=2, seq_len=120, chunk=16), [t for t in range(1, 240) if t != 120]),
}


@pytest.mark.parametrize("path", ["recomputing", "saved"])
@pytest.mark.parametrize("case", list(BACKWARD_CASES))
@pytest.mark.parametrize("family", list(FAMILIES))
def test_backward(family, case, path):
    """forward -> backward against oracle.backward, all seven input
    gradients, both the backward that recomputes the forward's state and the
    one that reads it back.  Where no delta reaches any token, nothing flows
    back into the target's inputs: dX0, the conv weights' and W_target's
    gradients are exactly zero."""
    shape, docs = BACKWARD_CASES[case]
    cfg = FAMILIES[family].with_(**shape)
    x = inputs.make_inputs(cfg, 46, "cuda", doc_starts=docs)
    c = inputs.make_cotangents(cfg, 46, "cuda")
    dt = ip.IPTTT_F32 if cfg.dtype == "f32" else ip.IPTTT_BF16
    p = ip.Problem(cfg.rows, cfg.seq_len, cfg.d_model, cfg.d_ff, cfg.chunk, dt, docs)
    w = [x[k] for k in ("H", "X0", "W_gate", "W_up", "W_down", "conv_w", "W_target")]
    if path == "recomputing":
        buf = ip.allocate(p, "cuda")
        ip.forward(p, *w, x["eta"], x["tau"], buf)
        g = ip.backward(p, buf, *w, x["eta"], x["tau"], c["dO"])
    else:
        buf = ip.allocate(p, "cuda", save=True)
        ip.forward(p, *w, x["eta"], x["tau"], buf)
        g = ip.Grads(p, "cuda")
        ip.ipttt_scan_apply_backward_saved(p, buf.Z, buf.V, x["W_down"], x["eta"], x["tau"], buf.alpha, buf.saved,
                                           c["dO"], g.dZ, g.dV, g.dW_down, g.ws)
        ip.ipttt_target_backward(p, x["X0"], x["conv_w"], x["W_target"], g.dV, g.dX0, g.dconv_w, g.dW_target, g.ws)
        ip.ipttt_z_backward_saved(p, x["H"], x["W_gate"], x["W_up"], buf.GU, g.dZ, g.dH, g.dW_gate, g.dW_up, g.ws)
    torch.cuda.synchronize()
    x64 = inputs.to_f64(x)
    ref = oracle.backward(x64["H"], x64["X0"], x64["W_gate"], x64["W_up"], x64["W_down"], x64["conv_w"],
                          x64["W_target"], np64(c["dO"]), rows=cfg.rows, T=cfg.seq_len, C=cfg.chunk,
                          eta=x["eta"], tau=x["tau"], doc_starts=docs)
    for k in ("dH", "dX0", "dW_gate", "dW_up", "dW_down", "dconv_w", "dW_target"):
        r = rel(np64(getattr(g, k)), ref[k])
        print(f"  [{cfg.name} {case} {path}] {k} rel {r:.2e}", flush=True)
        assert r <= tol(cfg), k
    if case != "one_token_chunks":
        for k in ("dX0", "dconv_w", "dW_target"):
            assert not np.any(ref[k]) and not torch.any(getattr(g, k)), k


@pytest.mark.parametrize("shape", ["65535_rows", "65535_chunks"])
@pytest.mark.parametrize("family", list(FAMILIES))
def test_largest_launch_grids(family, shape):
    """Rows, and (row, chunk) pairs, ride in the y dimension of launch grids,
    which the library takes up to 65535 (the problem check rejects more):
    65535 one-token rows (every kernel's grid at that many rows or chunks),
    and one row of 65535 one-token chunks.  Forward and backward against the
    oracle at widths of 64."""
    rows, T = (65535, 1) if shape == "65535_rows" else (1, 65535)
    cfg = FAMILIES[family].with_(d_model=64 if family == "fast_bf16" else 72, d_ff=64 if family == "fast_bf16" else 136,
                                 rows=rows, seq_len=T, chunk=1)
    x = inputs.make_inputs(cfg, 47, "cuda")
    c = inputs.make_cotangents(cfg, 47, "cuda")
    dt = ip.IPTTT_F32 if cfg.dtype == "f32" else ip.IPTTT_BF16
    p = ip.Problem(cfg.rows, cfg.seq_len, cfg.d_model, cfg.d_ff, cfg.chunk, dt, None)
    w = [x[k] for k in ("H", "X0", "W_gate", "W_up", "W_down", "conv_w", "W_target")]
    buf = ip.allocate(p, "cuda")
    ip.forward(p, *w, x["eta"], x["tau"], buf)
    g = ip.backward(p, buf, *w, x["eta"], x["tau"], c["dO"])
    torch.cuda.synchronize()
    x64 = inputs.to_f64(x)
    ref = run_oracle(cfg, x64)
    r = rel(np64(buf.O), ref["O"])
    print(f"  [{cfg.name} {shape}] O rel {r:.2e}", flush=True)
    assert r <= tol(cfg)
    refb = oracle.backward(x64["H"], x64["X0"], x64["W_gate"], x64["W_up"], x64["W_down"], x64["conv_w"],
                           x64["W_target"], np64(c["dO"]), rows=cfg.rows, T=cfg.seq_len, C=cfg.chunk,
                           eta=x["eta"], tau=x["tau"])
    for k in ("dH", "dX0", "dW_gate", "dW_up", "dW_down", "dconv_w", "dW_target"):
        r = rel(np64(getattr(g, k)), refb[k])
        print(f"  [{cfg.name} {shape}] {k} rel {r:.2e}", flush=True)
        assert r <= tol(cfg), k
