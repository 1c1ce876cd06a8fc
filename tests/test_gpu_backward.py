"""GPU parity of the backward pass against the fp64 oracle's gradients.

Each backward call is checked on its own, from seeded inputs shared with the
oracle (Z, V, dO for the scan/apply backward; X0, the target weights and dV
for the target backward; H, W_gate, W_up and dZ for the gated MLP), and the
whole chain forward -> backward is checked end to end against
oracle.backward, which computes every gradient from H and X0.  Tolerances
are those of the forward: Frobenius-relative 1e-2 for bf16 data, 1e-4 for
fp32.  The clip is exercised both off (tau = 0) and on (tau = 1e-3, orders
of magnitude below every segment's delta norm with these inputs, so its
derivative acts on every carried delta).
"""
import numpy as np
import pytest
import torch

import oracle
import test_weight_mlp_amd as ip
from test_weight_mlp_amd import inputs
from gpu_helpers import np64, rel, tol

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

C = inputs.CONFIGS
CASES = {
    "bf16_wide": (C["4b_32k"].with_(name="bf16_wide", d_model=256, d_ff=384, rows=2, seq_len=1300, chunk=256,
                                    eta=1e-2), [700, 1300 + 100]),
    "bf16_narrow": (C["4b_32k"].with_(name="bf16_narrow", d_model=136, d_ff=200, rows=1, seq_len=600,
                                      chunk=128, eta=1e-2), [333]),
    "f32": (C["tiny_f32"].with_(name="f32", d_model=72, d_ff=136, rows=2, seq_len=300, chunk=48, eta=5e-2),
            [77, 300 + 5]),
    # a chunk that is not a whole number of 64-token stages on the 8-wave
    # path: the clip's products over a chunk's tokens run their last stage
    # on the zero padding of the chunk Grams
    "bf16_odd_chunk": (C["4b_32k"].with_(name="bf16_odd_chunk", d_model=128, d_ff=192, rows=2, seq_len=450,
                                         chunk=100, eta=1e-2), [130, 450 + 260]),
    # the 8-wave products at their shortest K loops: one 64-deep stage
    # (K = d_model and K = chunk) and an odd count of three (K = d_ff)
    "bf16_short_k": (C["4b_32k"].with_(name="bf16_short_k", d_model=64, d_ff=192, rows=2, seq_len=700, chunk=64,
                                       eta=1e-2), [250, 700 + 333]),
}
TAUS = {"noclip": 0.0, "clip": 1e-3}


def _problem(cfg, docs, target=ip.IPTTT_TARGET_LM):
    dt = ip.IPTTT_F32 if cfg.dtype == "f32" else ip.IPTTT_BF16
    return ip.Problem(cfg.rows, cfg.seq_len, cfg.d_model, cfg.d_ff, cfg.chunk, dt, docs, target=target)


def _check(got, ref, cfg, what):
    r = rel(got if isinstance(got, np.ndarray) else np64(got), ref)
    print(f"    {what}: rel {r:.2e}", flush=True)
    assert r <= tol(cfg), what


@pytest.mark.parametrize("clip", list(TAUS))
@pytest.mark.parametrize("name", list(CASES))
def test_scan_apply_backward(name, clip):
    cfg, docs = CASES[name]
    tau = TAUS[clip]
    x = inputs.make_inputs(cfg, 21, "cuda", doc_starts=docs)
    c = inputs.make_cotangents(cfg, 21, "cuda")
    print(f"[{name}] scan/apply backward, tau {tau}", flush=True)
    p = _problem(cfg, docs)
    g = ip.Grads(p, "cuda")
    ip.ipttt_scan_apply_backward(p, c["Z"], c["V"], x["W_down"], x["eta"], tau, c["dO"], g.dZ, g.dV, g.dW_down,
                                 g.ws)
    torch.cuda.synchronize()
    ref = oracle.backward_scan_apply(np64(c["Z"]), np64(c["V"]), np64(x["W_down"]), np64(c["dO"]),
                                     rows=cfg.rows, T=cfg.seq_len, C=cfg.chunk, eta=x["eta"], tau=tau,
                                     doc_starts=docs)
    _check(g.dZ, ref["dZ"], cfg, "dZ")
    _check(g.dV, ref["dV"], cfg, "dV")
    _check(g.dW_down, ref["dW_down"], cfg, "dW_down")


@pytest.mark.parametrize("target", ["lm", "no_conv", "no_proj"])
@pytest.mark.parametrize("name", list(CASES))
def test_target_backward(name, target):
    cfg, docs = CASES[name]
    kind = {"lm": ip.IPTTT_TARGET_LM, "no_conv": ip.IPTTT_TARGET_NO_CONV, "no_proj": ip.IPTTT_TARGET_NO_PROJ}
    x = inputs.make_inputs(cfg, 22, "cuda", doc_starts=docs)
    c = inputs.make_cotangents(cfg, 22, "cuda")
    print(f"[{name}] target backward, {target}", flush=True)
    p = _problem(cfg, docs, kind[target])
    g = ip.Grads(p, "cuda")
    conv = None if target == "no_conv" else x["conv_w"]
    wt = None if target == "no_proj" else x["W_target"]
    ip.ipttt_target_backward(p, x["X0"], conv, wt, c["dV"], g.dX0, g.dconv_w, g.dW_target, g.ws)
    torch.cuda.synchronize()
    ref = oracle.backward_target(np64(x["X0"]), np64(x["conv_w"]), np64(x["W_target"]), np64(c["dV"]),
                                 rows=cfg.rows, T=cfg.seq_len, C=cfg.chunk, doc_starts=docs, target=target)
    _check(g.dX0, ref["dX0"], cfg, "dX0")
    if target != "no_conv":
        _check(g.dconv_w, ref["dconv_w"], cfg, "dconv_w")
    if target != "no_proj":
        _check(g.dW_target, ref["dW_target"], cfg, "dW_target")


@pytest.mark.parametrize("name", list(CASES))
def test_z_backward(name):
    cfg, docs = CASES[name]
    x = inputs.make_inputs(cfg, 23, "cuda", doc_starts=docs)
    c = inputs.make_cotangents(cfg, 23, "cuda")
    print(f"[{name}] gated MLP backward", flush=True)
    p = _problem(cfg, docs)
    g = ip.Grads(p, "cuda")
    ip.ipttt_z_backward(p, x["H"], x["W_gate"], x["W_up"], c["dZ"], g.dH, g.dW_gate, g.dW_up, g.ws)
    torch.cuda.synchronize()
    ref = oracle.backward_z(np64(x["H"]), np64(x["W_gate"]), np64(x["W_up"]), np64(c["dZ"]))
    _check(g.dH, ref["dH"], cfg, "dH")
    _check(g.dW_gate, ref["dW_gate"], cfg, "dW_gate")
    _check(g.dW_up, ref["dW_up"], cfg, "dW_up")


@pytest.mark.parametrize("name", list(CASES))
def test_z_save_and_backward_from_saved_products(name):
    """ipttt_z_save writes the same Z as ipttt_z (bit for bit) and G = H
    W_gate^T, U = H W_up^T; ipttt_z_backward_saved from them gives the
    oracle's gradients."""
    cfg, docs = CASES[name]
    x = inputs.make_inputs(cfg, 29, "cuda", doc_starts=docs)
    c = inputs.make_cotangents(cfg, 29, "cuda")
    print(f"[{name}] gated MLP forward (saved G, U) and backward from them", flush=True)
    p = _problem(cfg, docs)
    n, f = cfg.rows * cfg.seq_len, cfg.d_ff
    Z0 = torch.empty((n, f), dtype=x["H"].dtype, device="cuda")
    Z1 = torch.empty_like(Z0)
    GU = torch.empty((2, n, f), dtype=x["H"].dtype, device="cuda")
    ip.ipttt_z(p, x["H"], x["W_gate"], x["W_up"], Z0)
    ip.ipttt_z_save(p, x["H"], x["W_gate"], x["W_up"], Z1, GU)
    g = ip.Grads(p, "cuda")
    ip.ipttt_z_backward_saved(p, x["H"], x["W_gate"], x["W_up"], GU, c["dZ"], g.dH, g.dW_gate, g.dW_up, g.ws)
    torch.cuda.synchronize()
    assert torch.equal(Z0, Z1)
    H, Wg, Wu = np64(x["H"]), np64(x["W_gate"]), np64(x["W_up"])
    _check(GU[0], H @ Wg.T, cfg, "G")
    _check(GU[1], H @ Wu.T, cfg, "U")
    ref = oracle.backward_z(H, Wg, Wu, np64(c["dZ"]))
    _check(g.dH, ref["dH"], cfg, "dH")
    _check(g.dW_gate, ref["dW_gate"], cfg, "dW_gate")
    _check(g.dW_up, ref["dW_up"], cfg, "dW_up")


@pytest.mark.parametrize("clip", list(TAUS))
@pytest.mark.parametrize("name", list(CASES))
def test_forward_backward_end_to_end(name, clip):
    """forward -> backward on the GPU against oracle.backward from H and X0:
    all seven input gradients."""
    cfg, docs = CASES[name]
    tau = TAUS[clip]
    x = inputs.make_inputs(cfg, 24, "cuda", doc_starts=docs)
    c = inputs.make_cotangents(cfg, 24, "cuda")
    print(f"[{name}] forward + backward, tau {tau}", flush=True)
    p = _problem(cfg, docs)
    buf = ip.allocate(p, "cuda")
    ip.forward(p, x["H"], x["X0"], x["W_gate"], x["W_up"], x["W_down"], x["conv_w"], x["W_target"], x["eta"], tau,
               buf)
    g = ip.backward(p, buf, x["H"], x["X0"], x["W_gate"], x["W_up"], x["W_down"], x["conv_w"], x["W_target"],
                    x["eta"], tau, c["dO"])
    torch.cuda.synchronize()
    x64 = inputs.to_f64(x)
    ref = oracle.backward(x64["H"], x64["X0"], x64["W_gate"], x64["W_up"], x64["W_down"], x64["conv_w"],
                          x64["W_target"], np64(c["dO"]), rows=cfg.rows, T=cfg.seq_len, C=cfg.chunk,
                          eta=x["eta"], tau=tau, doc_starts=docs)
    for k in ("dH", "dX0", "dW_gate", "dW_up", "dW_down", "dconv_w", "dW_target"):
        _check(getattr(g, k), ref[k], cfg, k)


@pytest.mark.parametrize("saved", ["saved", "alpha_only"])
@pytest.mark.parametrize("clip", list(TAUS))
@pytest.mark.parametrize("name", list(CASES))
def test_forward_backward_from_saved_state(name, clip, saved):
    """ipttt_z_save and ipttt_scan_apply_save in the forward, then
    ipttt_scan_apply_backward_saved with the forward's clip scales and either
    its saved chunk weights or none (recomputed), and ipttt_z_backward_saved:
    all seven input gradients against oracle.backward."""
    cfg, docs = CASES[name]
    tau = TAUS[clip]
    x = inputs.make_inputs(cfg, 26, "cuda", doc_starts=docs)
    c = inputs.make_cotangents(cfg, 26, "cuda")
    print(f"[{name}] forward (save) + backward ({saved}), tau {tau}", flush=True)
    p = _problem(cfg, docs)
    buf = ip.allocate(p, "cuda", save=True)
    if cfg.dtype == "bf16" and cfg.d_model % 64 == 0 and cfg.d_ff % 64 == 0:
        assert buf.saved is not None and buf.saved.numel() == ip.ipttt_saved_bytes(p)
    else:
        assert buf.saved is None
    if saved == "alpha_only":
        buf.saved = None
    ip.forward(p, x["H"], x["X0"], x["W_gate"], x["W_up"], x["W_down"], x["conv_w"], x["W_target"], x["eta"], tau,
               buf)
    g = ip.Grads(p, "cuda")
    ip.ipttt_scan_apply_backward_saved(p, buf.Z, buf.V, x["W_down"], x["eta"], tau, buf.alpha, buf.saved, c["dO"],
                                       g.dZ, g.dV, g.dW_down, g.ws)
    ip.ipttt_target_backward(p, x["X0"], x["conv_w"], x["W_target"], g.dV, g.dX0, g.dconv_w, g.dW_target, g.ws)
    ip.ipttt_z_backward_saved(p, x["H"], x["W_gate"], x["W_up"], buf.GU, g.dZ, g.dH, g.dW_gate, g.dW_up, g.ws)
    torch.cuda.synchronize()
    x64 = inputs.to_f64(x)
    ref = oracle.backward(x64["H"], x64["X0"], x64["W_gate"], x64["W_up"], x64["W_down"], x64["conv_w"],
                          x64["W_target"], np64(c["dO"]), rows=cfg.rows, T=cfg.seq_len, C=cfg.chunk,
                          eta=x["eta"], tau=tau, doc_starts=docs)
    for k in ("dH", "dX0", "dW_gate", "dW_up", "dW_down", "dconv_w", "dW_target"):
        _check(getattr(g, k), ref[k], cfg, k)


def test_saved_state_backward_matches_recomputing_one():
    """The saved-state backward and the recomputing one take the same inputs
    through the same kernels apart from where the chunk weights and the clip
    norms come from: their gradients agree to a few bf16 roundings."""
    cfg, docs = CASES["bf16_wide"]
    tau = TAUS["clip"]
    x = inputs.make_inputs(cfg, 27, "cuda", doc_starts=docs)
    c = inputs.make_cotangents(cfg, 27, "cuda")
    p = _problem(cfg, docs)
    buf = ip.allocate(p, "cuda", save=True)
    ip.forward(p, x["H"], x["X0"], x["W_gate"], x["W_up"], x["W_down"], x["conv_w"], x["W_target"], x["eta"], tau,
               buf)
    a = ip.Grads(p, "cuda")
    b = ip.Grads(p, "cuda")
    ip.ipttt_scan_apply_backward_saved(p, buf.Z, buf.V, x["W_down"], x["eta"], tau, buf.alpha, buf.saved, c["dO"],
                                       a.dZ, a.dV, a.dW_down, a.ws)
    ip.ipttt_scan_apply_backward(p, buf.Z, buf.V, x["W_down"], x["eta"], tau, c["dO"], b.dZ, b.dV, b.dW_down, b.ws)
    torch.cuda.synchronize()
    for k in ("dZ", "dV", "dW_down"):
        r = rel(np64(getattr(a, k)), np64(getattr(b, k)))
        print(f"    {k}: saved vs recomputed rel {r:.2e}", flush=True)
        assert r <= 2e-3, k


# ------------------------------------------------------------- full size

FULL = {"4b_32k": C["4b_32k"], "4b_128k": C["4b_128k"],
        # a chunk that is not a whole number of 64-token stages
        "4b_32k_c500": C["4b_32k"].with_(name="4b_32k_c500", chunk=500)}


@pytest.mark.parametrize("name", list(FULL))
def test_backward_full_size_first_chunks(name):
    """4B workloads (1 x 32768 tokens with C 512 or 500, and 1 x 131072 tokens
    with C 1024; d 2560, f 9728, clip 1e-5) in the launch configuration
    bench.py --backward times (the forward saves its gate products and chunk
    weights, the backward reuses them), with dO zero outside the first two
    chunks.  Nothing after chunk 1 then receives a gradient: dH and dX0 are
    exactly zero from there on, and every gradient equals that of the first
    two chunks alone, which the oracle computes."""
    cfg = FULL[name]
    K = 2
    n = K * cfg.chunk
    x = inputs.make_inputs(cfg, 25, "cuda")
    dO = inputs.make_cotangents(cfg, 25, "cuda")["dO"]
    dO[n:] = 0
    print(f"[{name}] forward (saved state) + backward, dO on the first two chunks", flush=True)
    p = _problem(cfg, None)
    buf = ip.allocate(p, "cuda", save=True)
    assert buf.saved is not None
    ip.forward(p, x["H"], x["X0"], x["W_gate"], x["W_up"], x["W_down"], x["conv_w"], x["W_target"], x["eta"],
               x["tau"], buf)
    g = ip.backward(p, buf, x["H"], x["X0"], x["W_gate"], x["W_up"], x["W_down"], x["conv_w"], x["W_target"],
                    x["eta"], x["tau"], dO)
    torch.cuda.synchronize()
    assert torch.count_nonzero(g.dH[n:]).item() == 0
    assert torch.count_nonzero(g.dX0[n:]).item() == 0
    got = {k: np64(getattr(g, k)) for k in ("dW_gate", "dW_up", "dW_down", "dconv_w", "dW_target")}
    got["dH"], got["dX0"] = np64(g.dH[:n]), np64(g.dX0[:n])
    del buf, g
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    w = {k: np64(x[k]) for k in ("W_gate", "W_up", "W_down", "conv_w", "W_target")}
    ref = oracle.backward(np64(x["H"][:n]), np64(x["X0"][:n]), w["W_gate"], w["W_up"], w["W_down"], w["conv_w"],
                          w["W_target"], np64(dO[:n]), rows=1, T=n, C=cfg.chunk, eta=x["eta"], tau=x["tau"])
    for k, v in got.items():
        _check(v, ref[k], cfg, k)


def test_backward_small_bf16_whole_row():
    """The small bf16 configuration at full width (d 1024, f 4096, C 512, no
    clip) over one whole 8192-token row, forward with saved state and
    backward with the output cotangent on every token: all gradients against
    the oracle, so the reverse scan carries adjoints through all 16 chunks
    of a full-width row."""
    cfg = C["small_bf16"].with_(rows=1)
    x = inputs.make_inputs(cfg, 27, "cuda")
    dO = inputs.make_cotangents(cfg, 27, "cuda")["dO"]
    print("[small_bf16] one whole row: forward (saved state) + backward, dO on every token", flush=True)
    p = _problem(cfg, None)
    buf = ip.allocate(p, "cuda", save=True)
    ip.forward(p, x["H"], x["X0"], x["W_gate"], x["W_up"], x["W_down"], x["conv_w"], x["W_target"], x["eta"],
               x["tau"], buf)
    g = ip.backward(p, buf, x["H"], x["X0"], x["W_gate"], x["W_up"], x["W_down"], x["conv_w"], x["W_target"],
                    x["eta"], x["tau"], dO)
    torch.cuda.synchronize()
    got = {k: np64(getattr(g, k)) for k in ("dH", "dX0", "dW_gate", "dW_up", "dW_down", "dconv_w", "dW_target")}
    del buf, g
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    w = {k: np64(x[k]) for k in ("W_gate", "W_up", "W_down", "conv_w", "W_target")}
    ref = oracle.backward(np64(x["H"]), np64(x["X0"]), w["W_gate"], w["W_up"], w["W_down"], w["conv_w"],
                          w["W_target"], np64(dO), rows=1, T=cfg.seq_len, C=cfg.chunk, eta=x["eta"], tau=x["tau"])
    for k, v in got.items():
        _check(v, ref[k], cfg, k)


def test_backward_packed_documents_full_size_first_chunks():
    """8 x 32768 packed rows (documents off the chunk grid) at full width, in
    the launch configuration bench.py --backward --config 4b_packed times,
    with dO zero outside the first two chunks of rows 0-3 (and on all of rows
    4-7): dH and dX0 vanish everywhere else, and every gradient equals that of
    the 4 x 1024-token problem of those chunks, documents inside them
    included, which the oracle computes."""
    cfg = C["4b_packed"]
    K, keep = 2, 4
    n = K * cfg.chunk
    # seed 31 puts document starts into chunks 0 and 1 of rows 1 and 2
    x = inputs.make_inputs(cfg, 31, "cuda")
    docs = [int(s) for s in x["doc_starts"]]
    dO = inputs.make_cotangents(cfg, 31, "cuda")["dO"]
    dO3 = dO.view(cfg.rows, cfg.seq_len, cfg.d_model)
    dO3[:, n:] = 0
    dO3[keep:] = 0
    print(f"[4b_packed] forward (saved state) + backward, dO on the first two chunks of rows 0-{keep - 1}", flush=True)
    p = _problem(cfg, docs)
    buf = ip.allocate(p, "cuda", save=True)
    ip.forward(p, x["H"], x["X0"], x["W_gate"], x["W_up"], x["W_down"], x["conv_w"], x["W_target"], x["eta"],
               x["tau"], buf)
    g = ip.backward(p, buf, x["H"], x["X0"], x["W_gate"], x["W_up"], x["W_down"], x["conv_w"], x["W_target"],
                    x["eta"], x["tau"], dO)
    torch.cuda.synchronize()
    dH3 = g.dH.view(cfg.rows, cfg.seq_len, -1)
    dX3 = g.dX0.view(cfg.rows, cfg.seq_len, -1)
    assert torch.count_nonzero(dH3[:, n:]).item() == 0 and torch.count_nonzero(dH3[keep:]).item() == 0
    assert torch.count_nonzero(dX3[:, n:]).item() == 0 and torch.count_nonzero(dX3[keep:]).item() == 0
    got = {k: np64(getattr(g, k)) for k in ("dW_gate", "dW_up", "dW_down", "dconv_w", "dW_target")}
    got["dH"] = np64(dH3[:keep, :n].reshape(keep * n, -1))
    got["dX0"] = np64(dX3[:keep, :n].reshape(keep * n, -1))
    sub = lambda t: np64(t.view(cfg.rows, cfg.seq_len, -1)[:keep, :n].reshape(keep * n, -1))
    H, X0, dOs = sub(x["H"]), sub(x["X0"]), sub(dO)
    del buf, g
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    # document starts inside the kept chunks, renumbered for rows of n tokens
    sd = [(s // cfg.seq_len) * n + s % cfg.seq_len for s in docs if s // cfg.seq_len < keep and s % cfg.seq_len < n]
    assert len(sd) > 0
    w = {k: np64(x[k]) for k in ("W_gate", "W_up", "W_down", "conv_w", "W_target")}
    ref = oracle.backward(H, X0, w["W_gate"], w["W_up"], w["W_down"], w["conv_w"], w["W_target"], dOs, rows=keep,
                          T=n, C=cfg.chunk, eta=x["eta"], tau=x["tau"], doc_starts=sd)
    for k, v in got.items():
        _check(v, ref[k], cfg, k)
