"""GPU tests of the scan and apply run in windows of a row's chunks.

A row whose per-chunk weights exceed the pass budget is walked in windows of
whole chunks; the fp32 state after a window's last chunk goes through the
workspace to the next window.  The state a chunk applies is the exclusive
prefix sum of its document's earlier clipped deltas (lijianxiong.blog
"In-Place Test-Time Training", 工程实现), restarted at each document start
(iplexlaw.co.kr review, section 6), so cutting the walk at a chunk boundary
changes nothing: every output, saved weight, carried state and diagnostic
delta must equal the one-pass result bit for bit, and the windowed run must
match the oracle.  IPTTT_PASS_BYTES shrinks the budget so that narrow shapes
take several windows; the 4B/128k row takes windows at the default budget.
"""
import numpy as np
import pytest
import torch

import oracle
import test_weight_mlp_amd as ip
from test_weight_mlp_amd import inputs
from gpu_helpers import np64, problem, rel, tol

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

# d and f multiples of 64: the 8-wave kernels, which run in passes; wide
# enough that the scan's regions set the workspace size
NARROW = inputs.CONFIGS["small_bf16"].with_(name="narrow_windows", d_model=512, d_ff=1024, rows=1, seq_len=4000,
                                            chunk=256, tau=1e-3, eta=0.05)


def _budget(cfg, chunks):
    """A pass budget that holds `chunks` chunks of one row: their weights and
    scaled V_hat, W_down's fragments and the carried fp32 state."""
    wd = cfg.d_model * cfg.d_ff * 2
    return wd + cfg.d_model * cfg.d_ff * 4 + chunks * (wd + cfg.chunk * cfg.d_model * 2)


def _docs(cfg, kind):
    C, T = cfg.chunk, cfg.seq_len
    if kind == "one":
        return np.zeros(0, np.int64)
    # inside chunks, at a window boundary (chunk 3 with 3-chunk windows), a
    # one-token document, and a start at the last chunk's first token
    s = [C + 17, 3 * C, 5 * C + 200, 5 * C + 201, 9 * C + 5, (cfg.n_chunks - 1) * C]
    return np.asarray(sorted(set(v for v in s if 0 < v < T)), np.int64)


def _scan_launches(fn):
    n = [0]

    def hook(name, stream):
        if name == "scan":
            n[0] += 1

    ip.ipttt_set_launch_hook(hook)
    try:
        fn()
        torch.cuda.synchronize()
    finally:
        ip.ipttt_set_launch_hook(None)
    return n[0]


def _prep(cfg, seed, ds):
    x = inputs.make_inputs(cfg, seed, "cuda", doc_starts=ds)
    p = problem(cfg, x["doc_starts"])
    buf = ip.allocate(p, "cuda")
    ip.ipttt_z(p, x["H"], x["W_gate"], x["W_up"], buf.Z)
    ip.ipttt_target(p, x["X0"], x["conv_w"], x["W_target"], buf.V, buf.ws)
    ip.ipttt_chunk_delta(p, buf.V, buf.Z, x["eta"], x["tau"], buf.alpha, None, buf.ws)
    torch.cuda.synchronize()
    return x, p, buf


@pytest.mark.parametrize("docs", ["one", "packed"])
def test_windows_equal_one_pass_and_the_oracle(docs, monkeypatch):
    cfg = NARROW
    monkeypatch.delenv("IPTTT_PASS_BYTES", raising=False)
    x, p, buf = _prep(cfg, 11, _docs(cfg, docs))
    O1 = torch.empty_like(buf.O)
    ip.ipttt_scan_apply(p, buf.Z, buf.V, x["W_down"], buf.alpha, x["eta"], O1, buf.ws)
    torch.cuda.synchronize()
    monkeypatch.setenv("IPTTT_PASS_BYTES", str(_budget(cfg, 3)))
    ws = torch.empty(ip.ipttt_workspace_bytes(p), dtype=torch.uint8, device="cuda")
    assert ws.numel() < buf.ws.numel()
    O3 = torch.zeros_like(buf.O)
    n = _scan_launches(lambda: ip.ipttt_scan_apply(p, buf.Z, buf.V, x["W_down"], buf.alpha, x["eta"], O3, ws))
    print(f"  [{docs}] {cfg.n_chunks} chunks in {n} windows", flush=True)
    assert n >= 3
    assert torch.equal(O3, O1)
    # the windowed run against the oracle's sequential loop
    w = {k: np64(x[k]) for k in ("H", "X0", "W_gate", "W_up", "W_down", "conv_w", "W_target")}
    ref = oracle.forward(w["H"], w["X0"], w["W_gate"], w["W_up"], w["W_down"], w["conv_w"], w["W_target"],
                         rows=1, T=cfg.seq_len, C=cfg.chunk, eta=x["eta"], tau=x["tau"],
                         doc_starts=list(x["doc_starts"]) or None)
    r = rel(np64(O3), ref["O"])
    print(f"  [{docs}] O rel {r:.2e}", flush=True)
    assert r <= tol(cfg)


def test_windows_with_a_larger_workspace_grow_back_to_one_pass(monkeypatch):
    """A workspace larger than the minimum gives longer windows, and one that
    holds the whole row a single pass; the outputs are the same."""
    cfg = NARROW
    monkeypatch.setenv("IPTTT_PASS_BYTES", str(_budget(cfg, 2)))
    x, p, buf = _prep(cfg, 12, _docs(cfg, "packed"))
    minimal = ip.ipttt_workspace_bytes(p)
    outs = []
    for extra, most in ((0, None), (6 * (cfg.d_model * cfg.d_ff * 2 + cfg.chunk * cfg.d_model * 2), None),
                        (cfg.n_chunks * cfg.d_model * cfg.d_ff * 2 + cfg.seq_len * cfg.d_model * 2, 1)):
        ws = torch.empty(minimal + extra, dtype=torch.uint8, device="cuda")
        O = torch.zeros_like(buf.O)
        n = _scan_launches(lambda: ip.ipttt_scan_apply(p, buf.Z, buf.V, x["W_down"], buf.alpha, x["eta"], O, ws))
        print(f"  workspace +{extra} bytes: {n} windows", flush=True)
        if most is not None:
            assert n == most
        outs.append((n, O))
    assert outs[0][0] > outs[1][0] > outs[2][0] == 1
    for _, O in outs[1:]:
        assert torch.equal(O, outs[0][1])


def test_saved_weights_and_carried_state_in_windows_equal_one_pass(monkeypatch):
    """ipttt_scan_apply_save writes every chunk's weights at its own offset,
    window by window; ipttt_scan_apply_carry hands S through the windows and
    out at the end (a continuing row started from S_in)."""
    cfg = NARROW
    monkeypatch.delenv("IPTTT_PASS_BYTES", raising=False)
    ds = _docs(cfg, "packed")
    x, p, buf = _prep(cfg, 13, ds)
    d, f = cfg.d_model, cfg.d_ff
    # chunks that start with a document start are never emitted: both saved
    # buffers start zeroed so that they compare whole
    saved1 = torch.zeros(ip.ipttt_saved_bytes(p), dtype=torch.uint8, device="cuda")
    O1 = torch.empty_like(buf.O)
    ip.ipttt_scan_apply_save(p, buf.Z, buf.V, x["W_down"], buf.alpha, x["eta"], O1, saved1, buf.ws)
    pc = ip.Problem(1, cfg.seq_len, d, f, cfg.chunk, ip.IPTTT_BF16, ds, continues=[1])
    g = torch.Generator(device="cuda").manual_seed(5)
    S_in = torch.randn(1, d, f, device="cuda", generator=g) * 1e-3
    S1 = torch.empty_like(S_in)
    Oc1 = torch.empty_like(buf.O)
    ip.ipttt_scan_apply_carry(pc, buf.Z, buf.V, x["W_down"], buf.alpha, x["eta"], S_in, S1, Oc1, buf.ws)
    torch.cuda.synchronize()

    monkeypatch.setenv("IPTTT_PASS_BYTES", str(_budget(cfg, 4)))
    ws = torch.empty(ip.ipttt_workspace_bytes(p), dtype=torch.uint8, device="cuda")
    saved4 = torch.zeros_like(saved1)
    O4 = torch.zeros_like(buf.O)
    n = _scan_launches(lambda: ip.ipttt_scan_apply_save(p, buf.Z, buf.V, x["W_down"], buf.alpha, x["eta"], O4,
                                                        saved4, ws))
    assert n >= 3
    assert torch.equal(O4, O1)
    assert torch.equal(saved4, saved1)
    ws = torch.empty(ip.ipttt_workspace_bytes(pc), dtype=torch.uint8, device="cuda")
    S4 = S_in.clone()  # in place: S_out = S_in
    Oc4 = torch.zeros_like(buf.O)
    n = _scan_launches(lambda: ip.ipttt_scan_apply_carry(pc, buf.Z, buf.V, x["W_down"], buf.alpha, x["eta"], S4,
                                                         S4, Oc4, ws))
    assert n >= 3
    assert torch.equal(Oc4, Oc1)
    assert torch.equal(S4, S1)


def test_diagnostic_deltas_in_windows_equal_one_pass(monkeypatch):
    """ipttt_chunk_delta's materialised deltas, made in windows of a row's
    chunks when a row's transposed copies exceed a quarter of the budget."""
    cfg = NARROW
    monkeypatch.delenv("IPTTT_PASS_BYTES", raising=False)
    x, p, buf = _prep(cfg, 14, _docs(cfg, "packed"))
    d, f = cfg.d_model, cfg.d_ff
    dW1 = torch.empty(cfg.n_chunks, d, f, device="cuda")
    a1 = torch.empty_like(buf.alpha)
    ip.ipttt_chunk_delta(p, buf.V, buf.Z, x["eta"], x["tau"], a1, dW1, buf.ws)
    torch.cuda.synchronize()
    per_chunk = 256 * (d + f) * 2
    monkeypatch.setenv("IPTTT_PASS_BYTES", str(4 * 3 * per_chunk))
    ws = torch.empty(ip.ipttt_workspace_bytes(p), dtype=torch.uint8, device="cuda")
    dW3 = torch.zeros_like(dW1)
    a3 = torch.zeros_like(a1)
    ip.ipttt_chunk_delta(p, buf.V, buf.Z, x["eta"], x["tau"], a3, dW3, ws)
    torch.cuda.synchronize()
    assert torch.equal(a3, a1)
    assert torch.equal(dW3, dW1)
