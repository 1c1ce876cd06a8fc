"""GPU tests of the scan's 256 x 128 state tiles at small sizes.

The forward and reverse scans cover the d x f state with as many 256 x 256
tiles as there are CUs and put the remaining f rows on 256 x 128 tiles.  At
the 4B shape that second kind runs the last 13 of 38 f rows; at the narrow
shapes of the other tests every tile is of the first kind.  IPTTT_SCAN_CUS
makes the plan assume fewer CUs, so that a narrow problem runs on both kinds:
with d 320 and f 448 and a plan for 2 CUs, f rows 0-255 take two 256 x 256
tiles and f rows 256-447 three 256 x 128 tiles, the last of them 64 columns
wide.  Every state element is accumulated over the same tokens in the same
order on both kinds, so outputs, saved chunk weights, the carried state and
the gradients must equal those of the default plan bit for bit, and match
the oracle (the exclusive prefix of lijianxiong.blog "In-Place Test-Time
Training", 工程实现; the reset at document starts of iplexlaw.co.kr review,
section 6) within the bf16 tolerance.
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

# ragged everywhere: d and f one and a half 256-tiles wide at most, a short
# last chunk, document starts inside chunks and at a chunk's first token
CFG = inputs.CONFIGS["4b_32k"].with_(name="scan_plan", d_model=320, d_ff=448, rows=2, seq_len=777, chunk=128,
                                     eta=1e-2, tau=1e-3)
DOCS = [100, 256, 300, 777 + 200]
SMALL_PLAN = "2"


def _problem(continues=None):
    return ip.Problem(CFG.rows, CFG.seq_len, CFG.d_model, CFG.d_ff, CFG.chunk, ip.IPTTT_BF16, DOCS,
                      continues=continues)


def _prep(seed, W_down_zero):
    x = inputs.make_inputs(CFG, seed, "cuda", doc_starts=DOCS)
    if W_down_zero:
        x["W_down"] = torch.zeros_like(x["W_down"])
    p = _problem()
    buf = ip.allocate(p, "cuda")
    ip.ipttt_z(p, x["H"], x["W_gate"], x["W_up"], buf.Z)
    ip.ipttt_target(p, x["X0"], x["conv_w"], x["W_target"], buf.V, buf.ws)
    ip.ipttt_chunk_delta(p, buf.V, buf.Z, x["eta"], x["tau"], buf.alpha, None, buf.ws)
    torch.cuda.synchronize()
    return x, p, buf


def _forward_calls(x, p, buf):
    """The scan/apply calls that run the forward scan: plain, saving the
    chunk weights, and carrying a state in and out."""
    O = torch.zeros_like(buf.O)
    ip.ipttt_scan_apply(p, buf.Z, buf.V, x["W_down"], buf.alpha, x["eta"], O, buf.ws)
    saved = torch.zeros(ip.ipttt_saved_bytes(p), dtype=torch.uint8, device="cuda")
    Os = torch.zeros_like(buf.O)
    ip.ipttt_scan_apply_save(p, buf.Z, buf.V, x["W_down"], buf.alpha, x["eta"], Os, saved, buf.ws)
    pc = _problem(continues=[1, 0])
    g = torch.Generator(device="cuda").manual_seed(3)
    S_in = torch.randn(CFG.rows, CFG.d_model, CFG.d_ff, device="cuda", generator=g) * 1e-3
    S_out = torch.zeros_like(S_in)
    Oc = torch.zeros_like(buf.O)
    ip.ipttt_scan_apply_carry(pc, buf.Z, buf.V, x["W_down"], buf.alpha, x["eta"], S_in, S_out, Oc, buf.ws)
    torch.cuda.synchronize()
    return {"O": O, "O_save": Os, "saved": saved, "O_carry": Oc, "S_out": S_out}


@pytest.mark.parametrize("w_down", ["zero", "drawn"])
def test_forward_scan_on_both_tile_kinds(w_down, monkeypatch):
    monkeypatch.delenv("IPTTT_SCAN_CUS", raising=False)
    x, p, buf = _prep(31, w_down == "zero")
    ref = _forward_calls(x, p, buf)
    monkeypatch.setenv("IPTTT_SCAN_CUS", SMALL_PLAN)
    got = _forward_calls(x, p, buf)
    for k in ref:
        assert torch.equal(got[k], ref[k]), k
    # against the oracle's sequential loop; with W_down = 0, O is the
    # fast-weight term alone
    w = {k: np64(x[k]) for k in ("H", "X0", "W_gate", "W_up", "W_down", "conv_w", "W_target")}
    o = oracle.forward(w["H"], w["X0"], w["W_gate"], w["W_up"], w["W_down"], w["conv_w"], w["W_target"],
                       rows=CFG.rows, T=CFG.seq_len, C=CFG.chunk, eta=x["eta"], tau=x["tau"], doc_starts=DOCS)
    r = rel(np64(got["O"]), o["O"])
    ra = rel(np64(buf.alpha).reshape(o["alpha"].shape), o["alpha"])
    print(f"  [{w_down}] O rel {r:.2e}, alpha rel {ra:.2e}", flush=True)
    assert r <= tol(CFG)
    assert ra <= tol(CFG)


def test_reverse_scan_on_both_tile_kinds(monkeypatch):
    x = inputs.make_inputs(CFG, 32, "cuda", doc_starts=DOCS)
    c = inputs.make_cotangents(CFG, 32, "cuda")
    p = _problem()

    def run():
        g = ip.Grads(p, "cuda")
        ip.ipttt_scan_apply_backward(p, c["Z"], c["V"], x["W_down"], x["eta"], x["tau"], c["dO"], g.dZ, g.dV,
                                     g.dW_down, g.ws)
        torch.cuda.synchronize()
        return g

    monkeypatch.delenv("IPTTT_SCAN_CUS", raising=False)
    a = run()
    monkeypatch.setenv("IPTTT_SCAN_CUS", SMALL_PLAN)
    b = run()
    for k in ("dZ", "dV", "dW_down"):
        assert torch.equal(getattr(b, k), getattr(a, k)), k
    ref = oracle.backward_scan_apply(np64(c["Z"]), np64(c["V"]), np64(x["W_down"]), np64(c["dO"]),
                                     rows=CFG.rows, T=CFG.seq_len, C=CFG.chunk, eta=x["eta"], tau=x["tau"],
                                     doc_starts=DOCS)
    for k in ("dZ", "dV", "dW_down"):
        r = rel(np64(getattr(b, k)), ref[k])
        print(f"  {k} rel {r:.2e}", flush=True)
        assert r <= tol(CFG), k


def test_plan_setting_out_of_range_is_ignored(monkeypatch):
    """Values that are not a positive count leave the device's CU count in
    place (same outputs as without the setting)."""
    x, p, buf = _prep(33, False)
    monkeypatch.delenv("IPTTT_SCAN_CUS", raising=False)
    O1 = torch.zeros_like(buf.O)
    ip.ipttt_scan_apply(p, buf.Z, buf.V, x["W_down"], buf.alpha, x["eta"], O1, buf.ws)
    for v in ("0", "-4", "x", ""):
        monkeypatch.setenv("IPTTT_SCAN_CUS", v)
        O2 = torch.zeros_like(buf.O)
        ip.ipttt_scan_apply(p, buf.Z, buf.V, x["W_down"], buf.alpha, x["eta"], O2, buf.ws)
        torch.cuda.synchronize()
        assert torch.equal(O2, O1), v
