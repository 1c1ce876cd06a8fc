"""GPU parity of the ablated targets (tencent article "榨干MLP的剩余价值",
验证模块三, objective decoupling): V_hat = X0 W_target without the conv, and
V_hat = Conv1D(X0) without the projection, through the whole layer, on the
bf16 8-wave kernels and on the general kernels (fp32, and bf16 widths that
are not multiples of 64).  The unused weight is passed as NULL."""
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
    "bf16_fast": (C["4b_32k"].with_(name="bf16_fast", d_model=256, d_ff=384, rows=2, seq_len=1300,
                                    chunk=256), [700, 1300 + 100]),
    "bf16_general": (C["4b_32k"].with_(name="bf16_general", d_model=136, d_ff=200, rows=1,
                                       seq_len=600, chunk=128), [333]),
    "f32_general": (C["tiny_f32"].with_(name="f32_general", d_model=72, d_ff=136, rows=2, seq_len=300,
                                        chunk=48, tau=2e-2, eta=5e-2), [77, 300 + 5]),
}
TARGETS = {ip.IPTTT_TARGET_NO_CONV: "no_conv", ip.IPTTT_TARGET_NO_PROJ: "no_proj"}


@pytest.mark.parametrize("target", list(TARGETS))
@pytest.mark.parametrize("name", list(CASES))
def test_target_variant_parity(name, target):
    cfg, docs = CASES[name]
    x = inputs.make_inputs(cfg, 4, "cuda", doc_starts=docs)
    x64 = inputs.to_f64(x)
    mode = TARGETS[target]
    print(f"[{name}] target {mode}", flush=True)
    dt = ip.IPTTT_F32 if cfg.dtype == "f32" else ip.IPTTT_BF16
    p = ip.Problem(cfg.rows, cfg.seq_len, cfg.d_model, cfg.d_ff, cfg.chunk, dt, x["doc_starts"],
                   target=target)
    buf = ip.allocate(p, "cuda")
    conv = None if target == ip.IPTTT_TARGET_NO_CONV else x["conv_w"]
    wt = None if target == ip.IPTTT_TARGET_NO_PROJ else x["W_target"]
    ip.forward(p, x["H"], x["X0"], x["W_gate"], x["W_up"], x["W_down"], conv, wt, x["eta"], x["tau"], buf)
    torch.cuda.synchronize()
    ref = oracle.forward(x64["H"], x64["X0"], x64["W_gate"], x64["W_up"], x64["W_down"], x64["conv_w"],
                         x64["W_target"], rows=cfg.rows, T=cfg.seq_len, C=cfg.chunk, eta=x64["eta"],
                         tau=x64["tau"], doc_starts=x64["doc_starts"], target=mode)
    assert rel(np64(buf.V), ref["V"]) <= tol(cfg)
    assert rel(np64(buf.alpha), ref["alpha"]) <= tol(cfg)
    assert rel(np64(buf.O), ref["O"]) <= tol(cfg)
    # the fast-weight term alone (W_down = 0), where the target matters most
    ip.forward(p, x["H"], x["X0"], x["W_gate"], x["W_up"], torch.zeros_like(x["W_down"]), conv, wt,
               x["eta"], x["tau"], buf)
    torch.cuda.synchronize()
    ref0 = oracle.forward(x64["H"], x64["X0"], x64["W_gate"], x64["W_up"], np.zeros_like(x64["W_down"]),
                          x64["conv_w"], x64["W_target"], rows=cfg.rows, T=cfg.seq_len, C=cfg.chunk,
                          eta=x64["eta"], tau=x64["tau"], doc_starts=x64["doc_starts"], target=mode)
    assert rel(np64(buf.O), ref0["O"]) <= tol(cfg)
