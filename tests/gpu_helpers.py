"""Shared helpers of the GPU parity tests: run the HIP path through the C ABI
and the fp64 oracle on the same seeded inputs, and compare."""
import numpy as np
import torch

import oracle
import test_weight_mlp_amd as ip
from test_weight_mlp_amd import inputs


def rel(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    nb = np.linalg.norm(b)
    return np.linalg.norm(a - b) / (nb if nb > 0 else 1.0)


def tol(cfg):
    """Frobenius-relative parity bound: 1e-4 for fp32 data, 1e-2 for bf16."""
    return 1e-4 if cfg.dtype == "f32" else 1e-2


def problem(cfg, doc_starts):
    dt = ip.IPTTT_F32 if cfg.dtype == "f32" else ip.IPTTT_BF16
    return ip.Problem(cfg.rows, cfg.seq_len, cfg.d_model, cfg.d_ff, cfg.chunk, dt, doc_starts)


def run_gpu(cfg, x, want_dW=False, W_down=None):
    p = problem(cfg, x["doc_starts"])
    buf = ip.allocate(p, "cuda", want_dW=want_dW)
    ip.forward(p, x["H"], x["X0"], x["W_gate"], x["W_up"],
               x["W_down"] if W_down is None else W_down, x["conv_w"], x["W_target"],
               x["eta"], x["tau"], buf)
    torch.cuda.synchronize()
    return p, buf


def run_oracle(cfg, x64, want_dW=False, W_down=None, max_chunks=None):
    return oracle.forward(x64["H"], x64["X0"], x64["W_gate"], x64["W_up"],
                          x64["W_down"] if W_down is None else W_down, x64["conv_w"],
                          x64["W_target"], rows=cfg.rows, T=cfg.seq_len, C=cfg.chunk,
                          eta=x64["eta"], tau=x64["tau"], doc_starts=x64["doc_starts"],
                          want_dW=want_dW, max_chunks=max_chunks)


def np64(t):
    return t.detach().to("cpu", torch.float64).numpy()
