"""Seeded synthetic inputs for the In-Place TTT layer forward.

This module only draws random numbers and packs document boundaries; it holds
none of the layer's arithmetic.  Both the HIP path (tests, bench) and the fp64
oracle consume what it returns, so the two sides always see the same rounded
values.

Shapes and distributions follow the workloads the pages describe: a 4B-class
gated MLP (d_model 2560, d_ff 9728), chunks of 512 or 1024 tokens, 32k to 128k
context, a depthwise k=5 convolution and a near-diagonal W_target.  ``N(0, v)``
below means variance ``v``; weights are ``N(0, 1/fan_in)``.

Every tensor is drawn in fp32 from its own ``torch.Generator`` (seeded from
``numpy.random.SeedSequence(seed)``), then rounded once with round-to-nearest-
even to the configuration dtype.  Drawing happens on the device the caller
names, so full-size inputs can be made directly in HBM.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np
import torch

# Fixed draw order: the i-th tensor always uses the i-th spawned seed.
TENSOR_ORDER = ("H", "X0", "W_gate", "W_up", "W_down", "W_target", "conv_w", "doc_lengths")


@dataclasses.dataclass(frozen=True)
class Config:
    name: str
    d_model: int
    d_ff: int
    rows: int
    seq_len: int
    chunk: int
    eta: float
    tau: float          # <= 0: no clip
    dtype: str          # "f32" or "bf16"
    conv_var: float
    target_kind: str    # "normal" (N(0,1/d)) or "sparse_diag" (I + 1% N(0,1e-2) off-diagonal)
    docs: str           # "one" (one document per row) or "loguniform"
    description: str = ""

    @property
    def n_chunks(self) -> int:
        return -(-self.seq_len // self.chunk)

    @property
    def tokens(self) -> int:
        return self.rows * self.seq_len

    def with_(self, **kw) -> "Config":
        return dataclasses.replace(self, **kw)


CONFIGS = {
    "tiny_f32": Config("tiny_f32", 64, 256, 1, 128, 16, 1e-2, 0.0, "f32", 0.1, "normal", "one",
                       "d64 f256, 1x128 tokens, C16, fp32, no clip"),
    "small_bf16": Config("small_bf16", 1024, 4096, 4, 8192, 512, 1e-3, 0.0, "bf16", 1e-2,
                         "sparse_diag", "one",
                         "d1024 f4096, 4x8192 tokens, C512, bf16, no clip"),
    "4b_32k": Config("4b_32k", 2560, 9728, 1, 32768, 512, 1e-3, 1e-5, "bf16", 0.05, "normal", "one",
                     "d2560 f9728, 1x32768 tokens, C512, bf16, clip 1e-5"),
    "4b_128k": Config("4b_128k", 2560, 9728, 1, 131072, 1024, 1e-3, 1e-5, "bf16", 0.05, "normal",
                      "one", "d2560 f9728, 1x131072 tokens, C1024, bf16, clip 1e-5"),
    "4b_packed": Config("4b_packed", 2560, 9728, 8, 32768, 512, 1e-3, 1e-5, "bf16", 0.05, "normal",
                        "loguniform",
                        "d2560 f9728, 8x32768 tokens, C512, bf16, clip 1e-5, packed documents"),
}


def torch_dtype(cfg: Config) -> torch.dtype:
    return torch.float32 if cfg.dtype == "f32" else torch.bfloat16


def _seeds(seed: int) -> dict:
    ss = np.random.SeedSequence(seed).spawn(len(TENSOR_ORDER))
    return {name: int(s.generate_state(1, dtype=np.uint64)[0] & 0x7FFF_FFFF_FFFF_FFFF)
            for name, s in zip(TENSOR_ORDER, ss)}


def _normal(shape, std, seed, device) -> torch.Tensor:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return torch.randn(shape, generator=g, device=device, dtype=torch.float32) * std


def _uniform(shape, seed, device) -> torch.Tensor:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return torch.rand(shape, generator=g, device=device, dtype=torch.float32)


def loguniform_doc_starts(rows: int, seq_len: int, chunk: int, seed: int,
                          lo: int = 256, hi: int = 32768) -> np.ndarray:
    """Flat document-start offsets (row starts excluded) for packed rows.

    Lengths are floor(exp(U(ln lo, ln hi))), drawn per row until the row is
    full; the last document is cut at the row end.  A length whose boundary
    would land on a multiple of ``chunk`` is drawn again, so boundaries never
    align with the chunk grid.
    """
    rng = np.random.default_rng(seed)
    starts = []
    for r in range(rows):
        pos = 0
        while True:
            while True:
                length = int(math.floor(math.exp(rng.uniform(math.log(lo), math.log(hi)))))
                if (pos + length) % chunk != 0 or pos + length >= seq_len:
                    break
            pos += length
            if pos >= seq_len:
                break
            starts.append(r * seq_len + pos)
    return np.asarray(starts, dtype=np.int64)


def make_inputs(cfg: Config, seed: int = 0, device: str = "cpu",
                doc_starts: Optional[np.ndarray] = None) -> dict:
    """Draw one problem instance.

    Returns torch tensors in the configuration dtype on ``device``:
    H, X0 [rows*seq_len, d]; W_gate, W_up [f, d]; W_down [d, f];
    W_target [d_in, d_out]; conv_w [d, 5]; and ``doc_starts`` as an int64
    numpy array of flat offsets (row starts excluded; empty for one document
    per row), plus the scalars eta and tau.
    """
    s = _seeds(seed)
    d, f, n = cfg.d_model, cfg.d_ff, cfg.tokens
    dt = torch_dtype(cfg)
    out = {
        "H": _normal((n, d), 1.0, s["H"], device).to(dt),
        "X0": _normal((n, d), 1.0, s["X0"], device).to(dt),
        "W_gate": _normal((f, d), 1.0 / math.sqrt(d), s["W_gate"], device).to(dt),
        "W_up": _normal((f, d), 1.0 / math.sqrt(d), s["W_up"], device).to(dt),
        "W_down": _normal((d, f), 1.0 / math.sqrt(f), s["W_down"], device).to(dt),
    }
    if cfg.target_kind == "sparse_diag":
        noise = _normal((d, d), 0.1, s["W_target"], device)
        g = torch.Generator(device=device)
        g.manual_seed(s["W_target"] ^ 0x5DEECE66D)
        mask = torch.rand((d, d), generator=g, device=device) < 0.01
        wt = torch.where(mask, noise, torch.zeros_like(noise))
        wt.fill_diagonal_(1.0)
        out["W_target"] = wt.to(dt)
    else:
        out["W_target"] = _normal((d, d), 1.0 / math.sqrt(d), s["W_target"], device).to(dt)
    out["conv_w"] = _normal((d, 5), math.sqrt(cfg.conv_var), s["conv_w"], device).to(dt)
    if doc_starts is None:
        if cfg.docs == "loguniform":
            doc_starts = loguniform_doc_starts(cfg.rows, cfg.seq_len, cfg.chunk, s["doc_lengths"])
        else:
            doc_starts = np.zeros(0, dtype=np.int64)
    out["doc_starts"] = np.asarray(doc_starts, dtype=np.int64)
    out["eta"] = float(cfg.eta)
    out["tau"] = float(cfg.tau)
    return out


def to_f64(inputs: dict) -> dict:
    """Exact fp64 numpy copies of the tensors (bf16 and fp32 widen exactly)."""
    res = {}
    for k, v in inputs.items():
        if isinstance(v, torch.Tensor):
            res[k] = v.detach().to("cpu", torch.float64).numpy()
        else:
            res[k] = v
    return res


def make_cotangents(cfg: Config, seed: int = 0, device: str = "cpu") -> dict:
    """Seeded stand-ins for the tensors the backward calls take besides the
    forward's inputs, in the configuration dtype: dO [rows*seq_len, d] (the
    output's cotangent, N(0, 1)); and, to test a backward call on its own,
    Z [tokens, f] ~ N(0, 1/4), V [tokens, d] ~ N(0, 1/4), dV [tokens, d]
    and dZ [tokens, f] ~ N(0, 1)."""
    ss = np.random.SeedSequence([seed, 0xBAC]).spawn(5)
    sd = [int(s.generate_state(1, dtype=np.uint64)[0] & 0x7FFF_FFFF_FFFF_FFFF) for s in ss]
    d, f, n = cfg.d_model, cfg.d_ff, cfg.tokens
    dt = torch_dtype(cfg)
    return {
        "dO": _normal((n, d), 1.0, sd[0], device).to(dt),
        "Z": _normal((n, f), 0.5, sd[1], device).to(dt),
        "V": _normal((n, d), 0.5, sd[2], device).to(dt),
        "dV": _normal((n, d), 1.0, sd[3], device).to(dt),
        "dZ": _normal((n, f), 1.0, sd[4], device).to(dt),
    }
