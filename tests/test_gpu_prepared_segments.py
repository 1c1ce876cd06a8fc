"""GPU tests of prepared segment descriptors (ipttt_problem.seg_table and
seg_bytes): a problem whose descriptors ipttt_segments_device built once must
give every call exactly what the calls give when each builds its own.

The descriptors encode the reset rule (iplexlaw.co.kr review, section 6: the
fast weight returns to W_down at every document start) and the conv's
zero padding at chunk ends and document starts (lijianxiong.blog
"In-Place Test-Time Training", 对齐语言模型的目标函数).  The cases put document
starts inside chunks, on chunk starts and at row starts, and flag a
continuing row, on both kernel families; the forward, the streamed call, the
allocation-free clip call and the backward are compared bit for bit, and the
prepared forward also against the oracle.
"""
import numpy as np
import pytest
import torch

import test_weight_mlp_amd as ip
from test_weight_mlp_amd import inputs
from gpu_helpers import np64, rel, run_oracle, tol

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

FAMILIES = {
    "general_f32": inputs.CONFIGS["tiny_f32"].with_(name="prepared_f32", rows=2, seq_len=100, d_model=72,
                                                    d_ff=136, chunk=16, eta=5e-2, tau=2e-2),
    "fast_bf16": inputs.CONFIGS["4b_32k"].with_(name="prepared_bf16", rows=2, seq_len=700, d_model=128,
                                                d_ff=192, chunk=128, eta=1e-2, tau=1e-3),
}
# flat token offsets: inside a chunk, on a chunk start, the second row's start
DOCS = {"general_f32": [21, 48, 100, 131], "fast_bf16": [200, 384, 700, 1000]}


def _problem(cfg, docs, continues=None):
    dt = ip.IPTTT_F32 if cfg.dtype == "f32" else ip.IPTTT_BF16
    return ip.Problem(cfg.rows, cfg.seq_len, cfg.d_model, cfg.d_ff, cfg.chunk, dt, docs, continues=continues)


def _both(cfg, docs, continues=None):
    plain = _problem(cfg, docs, continues)
    prepared = _problem(cfg, docs, continues).prepare_segments()
    return plain, prepared


@pytest.mark.parametrize("family", list(FAMILIES))
def test_prepared_descriptors_equal_the_built_ones(family):
    cfg = FAMILIES[family]
    p = _problem(cfg, DOCS[family], continues=[0, 1]).prepare_segments()
    table, segs = p._segments
    torch.cuda.synchronize()
    ref_t = torch.zeros_like(table)
    ref_s = torch.zeros_like(segs)
    ip.ipttt_segments_device(_problem(cfg, DOCS[family], continues=[0, 1]), ref_t, ref_s)
    torch.cuda.synchronize()
    assert torch.equal(table, ref_t) and torch.equal(segs, ref_s)
    host = ip.ipttt_segment_table(_problem(cfg, DOCS[family], continues=[0, 1]))
    assert np.array_equal(table.cpu().numpy(), np.asarray(host).reshape(-1))


@pytest.mark.parametrize("family", list(FAMILIES))
def test_forward_and_backward_with_prepared_descriptors(family):
    cfg = FAMILIES[family]
    x = inputs.make_inputs(cfg, 71, "cuda", doc_starts=DOCS[family])
    plain, prepared = _both(cfg, x["doc_starts"])
    args = (x["H"], x["X0"], x["W_gate"], x["W_up"], x["W_down"], x["conv_w"], x["W_target"], x["eta"], x["tau"])
    outs = []
    for p in (plain, prepared):
        buf = ip.allocate(p, "cuda", save=True)
        ip.forward(p, *args, buf)
        dO = torch.randn(buf.O.shape, generator=torch.Generator("cpu").manual_seed(5)).to(buf.O)
        g = ip.backward(p, buf, *args, dO)
        alpha_na = torch.empty_like(buf.alpha)
        ip.ipttt_chunk_delta_noalloc(p, buf.V, buf.Z, x["eta"], x["tau"], alpha_na)
        torch.cuda.synchronize()
        outs.append((buf, g, alpha_na))
    (b0, g0, a0), (b1, g1, a1) = outs
    for name in ("O", "Z", "V", "alpha"):
        assert torch.equal(getattr(b0, name), getattr(b1, name)), name
    assert torch.equal(a0, a1) and torch.equal(a0, b0.alpha)
    for name in ("dH", "dX0", "dW_gate", "dW_up", "dW_down", "dconv_w", "dW_target"):
        assert torch.equal(getattr(g0, name), getattr(g1, name)), name
    o = run_oracle(cfg, inputs.to_f64(x))
    r = rel(np64(b1.O), o["O"])
    print(f"  [{cfg.name}] prepared-descriptor O rel to the oracle {r:.2e}", flush=True)
    assert r <= tol(cfg)


@pytest.mark.parametrize("family", list(FAMILIES))
def test_streamed_call_with_prepared_descriptors(family):
    cfg = FAMILIES[family]
    x = inputs.make_inputs(cfg, 73, "cuda", doc_starts=DOCS[family])
    plain, prepared = _both(cfg, x["doc_starts"], continues=[1, 0])
    S_in = 1e-3 * torch.randn((cfg.rows, cfg.d_model, cfg.d_ff), generator=torch.Generator("cpu").manual_seed(9)
                              ).to("cuda")
    res = []
    for p in (plain, prepared):
        S_out = torch.empty_like(S_in)
        buf = ip.forward(p, x["H"], x["X0"], x["W_gate"], x["W_up"], x["W_down"], x["conv_w"], x["W_target"],
                         x["eta"], x["tau"], S_in=S_in, S_out=S_out)
        torch.cuda.synchronize()
        res.append((buf.O, S_out))
    assert torch.equal(res[0][0], res[1][0]) and torch.equal(res[0][1], res[1][1])


def test_prepared_descriptors_can_be_dropped():
    cfg = FAMILIES["fast_bf16"]
    p = _problem(cfg, DOCS["fast_bf16"]).prepare_segments()
    p.use_segments(None, None)
    assert p._c.seg_table is None and p._c.seg_bytes is None and ip.ipttt_validate(p) == 0
