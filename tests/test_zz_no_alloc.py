"""ipttt_chunk_delta_noalloc, the allocation-free variant of ipttt_chunk_delta
(its scratch in a static device array), against ipttt_chunk_delta through
the C ABI: two calls in a row, the second on a smaller problem, each
compared bit for bit (the same kernels produce both), plus the rejection of
a problem whose scratch exceeds the array, before anything is launched."""
import ctypes

import numpy as np
import pytest
import torch

import test_weight_mlp_amd as ip
from test_weight_mlp_amd import inputs

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def _case(cfg, seed, docs):
    x = inputs.make_inputs(cfg, seed, "cuda", doc_starts=docs)
    dt = ip.IPTTT_F32 if cfg.dtype == "f32" else ip.IPTTT_BF16
    p = ip.Problem(cfg.rows, cfg.seq_len, cfg.d_model, cfg.d_ff, cfg.chunk, dt, x["doc_starts"])
    buf = ip.allocate(p, "cuda")
    ip.ipttt_z(p, x["H"], x["W_gate"], x["W_up"], buf.Z)
    ip.ipttt_target(p, x["X0"], x["conv_w"], x["W_target"], buf.V, buf.ws)
    return x, p, buf


def _both(x, p, buf, tau):
    ref = torch.full_like(buf.alpha, -1.0)
    got = torch.full_like(buf.alpha, -2.0)
    ip.ipttt_chunk_delta(p, buf.V, buf.Z, x["eta"], tau, ref, None, buf.ws)
    ip.ipttt_chunk_delta_noalloc(p, buf.V, buf.Z, x["eta"], tau, got)
    torch.cuda.synchronize()
    return ref, got


@pytest.mark.parametrize("tau", [1e-5, 2e-3])
def test_noalloc_equals_workspace_call_twice_in_a_row(tau):
    C = inputs.CONFIGS
    big = C["4b_packed"].with_(name="big", d_model=256, d_ff=384, rows=4, seq_len=4096, chunk=512)
    small = C["4b_32k"].with_(name="small", d_model=128, d_ff=192, rows=1, seq_len=700, chunk=128)
    starts = {"big": inputs.loguniform_doc_starts(4, 4096, 512, 3), "small": np.array([77, 300], np.int64)}
    print(f"[noalloc] tau {tau}: 4 x 4096 tokens (d 256, f 384, C 512), then 1 x 700 (d 128, f 192, C 128)",
          flush=True)
    for cfg in (big, small):
        x, p, buf = _case(cfg, 9, starts[cfg.name])
        ref, got = _both(x, p, buf, tau)
        assert torch.all(ref >= 0) and torch.all(ref <= 1)
        assert torch.equal(got, ref), cfg.name
        if tau == 1e-5:
            assert torch.all(ref < 1)   # every chunk clipped at the pages' threshold


def test_noalloc_rejects_a_problem_beyond_its_scratch_before_any_launch():
    lib = ip.library()
    v = ctypes.c_void_p
    # per-token segment bytes alone exceed the array
    p = ip.Problem(1, ip.IPTTT_NOALLOC_SCRATCH_BYTES + 1, 64, 128, 512, ip.IPTTT_BF16)
    alpha = torch.full((1,), 7.0, device="cuda")
    assert lib.ipttt_chunk_delta_noalloc(p.ref, v(256), v(256), 1e-3, 1e-5, v(alpha.data_ptr()), None) == 9
    torch.cuda.synchronize()
    assert alpha.item() == 7.0
    assert "static scratch" in lib.ipttt_status_string(9).decode()
