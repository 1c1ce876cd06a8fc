"""GPU parity of the state carried across calls (ipttt_scan_apply_carry): one
long sequence read in pieces that are whole numbers of chunks, each call
taking the open document's fp32 state S in and handing the new one out.

  - one call against the oracle: O and S_out, rows that continue (from a
    random S_in) and rows that do not, documents inside the pieces;
  - pieces against one call over the whole sequence, bit for bit (O and the
    final S): the kernels do the same arithmetic in the same order either way;
  - S_out written in place over S_in;
  - at the full 4B workload size, in the launch configuration bench.py
    times: the two-piece reading bit for bit against one call, and S_out
    against the oracle where only two chunks carry a delta.
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
    # bf16 8-wave kernels (d, f multiples of 64); row 0 has a document that
    # spans the split at 1024, row 1 one that starts exactly there
    "bf16_fast": (C["4b_32k"].with_(name="bf16_fast", d_model=256, d_ff=384, rows=2, seq_len=1792,
                                    chunk=256, tau=2e-3, eta=1e-2), [300, 1792 + 1024, 1792 + 1500], 1024),
    # general kernels: bf16 widths that are not multiples of 64, and fp32
    "bf16_general": (C["4b_32k"].with_(name="bf16_general", d_model=136, d_ff=200, rows=2, seq_len=640,
                                       chunk=128, tau=2e-3, eta=1e-2), [333, 640 + 77], 256),
    "f32_general": (C["tiny_f32"].with_(name="f32_general", d_model=72, d_ff=136, rows=2, seq_len=288,
                                        chunk=48, tau=2e-2, eta=5e-2), [77, 288 + 5], 144),
}


def _problem(cfg, T, docs, continues=None):
    dt = ip.IPTTT_F32 if cfg.dtype == "f32" else ip.IPTTT_BF16
    return ip.Problem(cfg.rows, T, cfg.d_model, cfg.d_ff, cfg.chunk, dt, docs, continues=continues)


def _piece(x, cfg, lo, hi):
    """Tokens [lo, hi) of every row, contiguous."""
    out = dict(x)
    for k in ("H", "X0"):
        out[k] = x[k].view(cfg.rows, cfg.seq_len, -1)[:, lo:hi].reshape(cfg.rows * (hi - lo), -1).contiguous()
    return out


def _piece_starts(docs, T, lo, hi):
    return [(s // T) * (hi - lo) + (s % T - lo) for s in docs if lo <= s % T < hi]


def _run(cfg, x, T, docs, continues=None, S_in=None, S_out=None, W_down=None):
    p = _problem(cfg, T, docs, continues)
    buf = ip.allocate(p, "cuda")
    ip.forward(p, x["H"], x["X0"], x["W_gate"], x["W_up"], x["W_down"] if W_down is None else W_down,
               x["conv_w"], x["W_target"], x["eta"], x["tau"], buf, carry=True, S_in=S_in, S_out=S_out)
    torch.cuda.synchronize()
    return buf


def _state(cfg, scale, seed):
    g = torch.Generator(device="cuda").manual_seed(seed)
    return torch.randn((cfg.rows, cfg.d_model, cfg.d_ff), generator=g, device="cuda") * scale


@pytest.mark.parametrize("name", list(CASES))
def test_carry_call_against_oracle(name):
    """Three rows: row 0 continues a document up to its first start, row 1
    continues one through its whole length (so its S_out is S_in plus every
    delta), row 2 starts fresh.  O and the carried-out state against the
    oracle, with W_down and without it (where the fast-weight term is all
    there is)."""
    cfg, docs, _ = CASES[name]
    cfg = cfg.with_(rows=3)
    docs = [s for s in docs if s < cfg.seq_len]
    x = inputs.make_inputs(cfg, 11, "cuda", doc_starts=docs)
    x64 = inputs.to_f64(x)
    cont = [1, 1, 0]
    wscale = float(x["W_down"].float().abs().mean())
    S_in = _state(cfg, 0.02 * wscale, 5)
    for W_down in (x["W_down"], torch.zeros_like(x["W_down"])):
        print(f"[{name}] carry call, |W_down| = {float(W_down.float().abs().mean()):.3g}", flush=True)
        S_out = torch.full_like(S_in, float("nan"))
        buf = _run(cfg, x, cfg.seq_len, docs, cont, S_in, S_out, W_down)
        ref = oracle.forward(x64["H"], x64["X0"], x64["W_gate"], x64["W_up"], np64(W_down), x64["conv_w"],
                             x64["W_target"], rows=cfg.rows, T=cfg.seq_len, C=cfg.chunk, eta=x64["eta"],
                             tau=x64["tau"], doc_starts=x64["doc_starts"], continues=cont, S_in=np64(S_in),
                             want_state=True)
        assert rel(np64(buf.alpha), ref["alpha"]) <= tol(cfg)
        assert rel(np64(buf.O), ref["O"]) <= tol(cfg)
        assert rel(np64(S_out), ref["S"]) <= tol(cfg)
        # row 0's state did come in: the first tokens differ from a fresh start
        assert not np.allclose(np64(buf.O[:8]), oracle.forward(
            x64["H"][:cfg.chunk], x64["X0"][:cfg.chunk], x64["W_gate"], x64["W_up"], np64(W_down),
            x64["conv_w"], x64["W_target"], rows=1, T=cfg.chunk, C=cfg.chunk, eta=x64["eta"],
            tau=x64["tau"])["O"][:8], rtol=1e-3, atol=0)


@pytest.mark.parametrize("name", list(CASES))
def test_pieces_equal_one_call_bit_exact(name):
    """Two calls over [0, split) and [split, T) with the state carried between
    them give the O and final S of one call over [0, T), bit for bit."""
    cfg, docs, split = CASES[name]
    x = inputs.make_inputs(cfg, 12, "cuda", doc_starts=docs)
    T = cfg.seq_len
    print(f"[{name}] one call vs pieces at {split}", flush=True)
    S_one = torch.empty((cfg.rows, cfg.d_model, cfg.d_ff), device="cuda")
    one = _run(cfg, x, T, docs, None, None, S_one)
    a = _piece(x, cfg, 0, split)
    S = torch.empty_like(S_one)
    pa = _run(cfg, a, split, _piece_starts(docs, T, 0, split), None, None, S)
    bx = _piece(x, cfg, split, T)
    # in place: S_out is S_in
    pb = _run(cfg, bx, T - split, _piece_starts(docs, T, split, T), [1] * cfg.rows, S, S)
    O = torch.cat([pa.O.view(cfg.rows, split, -1), pb.O.view(cfg.rows, T - split, -1)], dim=1)
    assert torch.equal(O.reshape(cfg.rows * T, -1), one.O)
    assert torch.equal(S, S_one)
    alpha = torch.cat([pa.alpha, pb.alpha], dim=1)
    assert torch.equal(alpha, one.alpha)


@pytest.mark.parametrize("name", list(CASES))
def test_carry_without_state_matches_plain_call(name):
    """With no state in or out, the carry entry computes what
    ipttt_scan_apply does, up to the rounding of W_down + S (once, instead
    of accumulating into W_down)."""
    cfg, docs, _ = CASES[name]
    x = inputs.make_inputs(cfg, 13, "cuda", doc_starts=docs)
    print(f"[{name}] carry entry without state", flush=True)
    p = _problem(cfg, cfg.seq_len, docs)
    plain = ip.allocate(p, "cuda")
    ip.forward(p, x["H"], x["X0"], x["W_gate"], x["W_up"], x["W_down"], x["conv_w"], x["W_target"],
               x["eta"], x["tau"], plain)
    carry = _run(cfg, x, cfg.seq_len, docs)
    assert rel(np64(carry.O), np64(plain.O)) <= tol(cfg)


# ------------------------------------------------------------- full size

def test_pieces_equal_one_call_full_size():
    """4B workload (d 2560, f 9728, C 512), 32768 tokens read as two pieces of
    16384: bit for bit the O and final S of one call over the 32768."""
    cfg = C["4b_32k"]
    x = inputs.make_inputs(cfg, 14, "cuda")
    T, split = cfg.seq_len, cfg.seq_len // 2
    print("[4b_32k] one call vs two pieces", flush=True)
    S_one = torch.empty((cfg.rows, cfg.d_model, cfg.d_ff), device="cuda")
    one = _run(cfg, x, T, None, None, None, S_one)
    O_one = one.O.clone()
    del one
    S = torch.empty_like(S_one)
    pa = _run(cfg, _piece(x, cfg, 0, split), split, None, None, None, S)
    O_a = pa.O.clone()
    del pa
    pb = _run(cfg, _piece(x, cfg, split, T), T - split, None, [1], S, S)
    assert torch.equal(O_a, O_one[:split])
    assert torch.equal(pb.O, O_one[split:])
    assert torch.equal(S, S_one)
    assert torch.count_nonzero(S).item() > 0
    del pb, S, S_one, O_one, O_a
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def test_final_state_against_oracle_full_size():
    """4B workload, X0 zero outside chunks 1 and N-1: only those chunks carry a
    delta, so the final state of the row's one document is the sum of their
    two clipped deltas (the last chunk's included, which only the carried-out
    state receives).  The oracle runs on those two chunks alone, laid end to
    end: the chunks between them add nothing, and no delta depends on the
    state."""
    cfg = C["4b_32k"]
    N = cfg.n_chunks
    x = inputs.make_inputs(cfg, 15, "cuda")
    keep = [1, N - 1]
    X0 = x["X0"].view(cfg.seq_len, cfg.d_model)
    mask = torch.zeros(cfg.seq_len, dtype=torch.bool, device="cuda")
    for j in keep:
        mask[j * cfg.chunk:(j + 1) * cfg.chunk] = True
    X0[~mask] = 0
    print("[4b_32k] final state, chunks 1 and N-1", flush=True)
    S = torch.empty((cfg.rows, cfg.d_model, cfg.d_ff), device="cuda")
    buf = _run(cfg, x, cfg.seq_len, None, None, None, S)
    alpha = np64(buf.alpha)
    del buf
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    rows = torch.cat([torch.arange(j * cfg.chunk, (j + 1) * cfg.chunk) for j in keep]).cuda()
    ref = oracle.forward(np64(x["H"][rows]), np64(x["X0"][rows]), np64(x["W_gate"]), np64(x["W_up"]),
                         np64(x["W_down"]), np64(x["conv_w"]), np64(x["W_target"]), rows=1,
                         T=2 * cfg.chunk, C=cfg.chunk, eta=float(x["eta"]), tau=float(x["tau"]),
                         want_state=True)
    assert rel(np64(S[0]), ref["S"][0]) <= tol(cfg)
    for k, j in enumerate(keep):
        assert abs(alpha[0, j] - ref["alpha"][0, k]) <= tol(cfg) * ref["alpha"][0, k]
    assert np.all(alpha[0, [j for j in range(N) if j not in keep]] == 1.0)


def test_decode_token_by_token_equals_prefill_bit_exact():
    """Decode with the same entry point: every token applies the state of its
    document as it stands (a call over that one token, S_in = S, no S_out),
    and when a chunk is complete, one call over the chunk's tokens folds the
    chunk's clipped delta into S (S_out = S_in = S).  The outputs equal one
    prefill call over the whole sequence, bit for bit."""
    cfg = C["4b_32k"].with_(name="decode", d_model=256, d_ff=384, rows=1, seq_len=3 * 32 + 5, chunk=32,
                            tau=2e-3, eta=1e-2)
    x = inputs.make_inputs(cfg, 16, "cuda")
    T, Cn = cfg.seq_len, cfg.chunk
    print("[decode] 101 tokens, chunk 32", flush=True)
    S_ref = torch.empty((1, cfg.d_model, cfg.d_ff), device="cuda")
    ref = _run(cfg, x, T, None, None, None, S_ref)
    S = torch.zeros_like(S_ref)
    O = torch.empty_like(ref.O)
    for t in range(T):
        one = _piece(x, cfg, t, t + 1)
        cont = [0] if t == 0 else [1]
        O[t] = _run(cfg.with_(chunk=1), one, 1, None, cont, S, None).O[0]
        if (t + 1) % Cn == 0 or t + 1 == T:
            lo = (t // Cn) * Cn
            _run(cfg, _piece(x, cfg, lo, t + 1), t + 1 - lo, None, [0] if lo == 0 else [1], S, S)
    assert torch.equal(O, ref.O)
    assert torch.equal(S, S_ref)


@pytest.mark.parametrize("w_down", ["zero", "drawn"])
def test_decode_token_by_token_against_oracle(w_down):
    """Decode as above (one call per token applying S as it stands; one call
    per completed chunk folding its clipped delta into S), compared with the
    oracle's sequential loop directly: every output token, and the final
    state.  With W_down = 0 the outputs are the fast-weight term alone (chunk
    0 exactly zero); with the drawn W_down, the whole layer output."""
    cfg = C["4b_32k"].with_(name="decode", d_model=256, d_ff=384, rows=1, seq_len=3 * 32 + 5, chunk=32,
                            tau=2e-3, eta=1e-2)
    x = inputs.make_inputs(cfg, 17, "cuda")
    if w_down == "zero":
        x["W_down"] = torch.zeros_like(x["W_down"])
    T, Cn = cfg.seq_len, cfg.chunk
    print(f"[decode] 101 tokens, chunk 32, W_down {w_down}, against the oracle", flush=True)
    S = torch.zeros((1, cfg.d_model, cfg.d_ff), device="cuda")
    O = torch.empty((T, cfg.d_model), dtype=x["H"].dtype, device="cuda")
    for t in range(T):
        O[t] = _run(cfg.with_(chunk=1), _piece(x, cfg, t, t + 1), 1, None, [0] if t == 0 else [1], S, None).O[0]
        if (t + 1) % Cn == 0 or t + 1 == T:
            lo = (t // Cn) * Cn
            _run(cfg, _piece(x, cfg, lo, t + 1), t + 1 - lo, None, [0] if lo == 0 else [1], S, S)
    torch.cuda.synchronize()
    ref = oracle.forward(np64(x["H"]), np64(x["X0"]), np64(x["W_gate"]), np64(x["W_up"]), np64(x["W_down"]),
                         np64(x["conv_w"]), np64(x["W_target"]), rows=1, T=T, C=Cn, eta=x["eta"], tau=x["tau"],
                         want_state=True)
    got = np64(O)
    r, rs = rel(got, ref["O"]), rel(np64(S[0]), ref["S"][0])
    print(f"    O rel {r:.2e}, final state rel {rs:.2e}", flush=True)
    assert r <= tol(cfg)
    assert rs <= tol(cfg)
    if w_down == "zero":
        assert np.count_nonzero(got[:Cn]) == 0
