"""GPU parity over whole rows: every chunk of a long row carries a delta, and
every output row is compared with the oracle's sequential loop.

The state a chunk applies is the exclusive prefix sum of the clipped deltas
of its document's earlier chunks (lijianxiong.blog "In-Place Test-Time
Training", 工程实现), restarted at every document start (iplexlaw.co.kr
review, section 6).  At the 4B shapes the fast-weight term Z S_i^T is far
below bf16 resolution next to Z W_down^T, so those runs set W_down = 0 and O
is the fast-weight term alone; a narrow long row (the 8-wave kernels, 64
chunks) also runs the backward with the output cotangent on the last two
chunks only, so that the reverse scan carries adjoints through every chunk.

The oracle runs a whole row here: about 15 s of host time at 4B/32k, and
about as much for the four rows of the small bf16 configuration.
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


def _free():
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _weights64(x):
    return {k: np64(x[k]) for k in ("W_gate", "W_up", "W_down", "W_target", "conv_w")}


def _per_chunk(got, ref, T, C):
    """Frobenius-relative error of each chunk of one row (chunks whose
    reference is exactly zero: the largest absolute value instead)."""
    out = []
    for i in range(-(-T // C)):
        g, r = got[i * C:(i + 1) * C], ref[i * C:(i + 1) * C]
        nr = np.linalg.norm(r)
        out.append(np.linalg.norm(g - r) / nr if nr > 0 else float(np.abs(g).max()))
    return np.asarray(out)


def _forward_row(cfg, x, b, ds, W_down):
    """Run the GPU forward over all rows, return row b's O and alpha, and the
    oracle's sequential loop over that row alone (rows are independent)."""
    p = problem(cfg, ds)
    buf = ip.allocate(p, "cuda")
    ip.forward(p, x["H"], x["X0"], x["W_gate"], x["W_up"], W_down, x["conv_w"], x["W_target"],
               x["eta"], x["tau"], buf)
    torch.cuda.synchronize()
    T = cfg.seq_len
    O = np64(buf.O[b * T:(b + 1) * T])
    alpha = np64(buf.alpha[b])
    del buf
    _free()
    sub = [int(s) - b * T for s in ds if b * T <= s < (b + 1) * T] if ds is not None and len(ds) else None
    w = _weights64(x)
    sl = slice(b * T, (b + 1) * T)
    print(f"    oracle over row {b}: {T} tokens, {len(sub or [])} document starts", flush=True)
    ref = oracle.forward(np64(x["H"][sl]), np64(x["X0"][sl]), w["W_gate"], w["W_up"], np64(W_down),
                         w["conv_w"], w["W_target"], rows=1, T=T, C=cfg.chunk, eta=x["eta"], tau=x["tau"],
                         doc_starts=sub)
    return O, alpha, ref, sub


def _check_row(cfg, O, alpha, ref, sub):
    T, C = cfg.seq_len, cfg.chunk
    pc = _per_chunk(O, ref["O"], T, C)
    # tokens on the reset state output exactly zero (W_down = 0): chunk 0 and,
    # in a chunk with a document start, every token from the first one on
    starts = np.asarray(sorted(set(sub or [])), np.int64)
    reset = np.zeros(T, bool)
    reset[:C] = True
    for i in range(1, -(-T // C)):
        inside = starts[(starts >= i * C) & (starts < min((i + 1) * C, T))]
        if len(inside):
            reset[inside[0]:min((i + 1) * C, T)] = True
    assert np.count_nonzero(O[reset]) == 0
    assert np.count_nonzero(ref["O"][reset]) == 0
    live = [i for i in range(len(pc)) if np.linalg.norm(ref["O"][i * C:(i + 1) * C]) > 0]
    worst = max(live, key=lambda i: pc[i])
    r = rel(O, ref["O"])
    ra = rel(alpha, ref["alpha"][0])
    print(f"    O rel {r:.2e} over the row; per chunk max {pc[worst]:.2e} (chunk {worst}), "
          f"median {np.median(pc[live]):.2e}; alpha rel {ra:.2e}", flush=True)
    assert r <= tol(cfg)
    assert pc[worst] <= tol(cfg)
    assert ra <= tol(cfg)


def test_whole_row_4b_32k_every_chunk_carries_a_delta():
    """4B/32k (d 2560, f 9728, C 512, clip 1e-5) with the bench's inputs and
    W_down = 0: all 32768 output rows and all 64 clip scales against the
    oracle, each chunk within the bound on its own."""
    cfg = inputs.CONFIGS["4b_32k"]
    x = inputs.make_inputs(cfg, 0, "cuda")
    print("[4b_32k] whole row, W_down = 0", flush=True)
    O, alpha, ref, sub = _forward_row(cfg, x, 0, x["doc_starts"], torch.zeros_like(x["W_down"]))
    _check_row(cfg, O, alpha, ref, sub)


def test_whole_packed_row_4b_every_chunk_carries_a_delta():
    """8 x 32768 packed documents at full width (the bench's 4b_packed
    launch, documents off the chunk grid), W_down = 0: the row with the most
    document starts against the oracle over that row."""
    cfg = inputs.CONFIGS["4b_packed"]
    x = inputs.make_inputs(cfg, 0, "cuda")
    ds = x["doc_starts"]
    T = cfg.seq_len
    counts = [int(np.count_nonzero((ds >= b * T) & (ds < (b + 1) * T))) for b in range(cfg.rows)]
    b = int(np.argmax(counts))
    print(f"[4b_packed] whole row {b} of 8, W_down = 0", flush=True)
    O, alpha, ref, sub = _forward_row(cfg, x, b, ds, torch.zeros_like(x["W_down"]))
    assert len(sub) >= 2
    _check_row(cfg, O, alpha, ref, sub)


def test_whole_rows_small_bf16_every_chunk_carries_a_delta():
    """The small bf16 configuration at full size (d 1024, f 4096, 4 rows of
    8192 tokens, C 512, no clip) with W_down = 0: every output row of all
    four rows against the oracle's loop over each row, each chunk within the
    bound on its own."""
    cfg = inputs.CONFIGS["small_bf16"]
    x = inputs.make_inputs(cfg, 0, "cuda")
    zero = torch.zeros_like(x["W_down"])
    for b in range(cfg.rows):
        print(f"[small_bf16] whole row {b} of {cfg.rows}, W_down = 0", flush=True)
        O, alpha, ref, sub = _forward_row(cfg, x, b, x["doc_starts"], zero)
        _check_row(cfg, O, alpha, ref, sub)


NARROW = inputs.CONFIGS["4b_32k"].with_(name="narrow_32k", d_model=256, d_ff=384)


def _narrow(docs, tau, seed):
    cfg = NARROW.with_(tau=tau)
    ds = inputs.loguniform_doc_starts(1, cfg.seq_len, cfg.chunk, seed + 5) if docs == "packed" else None
    return cfg, inputs.make_inputs(cfg, seed, "cuda", doc_starts=ds)


@pytest.mark.parametrize("tau", [1e-5, 0.0])
@pytest.mark.parametrize("docs", ["one", "packed"])
def test_whole_narrow_row_64_chunks(docs, tau):
    """d 256, f 384, 32768 tokens, C 512 (64 chunks) on the 8-wave kernels,
    W_down = 0: every output row and clip scale against the oracle."""
    cfg, x = _narrow(docs, tau, 40)
    print(f"[narrow 32k] {docs} documents, tau {tau}, W_down = 0", flush=True)
    O, alpha, ref, sub = _forward_row(cfg, x, 0, x["doc_starts"], torch.zeros_like(x["W_down"]))
    _check_row(cfg, O, alpha, ref, sub)


@pytest.mark.parametrize("docs,tau", [("one", 1e-5), ("packed", 0.0), ("packed", 1e-5)])
def test_whole_narrow_row_backward_from_the_last_two_chunks(docs, tau):
    """The backward (forward with saved state, then the three backward calls)
    of the narrow 64-chunk row with dO nonzero on the last two chunks only:
    chunk 62 applies the deltas of every earlier chunk of its document, so
    their adjoints run back through the whole row.  Every gradient against
    the oracle's backward over the row."""
    cfg, x = _narrow(docs, tau, 41)
    T, C = cfg.seq_len, cfg.chunk
    dO = inputs.make_cotangents(cfg, 41, "cuda")["dO"]
    dO[:T - 2 * C] = 0
    ds = [int(s) for s in x["doc_starts"]]
    print(f"[narrow 32k] backward, {docs} documents, tau {tau}, dO on chunks 62-63", flush=True)
    p = problem(cfg, ds)
    buf = ip.allocate(p, "cuda", save=True)
    ip.forward(p, x["H"], x["X0"], x["W_gate"], x["W_up"], x["W_down"], x["conv_w"], x["W_target"], x["eta"],
               x["tau"], buf)
    g = ip.backward(p, buf, x["H"], x["X0"], x["W_gate"], x["W_up"], x["W_down"], x["conv_w"], x["W_target"],
                    x["eta"], x["tau"], dO)
    torch.cuda.synchronize()
    names = ("dH", "dX0", "dW_gate", "dW_up", "dW_down", "dconv_w", "dW_target")
    got = {k: np64(getattr(g, k)) for k in names}
    del buf, g
    _free()
    w = _weights64(x)
    ref = oracle.backward(np64(x["H"]), np64(x["X0"]), w["W_gate"], w["W_up"], w["W_down"], w["conv_w"],
                          w["W_target"], np64(dO), rows=1, T=T, C=C, eta=x["eta"], tau=x["tau"],
                          doc_starts=ds or None)
    # the adjoints reach the first chunk of the last chunks' document
    first = max([s for s in ds if s < T - 2 * C], default=0)
    first_chunk = first // C
    assert np.linalg.norm(ref["dH"][first_chunk * C:(first_chunk + 1) * C]) > 0
    for k in names:
        r = rel(got[k], ref[k])
        print(f"    {k}: rel {r:.2e}", flush=True)
        assert r <= tol(cfg), k
    # dH per chunk, over the chunks the gradient reaches (reported)
    pc = _per_chunk(got["dH"], ref["dH"], T, C)
    live = [i for i in range(len(pc)) if np.linalg.norm(ref["dH"][i * C:(i + 1) * C]) > 0]
    print(f"    dH per chunk: max {max(pc[live]):.2e}, median {np.median(pc[live]):.2e} over {len(live)} chunks",
          flush=True)
