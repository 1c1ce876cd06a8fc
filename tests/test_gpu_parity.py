"""GPU parity: every call of the C ABI against the fp64 oracle on the same
seeded inputs, at sizes the oracle finishes in seconds that still span several
tiles and ragged edges (tokens, chunks, features, documents)."""
import numpy as np
import pytest
import torch

import oracle
import test_weight_mlp_amd as ip
from test_weight_mlp_amd import inputs
from gpu_helpers import np64, problem, rel, run_gpu, run_oracle, tol

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

C = inputs.CONFIGS
CASES = {
    # the tiny fp32 configuration exactly
    "tiny_f32": (C["tiny_f32"], None),
    # fp32, ragged everything: partial feature tiles, short last chunk, documents, clip
    "f32_ragged_docs_clip": (C["tiny_f32"].with_(name="f32_ragged", d_model=136, d_ff=200, rows=2,
                                                 seq_len=333, chunk=40, tau=2e-2, eta=5e-2),
                             [17, 80, 81, 200, 333 + 40, 333 + 150]),
    # the small bf16 distributions at reduced width, several chunks of 256
    "bf16_small_like": (C["small_bf16"].with_(name="bf16_small_like", d_model=256, d_ff=512, rows=2,
                                              seq_len=1100, chunk=256), None),
    # the 4B distributions (clip at 1e-5) at reduced width
    "bf16_4b_like_clip": (C["4b_32k"].with_(name="bf16_4b_like", d_model=256, d_ff=384,
                                            seq_len=2048), None),
    # the 8-wave kernels with a chunk that is not a whole number of their
    # 64-token stages, documents inside chunks
    "bf16_odd_chunk": (C["4b_32k"].with_(name="bf16_odd_chunk", d_model=192, d_ff=320, rows=2, seq_len=900,
                                         chunk=100, tau=1e-3, eta=1e-2), [130, 400, 900 + 250]),
    # bf16 on the general kernels (widths not multiples of 64), ragged tiles
    # and chunks, documents, clip
    "bf16_general": (C["4b_32k"].with_(name="bf16_general", d_model=136, d_ff=200, rows=2, seq_len=520,
                                       chunk=72, tau=1e-3, eta=1e-2), [50, 144, 520 + 300]),
    # packed documents, boundaries off the chunk grid
    "bf16_packed": (C["4b_packed"].with_(name="bf16_packed", d_model=128, d_ff=320, rows=3,
                                         seq_len=1500, chunk=128), "loguniform"),
}


def _inputs(name, seed=0):
    cfg, docs = CASES[name]
    if docs == "loguniform":
        docs = inputs.loguniform_doc_starts(cfg.rows, cfg.seq_len, cfg.chunk, seed + 99, lo=40,
                                            hi=1500)
    x = inputs.make_inputs(cfg, seed, "cuda", doc_starts=docs)
    return cfg, x, inputs.to_f64(x)


_cache = {}


def _both(name):
    if name not in _cache:
        cfg, x, x64 = _inputs(name)
        p, buf = run_gpu(cfg, x, want_dW=True)
        ref = run_oracle(cfg, x64, want_dW=True)
        _cache[name] = (cfg, x, x64, p, buf, ref)
    return _cache[name]


@pytest.mark.parametrize("name", list(CASES))
def test_z_parity(name):
    cfg, x, x64, p, buf, ref = _both(name)
    print(f"[{name}] Z", flush=True)
    assert rel(np64(buf.Z), ref["Z"]) <= tol(cfg)


@pytest.mark.parametrize("name", list(CASES))
def test_target_parity(name):
    cfg, x, x64, p, buf, ref = _both(name)
    assert rel(np64(buf.V), ref["V"]) <= tol(cfg)


@pytest.mark.parametrize("name", list(CASES))
def test_alpha_and_delta_parity(name):
    cfg, x, x64, p, buf, ref = _both(name)
    a = buf.alpha.cpu().double().numpy()
    if cfg.tau <= 0:
        assert np.all(a == 1.0)
    else:
        assert rel(a, ref["alpha"]) <= tol(cfg)
    dW = np64(buf.dW).reshape(ref["dW"].shape)
    assert rel(dW, ref["dW"]) <= tol(cfg)
    if cfg.tau > 0:
        # carried deltas that were clipped have norm tau
        n = np.linalg.norm(dW.reshape(dW.shape[0], dW.shape[1], -1), axis=2)
        clipped = ref["alpha"] < 1.0
        if clipped.any():
            assert np.max(np.abs(n[clipped] - cfg.tau)) <= tol(cfg) * cfg.tau


@pytest.mark.parametrize("name", list(CASES))
def test_output_parity(name):
    cfg, x, x64, p, buf, ref = _both(name)
    assert rel(np64(buf.O), ref["O"]) <= tol(cfg)


@pytest.mark.parametrize("name", list(CASES))
def test_zero_w_down_isolates_fast_weight_term(name):
    """With W_down = 0 the output is Z S_i^T alone, the only place where a
    clipped fast-weight term is visible; reset-state tokens give exactly 0."""
    cfg, x, x64, p, _, _ = _both(name)
    Wd0 = torch.zeros_like(x["W_down"])
    _, buf = run_gpu(cfg, x, W_down=Wd0)
    ref = run_oracle(cfg, x64, W_down=np.zeros_like(x64["W_down"]))
    O = np64(buf.O)
    assert rel(O, ref["O"]) <= tol(cfg)
    tbl = oracle.segment_table(cfg.rows, cfg.seq_len, cfg.chunk, x["doc_starts"])
    starts = oracle.row_starts(cfg.rows, cfg.seq_len, x["doc_starts"])
    for b in range(cfg.rows):
        doc = np.searchsorted(starts[b], np.arange(cfg.seq_len), side="right") - 1
        first_chunk = starts[b][doc] // cfg.chunk
        fresh = (np.arange(cfg.seq_len) // cfg.chunk) == first_chunk
        rows_ = O[b * cfg.seq_len:(b + 1) * cfg.seq_len]
        assert np.all(rows_[fresh] == 0.0)
        assert np.all(ref["O"][b * cfg.seq_len:(b + 1) * cfg.seq_len][fresh] == 0.0)
    assert tbl.shape[1] == p.n_chunks


@pytest.mark.parametrize("name", ["f32_ragged_docs_clip", "bf16_packed"])
def test_segments_device_bit_exact(name):
    cfg, x, x64, p, _, _ = _both(name)
    table = torch.empty((p.rows, p.n_chunks, 3), dtype=torch.int32, device="cuda")
    segs = torch.empty(p.tokens, dtype=torch.uint8, device="cuda")
    ip.ipttt_segments_device(p, table, segs)
    torch.cuda.synchronize()
    ref = oracle.segment_table(cfg.rows, cfg.seq_len, cfg.chunk, x["doc_starts"])
    assert np.array_equal(table.cpu().numpy(), ref.astype(np.int32))
    s = segs.cpu().numpy().astype(np.int64)
    starts = oracle.row_starts(cfg.rows, cfg.seq_len, x["doc_starts"])
    for b in range(cfg.rows):
        end = oracle.window_end(cfg.seq_len, cfg.chunk, starts[b])
        taps = np.minimum(5, end - np.arange(cfg.seq_len))
        flag = np.isin(np.arange(cfg.seq_len), starts[b])
        row = s[b * cfg.seq_len:(b + 1) * cfg.seq_len]
        assert np.array_equal(row & 7, taps)
        assert np.array_equal((row >> 7) == 1, flag)


def _check_segments(rows, T, C, starts, continues):
    p = ip.Problem(rows, T, 64, 64, C, ip.IPTTT_BF16, np.asarray(starts, np.int64), continues=continues)
    table = torch.empty((rows, p.n_chunks, 3), dtype=torch.int32, device="cuda")
    segs = torch.empty(rows * T, dtype=torch.uint8, device="cuda")
    ip.ipttt_segments_device(p, table, segs)
    torch.cuda.synchronize()
    ref = oracle.segment_table(rows, T, C, list(starts), continues=continues)
    assert np.array_equal(table.cpu().numpy(), ref.astype(np.int32))
    s = segs.cpu().numpy().astype(np.int64)
    rs = oracle.row_starts(rows, T, list(starts), continues=continues)
    for b in range(rows):
        end = oracle.window_end(T, C, rs[b])
        row = s[b * T:(b + 1) * T]
        assert np.array_equal(row & 7, np.minimum(5, end - np.arange(T)))
        assert np.array_equal((row >> 7) == 1, np.isin(np.arange(T), rs[b]))


@pytest.mark.parametrize("case", ["one_launch", "batched"])
def test_segments_device_both_builders_bit_exact(case):
    """The descriptors come from one kernel when the listed tokens (document
    starts and continuing rows) fit in one kernel-argument batch of 384, and
    from the init / mark / finish kernels otherwise; both must equal the
    oracle's table, conv tap counts and start flags, with continuing rows
    (one of them also listing a start at its first token), starts at chunk
    edges and on adjacent tokens."""
    rows, T, C = 3, 3000, 256
    rng = np.random.default_rng(7)
    cont = [0, 1, 1]
    edge = [5, 256, 257, 511, 512, 2999, T, 2 * T + 1000, 2 * T + 1001]
    if case == "one_launch":
        starts = sorted(set(edge + list(rng.integers(0, rows * T, 40))))
    else:
        starts = sorted(set(edge + list(rng.integers(0, rows * T, 900))))
        assert len(starts) > 384
    _check_segments(rows, T, C, starts, cont)


def test_deterministic_bitwise():
    cfg, x, _, _, buf, _ = _both("bf16_packed")
    _, again = run_gpu(cfg, x)
    assert torch.equal(again.O, buf.O)
    assert torch.equal(again.alpha, buf.alpha)


def test_documents_independent_bitwise_on_gpu():
    """Changing one document's tokens leaves every other document's outputs
    bit-identical (reset at document boundaries)."""
    cfg, x, _, p, buf, _ = _both("bf16_packed")
    s = [0] + list(x["doc_starts"][x["doc_starts"] < cfg.seq_len]) + [cfg.seq_len]
    lo, hi = int(s[1]), int(s[2])  # the second document of row 0
    y = dict(x)
    for k in ("H", "X0"):
        y[k] = x[k].clone()
        y[k][lo:hi] = torch.randn_like(y[k][lo:hi].float()).to(y[k].dtype)
    _, b2 = run_gpu(cfg, y)
    assert not torch.equal(b2.O[lo:hi], buf.O[lo:hi])
    assert torch.equal(b2.O[:lo], buf.O[:lo])
    assert torch.equal(b2.O[hi:], buf.O[hi:])


def test_eta_zero_equals_zero_conv_bitwise():
    """Both make the fast weight stay at W_down: the two runs agree bit for bit
    and match the plain gated MLP."""
    cfg, x, x64, _, _, _ = _both("bf16_small_like")
    a = dict(x, eta=0.0)
    b = dict(x, conv_w=torch.zeros_like(x["conv_w"]))
    _, ba = run_gpu(cfg, a)
    _, bb = run_gpu(cfg, b)
    assert torch.equal(ba.O, bb.O)
    ref = oracle.plain_mlp(x64["H"], x64["W_gate"], x64["W_up"], x64["W_down"])
    assert rel(np64(ba.O), ref) <= tol(cfg)
