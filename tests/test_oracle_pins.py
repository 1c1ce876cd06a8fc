"""Pins of the fp64 oracle against what the pages and the mathematics fix.

None of these checks re-types the oracle's formula: each compares it with a
library routine, a closed form, an invariant, a hand-derived table or brute
force.  Sources are cited by page and section (see the oracle's header for the
page list).
"""
import json
import os

import numpy as np
import pytest
import scipy.special
import torch

import oracle

RNG = np.random.default_rng(1234)


def _problem(rows=1, T=48, C=8, d=6, f=10, seed=0, conv_std=0.3):
    r = np.random.default_rng(seed)
    n = rows * T
    return dict(
        H=r.standard_normal((n, d)),
        X0=r.standard_normal((n, d)),
        W_gate=r.standard_normal((f, d)) / np.sqrt(d),
        W_up=r.standard_normal((f, d)) / np.sqrt(d),
        W_down=r.standard_normal((d, f)) / np.sqrt(f),
        conv_w=r.standard_normal((d, 5)) * conv_std,
        W_target=r.standard_normal((d, d)) / np.sqrt(d),
    )


def _fwd(p, **kw):
    return oracle.forward(p["H"], p["X0"], p["W_gate"], p["W_up"], p["W_down"], p["conv_w"],
                          p["W_target"], **kw)


def _torch_gated_mlp(p):
    """Gated MLP built from torch library ops in fp64 ([JX] 方法 > 原地自适应)."""
    H = torch.from_numpy(p["H"])
    g = torch.nn.functional.linear(H, torch.from_numpy(p["W_gate"]))
    u = torch.nn.functional.linear(H, torch.from_numpy(p["W_up"]))
    return torch.nn.functional.linear(torch.nn.functional.silu(g) * u,
                                      torch.from_numpy(p["W_down"])).numpy()


def _rel(a, b):
    return np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300)


# ---------------------------------------------------------------- activation

def test_silu_matches_library_and_is_finite():
    x = np.concatenate([RNG.standard_normal(1000) * 10, [-800.0, -60.0, 0.0, 60.0, 800.0]])
    ref = x * scipy.special.expit(x)
    got = oracle.silu(x)
    assert np.all(np.isfinite(got))
    np.testing.assert_allclose(got, ref, rtol=1e-14, atol=1e-300)


def test_intermediate_matches_torch_swiglu():
    p = _problem(T=16, d=7, f=9)
    H = torch.from_numpy(p["H"])
    ref = (torch.nn.functional.silu(H @ torch.from_numpy(p["W_gate"]).T)
           * (H @ torch.from_numpy(p["W_up"]).T)).numpy()
    assert _rel(oracle.intermediate(p["H"], p["W_gate"], p["W_up"]), ref) < 1e-14


# ----------------------------------------------------- P1, P2, P3: reductions

def test_plain_mlp_matches_torch_and_a_hand_derived_value():
    """oracle.plain_mlp, the reference of the GPU's eta = 0 and reset-token
    checks, against torch's gated MLP (F.linear and F.silu, fp64) on random
    weights, and against one value worked out by hand ([JX] 方法 > 原地自适应:
    O = (phi(H W_gate^T) * (H W_up^T)) W_down^T).  With H = 2, W_gate = ln(3)/2,
    W_up = 3/2 and W_down = 2 (d = f = 1): g = ln 3, sigmoid(ln 3) = 3/4, so
    Z = (3/4 ln 3) * 3 and O = 4.5 ln 3.  A dropped activation, a swapped
    gate and up, or a transposed weight fails one of the two."""
    p = _problem(T=40, d=6, f=10, seed=11)
    got = oracle.plain_mlp(p["H"], p["W_gate"], p["W_up"], p["W_down"])
    assert _rel(got, _torch_gated_mlp(p)) < 1e-14
    o = oracle.plain_mlp(np.array([[2.0]]), np.array([[np.log(3.0) / 2]]), np.array([[1.5]]), np.array([[2.0]]))
    assert abs(o[0, 0] - 4.5 * np.log(3.0)) < 1e-14
    # f != d with asymmetric weights: gate and up must not be interchangeable
    q = _problem(T=8, d=3, f=5, seed=12)
    swapped = oracle.plain_mlp(q["H"], q["W_up"], q["W_gate"], q["W_down"])
    assert _rel(swapped, oracle.plain_mlp(q["H"], q["W_gate"], q["W_up"], q["W_down"])) > 1e-3


@pytest.mark.parametrize("docs", [[], [13, 29]])
def test_p1_eta_zero_is_plain_gated_mlp(docs):
    """eta = 0: the fast weight never moves, the layer is the gated MLP."""
    p = _problem()
    out = _fwd(p, rows=1, T=48, C=8, eta=0.0, tau=0.0, doc_starts=docs)
    assert _rel(out["O"], _torch_gated_mlp(p)) < 1e-13


@pytest.mark.parametrize("C", [48, 64, 1000])
def test_p2_single_chunk_is_plain_gated_mlp(C):
    """C >= T: one chunk, applied with W_down before any update ([JX] 步骤一)."""
    p = _problem()
    out = _fwd(p, rows=1, T=48, C=C, eta=0.5, tau=0.0)
    assert _rel(out["O"], _torch_gated_mlp(p)) < 1e-13


def test_p3_zero_conv_gives_zero_target_and_plain_mlp():
    """Zero conv (the near-zero init of [TC] 验证模块一) makes V_hat = 0, so the
    update is zero and the model equals the original MLP for any eta."""
    p = _problem()
    p["conv_w"] = np.zeros_like(p["conv_w"])
    out = _fwd(p, rows=1, T=48, C=8, eta=3.0, tau=0.0, doc_starts=[20])
    assert np.all(out["V"] == 0.0)
    assert _rel(out["O"], _torch_gated_mlp(p)) < 1e-13


# ------------------------------------- P4: three independent forms agree

def _dual_form(p, V, Z, alpha, rows, T, C, eta, doc_starts):
    """O = Z W_down^T + eta (M * Z Z^T)(a * V_hat), written from the unrolled
    sum ([JX] 工程实现) expanded token by token as in Theorem 1's logit change
    ([JX] 理论分析): M[t,s] = 1 when s is in an earlier chunk of t's document,
    a[s] = clip scale of s's segment."""
    O = np.zeros((rows * T, p["W_down"].shape[0]))
    for b in range(rows):
        starts = np.union1d([0], [s - b * T for s in doc_starts if b * T <= s < (b + 1) * T])
        doc = np.searchsorted(starts, np.arange(T), side="right") - 1
        chunk = np.arange(T) // C
        M = (doc[:, None] == doc[None, :]) & (chunk[None, :] < chunk[:, None])
        a = alpha[b]
        sl = slice(b * T, (b + 1) * T)
        Zb, Vb = Z[sl], V[sl]
        O[sl] = Zb @ p["W_down"].T + eta * ((M * (Zb @ Zb.T)) @ (a[:, None] * Vb))
    return O


@pytest.mark.parametrize("T,C,docs,tau", [
    (48, 8, [], 0.0),
    (50, 8, [], 0.0),            # ragged last chunk
    (48, 8, [13, 29, 30], 0.0),  # documents cut chunks
    (96, 16, [40, 97, 130], 0.0),  # two rows
    (48, 8, [13, 29], 0.05),     # clip active in some segments
])
def test_p4_sequential_equals_prefix_scan_equals_dual(T, C, docs, tau):
    rows = 2 if T == 96 else 1
    Tr = 48 if rows == 2 else T
    p = _problem(rows=rows, T=Tr, C=C, seed=T + C)
    eta = 0.3
    out = _fwd(p, rows=rows, T=Tr, C=C, eta=eta, tau=tau, doc_starts=docs)
    O_scan = oracle.forward_prefix_scan(out["Z"], out["V"], p["W_down"], rows=rows, T=Tr, C=C,
                                        eta=eta, tau=tau, doc_starts=docs)
    assert _rel(O_scan, out["O"]) < 1e-12
    # Per-token clip scale for the dual form: recompute each segment's scale
    # from scratch with numpy's norm.
    N = -(-Tr // C)
    a = np.ones((rows, Tr))
    for b in range(rows):
        starts = np.union1d([0], [s - b * Tr for s in docs if b * Tr <= s < (b + 1) * Tr])
        doc = np.searchsorted(starts, np.arange(Tr), side="right") - 1
        for i in range(N):
            lo, hi = i * C, min((i + 1) * C, Tr)
            for dc in np.unique(doc[lo:hi]):
                idx = lo + np.nonzero(doc[lo:hi] == dc)[0]
                g = b * Tr + idx
                n = eta * np.linalg.norm(out["V"][g].T @ out["Z"][g], "fro")
                a[b, idx] = tau / n if (tau > 0 and n > tau) else 1.0
    O_dual = _dual_form(p, out["V"], out["Z"], a, rows, Tr, C, eta, docs)
    assert _rel(O_dual, out["O"]) < 1e-12
    if tau > 0:
        assert np.any(a < 1.0), "the clip case must clip something"


# --------------------------------------------- P5, P6, P10: the update rule

def test_p5_delta_linear_in_eta_bit_exact():
    p = _problem()
    a = _fwd(p, rows=1, T=48, C=8, eta=0.125, tau=0.0, want_dW=True)["dW"]
    b = _fwd(p, rows=1, T=48, C=8, eta=0.25, tau=0.0, want_dW=True)["dW"]
    assert np.array_equal(b, 2.0 * a)


def test_p6_delta_is_negative_gradient_of_inner_product_loss():
    """Update W <- W - eta grad_W L with L = -<Z W^T, V_hat>_F
    ([JX] 步骤二 and 对齐语言模型的目标函数): checked with torch autograd."""
    p = _problem()
    eta = 0.7
    out = _fwd(p, rows=1, T=48, C=8, eta=eta, tau=0.0, want_dW=True)
    for i in (0, 3, 5):
        Zc = torch.from_numpy(out["Z"][i * 8:(i + 1) * 8])
        Vc = torch.from_numpy(out["V"][i * 8:(i + 1) * 8])
        W = torch.from_numpy(p["W_down"].copy()).requires_grad_(True)
        loss = -(Zc @ W.T * Vc).sum()
        loss.backward()
        assert _rel(out["dW"][0, i], (-eta * W.grad).numpy()) < 1e-14


def test_p10_clip_sets_norm_to_tau_or_leaves_delta_untouched():
    p = _problem()
    eta = 0.3
    raw = _fwd(p, rows=1, T=48, C=8, eta=eta, tau=0.0, want_dW=True)
    norms = np.linalg.norm(raw["dW"][0].reshape(6, -1), axis=1)
    tau = float(np.median(norms))
    clip = _fwd(p, rows=1, T=48, C=8, eta=eta, tau=tau, want_dW=True)
    for i in range(6):
        if norms[i] > tau:
            assert abs(np.linalg.norm(clip["dW"][0, i]) - tau) < 1e-14 * tau
            assert clip["alpha"][0, i] < 1.0
        else:
            assert np.array_equal(clip["dW"][0, i], raw["dW"][0, i])
            assert clip["alpha"][0, i] == 1.0


# --------------------------------------------------- P7, P8, P11: structure

def test_p7_documents_are_independent_bit_exact():
    """Reset at document boundaries: no information crosses documents
    ([IP] §6, §8; [AD] 四)."""
    T, C, cut = 48, 8, 19
    p = _problem(seed=5)
    base = _fwd(p, rows=1, T=T, C=C, eta=0.4, tau=0.0, doc_starts=[cut])["O"]
    q = {k: v.copy() for k, v in p.items()}
    q["H"][:cut] += RNG.standard_normal(q["H"][:cut].shape)
    q["X0"][:cut] += RNG.standard_normal(q["X0"][:cut].shape)
    pert = _fwd(q, rows=1, T=T, C=C, eta=0.4, tau=0.0, doc_starts=[cut])["O"]
    assert np.array_equal(base[cut:], pert[cut:])
    assert not np.allclose(base[:cut], pert[:cut])
    # The same document B behind other documents (a different split of the
    # tokens before it) at the same row offset reproduces B's outputs.
    r = {k: v.copy() for k, v in p.items()}
    r["H"][:cut] = RNG.standard_normal(r["H"][:cut].shape)
    r["X0"][:cut] = RNG.standard_normal(r["X0"][:cut].shape)
    other = _fwd(r, rows=1, T=T, C=C, eta=0.4, tau=0.0, doc_starts=[7, cut])["O"]
    assert np.array_equal(base[cut:], other[cut:])


def _dependence(p, T, C, docs, which):
    base = _fwd(p, rows=1, T=T, C=C, eta=0.5, tau=0.0, doc_starts=docs)["O"]
    dep = np.zeros((T, T), dtype=bool)  # dep[t, s]: O[t] moves when input s moves
    for s in range(T):
        q = {k: v.copy() for k, v in p.items()}
        q[which][s] += 1.0
        o = _fwd(q, rows=1, T=T, C=C, eta=0.5, tau=0.0, doc_starts=docs)["O"]
        dep[:, s] = np.any(o != base, axis=1)
    return dep


@pytest.mark.parametrize("which", ["H", "X0"])
def test_p8_brute_force_dependence_pattern(which):
    """O[t] depends on H[s] iff s == t or s lies in an earlier chunk of t's
    document; on X0[s] only through earlier chunks of the same document:
    apply before update ([IP] §3), exclusive prefix ([IP] §6), edge padding
    ([AD] 七), reset ([IP] §6)."""
    T, C, docs = 22, 5, [8, 17]
    p = _problem(T=T, d=4, f=6, seed=11)
    dep = _dependence(p, T, C, docs, which)
    starts = np.array([0] + docs)
    doc = np.searchsorted(starts, np.arange(T), side="right") - 1
    ch = np.arange(T) // C
    exp = (doc[:, None] == doc[None, :]) & (ch[None, :] < ch[:, None])
    if which == "H":
        exp |= np.eye(T, dtype=bool)
    assert np.array_equal(dep, exp)


def test_p11_zero_w_down_zero_output_on_reset_tokens():
    """With W_down = 0, O = Z S_i^T: tokens that still hold the reset state
    (chunk 0 of each document, and tokens after a start in their chunk) give
    exactly 0; tokens with history do not."""
    T, C, docs = 40, 8, [13, 30]
    p = _problem(T=T, seed=3)
    p["W_down"] = np.zeros_like(p["W_down"])
    O = _fwd(p, rows=1, T=T, C=C, eta=0.5, tau=0.0, doc_starts=docs)["O"]
    starts = np.array([0] + docs)
    doc = np.searchsorted(starts, np.arange(T), side="right") - 1
    first_chunk_of_doc = np.array([starts[dc] // C for dc in doc])
    fresh = (np.arange(T) // C) == first_chunk_of_doc
    assert np.all(O[fresh] == 0.0)
    assert np.all(np.any(O[~fresh] != 0.0, axis=1))


# ------------------------------------------------------------ P12: targets

@pytest.mark.parametrize("tap", [0, 1, 3])
def test_p12_one_hot_tap_shifts_embeddings_with_edge_zeros(tap):
    """Conv tap k multiplies X0[t+k]; zero where t+k reaches the chunk end or
    the next document ([TC] 详细步骤 3; [IP] §6)."""
    T, C, docs, d = 30, 8, [11, 20], 5
    r = np.random.default_rng(2)
    X0 = r.standard_normal((T, d))
    w = np.zeros((d, 5))
    w[:, tap] = 1.0
    V = oracle.lm_target(X0, w, np.eye(d), 1, T, C, docs)
    starts = [0] + docs
    for t in range(T):
        nxt = min([s for s in starts if s > t] + [T])
        end = min((t // C + 1) * C, nxt)
        if t + tap < end:
            assert np.array_equal(V[t], X0[t + tap])
        else:
            assert np.all(V[t] == 0.0)


def test_target_projection_orientation():
    """V_hat = Conv1D(X0) W_target: W_target multiplies from the right
    ([JX] 对齐语言模型的目标函数), so with tap 0 V_hat[t] = sum_c X0[t,c] W_target[c,:]."""
    r = np.random.default_rng(9)
    X0 = r.standard_normal((8, 3))
    Wt = r.standard_normal((3, 3))
    w = np.zeros((3, 5))
    w[:, 0] = 1.0
    V = oracle.lm_target(X0, w, Wt, 1, 8, 8)
    for t in range(8):
        ref = sum(X0[t, c] * Wt[c] for c in range(3))
        assert np.max(np.abs(V[t] - ref)) < 1e-15 * np.abs(X0[t]).sum() * np.abs(Wt).max()


# -------------------------------------------- P13: hand-derived segment tables

def test_p13_segment_tables_and_window_ends_match_golden(golden_dir):
    with open(os.path.join(golden_dir, "segment_tables.json")) as fh:
        g = json.load(fh)
    for case in g["cases"]:
        tbl = oracle.segment_table(case["rows"], case["T"], case["C"], case["doc_starts"])
        assert tbl.tolist() == case["table"], case["name"]
        starts = oracle.row_starts(case["rows"], case["T"], case["doc_starts"])
        for b in range(case["rows"]):
            ends = oracle.window_end(case["T"], case["C"], starts[b])
            assert ends.tolist() == case["window_end"][b], case["name"]


# ----------------------------------------------------------- P9: Theorem 1

def _induction(seed, tap):
    """Theorem 1 setting ([JX] 理论分析): near-orthogonal embeddings, key k* at
    t* followed by value v*, the same key queried later at n."""
    r = np.random.default_rng(seed)
    Vocab, d, f, T, C, eta = 32, 64, 256, 64, 16, 0.01
    Q, _ = np.linalg.qr(r.standard_normal((d, d)))
    E = Q[:Vocab] + r.normal(0, 0.02, (Vocab, d))
    E /= np.linalg.norm(E, axis=1, keepdims=True)
    k_star, v_star = 0, 1
    x = r.integers(2, Vocab, T)
    t_star, n = 5, 40
    x[t_star], x[t_star + 1], x[n] = k_star, v_star, k_star
    H = X0 = E[x]
    Wg = r.standard_normal((f, d)) / np.sqrt(d)
    Wu = r.standard_normal((f, d)) / np.sqrt(d)
    Wd = r.standard_normal((d, f)) / np.sqrt(f)
    w = np.zeros((d, 5))
    w[:, tap] = 1.0
    args = (H, X0, Wg, Wu, Wd, w, np.eye(d))
    O1 = oracle.forward(*args, rows=1, T=T, C=C, eta=eta)
    O0 = oracle.forward(*args, rows=1, T=T, C=C, eta=0.0)
    dl = E @ (O1["O"][n] - O0["O"][n])
    # Closed form: eta * sum over tokens of earlier chunks (e_w^T v_t)(z_t^T z_n)
    prior = np.arange(T) < (n // C) * C
    Zt, Vt = O1["Z"][prior], O1["V"][prior]
    closed = eta * (E @ Vt.T) @ (Zt @ O1["Z"][n])
    return dl, closed, v_star, k_star


def test_p9_induction_head_lm_target_raises_value_logit():
    hits = 0
    for seed in range(12):
        dl, closed, v_star, _ = _induction(seed, tap=1)
        assert _rel(dl, closed) < 1e-10
        hits += int(np.argmax(dl) == v_star and dl[v_star] > 0)
    assert hits == 12


def test_p9_reconstruction_target_does_not_single_out_value():
    wins, dv = 0, []
    for seed in range(12):
        dl, closed, v_star, k_star = _induction(seed, tap=0)
        assert _rel(dl, closed) < 1e-10
        wins += int(np.argmax(dl) == v_star)
        dv.append(dl[v_star])
    lm = np.mean([_induction(s, tap=1)[0][1] for s in range(12)])
    assert wins == 0
    assert abs(np.mean(dv)) < 0.2 * lm


@pytest.mark.parametrize("case", range(4))
def test_outputs_at_equals_sequential_loop(case):
    """outputs_at (unrolled sum, only what the requested tokens need, zero
    chunks skipped) reproduces the sequential loop at every token, with and
    without chunks of zero X0, documents, the clip, ragged T and two rows."""
    rng = np.random.default_rng(100 + case)
    rows, T, C, d, f = 2, 53 + 7 * case, 8, 12, 20
    M = rows * T
    H = rng.standard_normal((M, d))
    X0 = rng.standard_normal((M, d))
    if case % 2 == 0:  # X0 zero outside a few chunks of each row
        keep = np.zeros(M, bool)
        for b in range(rows):
            for j in (1, 3 + case):
                keep[b * T + j * C: b * T + min((j + 1) * C, T)] = True
        X0[~keep] = 0.0
    Wg, Wu = rng.standard_normal((f, d)) / np.sqrt(d), rng.standard_normal((f, d)) / np.sqrt(d)
    Wd, Wt = rng.standard_normal((d, f)) / np.sqrt(f), rng.standard_normal((d, d)) / np.sqrt(d)
    conv = rng.standard_normal((d, 5)) * 0.3
    docs = [T + 5, T + 29] if case >= 2 else None
    tau = 0.05 if case in (1, 2) else 0.0
    ref = oracle.forward(H, X0, Wg, Wu, Wd, conv, Wt, rows=rows, T=T, C=C, eta=0.1, tau=tau, doc_starts=docs)
    toks = np.arange(M)
    got, alpha = oracle.outputs_at(H, X0, Wg, Wu, Wd, conv, Wt, rows=rows, T=T, C=C, eta=0.1, tau=tau,
                            doc_starts=docs, tokens=toks)
    assert np.max(np.abs(got - ref["O"])) <= 1e-12 * np.max(np.abs(ref["O"]))
    for (b, j), a in alpha.items():
        assert a == ref["alpha"][b, j]


def test_target_variants_reduce_to_the_lm_target():
    """The ablated targets against the general definition: no conv is the
    LM target with a conv that passes tap 0 through (one-hot weights), no
    projection is the LM target with W_target = I."""
    pr = _problem(rows=2, T=37, C=8, d=6, f=10, seed=5)
    docs = [5, 37 + 20]
    one_hot = np.zeros((6, 5))
    one_hot[:, 0] = 1.0
    a = oracle.lm_target(pr["X0"], None, pr["W_target"], 2, 37, 8, docs, target="no_conv")
    b = oracle.lm_target(pr["X0"], one_hot, pr["W_target"], 2, 37, 8, docs)
    assert np.max(np.abs(a - b)) <= 1e-13 * np.max(np.abs(b))
    c = oracle.lm_target(pr["X0"], pr["conv_w"], None, 2, 37, 8, docs, target="no_proj")
    e = oracle.lm_target(pr["X0"], pr["conv_w"], np.eye(6), 2, 37, 8, docs)
    assert np.max(np.abs(c - e)) <= 1e-13 * np.max(np.abs(e))
    with pytest.raises(ValueError):
        oracle.lm_target(pr["X0"], pr["conv_w"], pr["W_target"], 2, 37, 8, docs, target="other")


# ------------------------------------------------- state carried across calls

def _piece(p, rows, T, lo, hi):
    """Tokens [lo, hi) of every row, as a problem of rows x (hi - lo)."""
    out = dict(p)
    for k in ("H", "X0"):
        out[k] = p[k].reshape(rows, T, -1)[:, lo:hi].reshape(rows * (hi - lo), -1)
    return out


def _piece_starts(docs, rows, T, lo, hi):
    n = hi - lo
    return [b * n + (s - b * T - lo) for s in docs for b in [s // T] if lo <= s - b * T < hi]


@pytest.mark.parametrize("split,tau", [(24, 0.0), (16, 0.3), (40, 0.05)])
def test_p14_streamed_pieces_equal_one_call(split, tau):
    """A long sequence read in two pieces, each a whole number of chunks, with
    the state of the open document carried from the first call into the
    second, gives the outputs and final state of one call over the whole
    sequence.  Row 0 has a document that spans the split, row 1 a document
    start exactly at the split (the listed start wins over the carry)."""
    rows, T, C = 2, 48, 8
    docs = [5, 30, T + 11, T + 24]
    p = _problem(rows=rows, T=T, C=C, d=6, f=10, seed=21)
    eta = 0.2
    one = _fwd(p, rows=rows, T=T, C=C, eta=eta, tau=tau, doc_starts=docs, want_state=True)
    a = _fwd(_piece(p, rows, T, 0, split), rows=rows, T=split, C=C, eta=eta, tau=tau,
             doc_starts=_piece_starts(docs, rows, T, 0, split), want_state=True)
    bpart = _fwd(_piece(p, rows, T, split, T), rows=rows, T=T - split, C=C, eta=eta, tau=tau,
                 doc_starts=_piece_starts(docs, rows, T, split, T), continues=[1, 1],
                 S_in=a["S"], want_state=True)
    O = np.concatenate([a["O"].reshape(rows, split, -1), bpart["O"].reshape(rows, T - split, -1)], axis=1)
    np.testing.assert_allclose(O.reshape(rows * T, -1), one["O"], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(np.concatenate([a["alpha"], bpart["alpha"]], axis=1), one["alpha"], rtol=1e-13)
    np.testing.assert_allclose(bpart["S"], one["S"], rtol=1e-12, atol=1e-15)
    # the carry matters: without it the second piece differs where the
    # document spans the split
    cold = _fwd(_piece(p, rows, T, split, T), rows=rows, T=T - split, C=C, eta=eta, tau=tau,
                doc_starts=_piece_starts(docs, rows, T, split, T))
    assert _rel(cold["O"], bpart["O"]) > 1e-6


def test_p15_final_state_is_the_sum_of_the_open_documents_deltas():
    """S after the last chunk = the sum of the clipped deltas of every chunk
    of the document open at the row's end (the unrolled sum of [JX] 工程实现):
    each chunk's last segment belongs to that document from its start on."""
    rows, T, C = 2, 40, 8
    docs = [13, T + 3, T + 17, T + 19]
    p = _problem(rows=rows, T=T, C=C, d=5, f=7, seed=5)
    out = _fwd(p, rows=rows, T=T, C=C, eta=0.3, tau=0.5, doc_starts=docs, want_state=True, want_dW=True)
    first_chunk = {0: 13 // C, 1: 19 // C}  # chunk of the last document start of each row
    for b in range(rows):
        ref = out["dW"][b, first_chunk[b]:].sum(axis=0)
        np.testing.assert_allclose(out["S"][b], ref, rtol=1e-12, atol=1e-15)
        assert np.linalg.norm(ref) > 0


def test_p16_carried_state_adds_to_w_down_until_the_first_start():
    """Tokens of a continuing row before its first document start apply
    W_down + S_in in the first chunk (the plain gated MLP with that weight),
    tokens from the start on apply W_down; S_in = 0 is the same as starting
    the row with a new document."""
    rows, T, C = 1, 24, 8
    p = _problem(rows=rows, T=T, C=C, d=6, f=9, seed=8)
    r = np.random.default_rng(3)
    S_in = r.standard_normal((1, 6, 9)) * 0.1
    out = _fwd(p, rows=rows, T=T, C=C, eta=0.4, tau=0.0, doc_starts=[5], continues=[1], S_in=S_in)
    q = dict(p, W_down=p["W_down"] + S_in[0])
    np.testing.assert_allclose(out["O"][:5], _torch_gated_mlp(q)[:5], rtol=1e-12)
    np.testing.assert_allclose(out["O"][5:8], _torch_gated_mlp(p)[5:8], rtol=1e-12)
    z0 = _fwd(p, rows=rows, T=T, C=C, eta=0.4, tau=0.0, doc_starts=[5], continues=[1],
              S_in=np.zeros((1, 6, 9)))
    plain = _fwd(p, rows=rows, T=T, C=C, eta=0.4, tau=0.0, doc_starts=[5])
    np.testing.assert_array_equal(z0["O"], plain["O"])


def test_p17_segment_table_of_a_continuing_row():
    """Hand-derived table (r0, l0, carry): T = 20, C = 8, one start at 11.
    A continuing row has no reset in chunk 0 (r0 = L = 8); a fresh row
    resets at 0."""
    cont = oracle.segment_table(1, 20, 8, [11], continues=[1])
    fresh = oracle.segment_table(1, 20, 8, [11])
    np.testing.assert_array_equal(cont[0], [[8, 0, 1], [3, 3, 1], [4, 0, 0]])
    np.testing.assert_array_equal(fresh[0], [[0, 0, 1], [3, 3, 1], [4, 0, 0]])
    # a listed start at the row start wins over the flag
    np.testing.assert_array_equal(oracle.segment_table(1, 20, 8, [0, 11], continues=[1])[0], fresh[0])


def test_outputs_at_with_carried_state_equals_sequential_loop():
    rows, T, C = 2, 40, 8
    p = _problem(rows=rows, T=T, C=C, d=6, f=8, seed=31)
    S_in = np.random.default_rng(2).standard_normal((rows, 6, 8)) * 0.05
    docs = [T + 21]
    kw = dict(rows=rows, T=T, C=C, eta=0.25, tau=0.2, doc_starts=docs, continues=[1, 1], S_in=S_in)
    full = _fwd(p, **kw)
    toks = np.array([0, 7, 19, 39, T + 2, T + 20, T + 21, T + 39])
    got, _ = oracle.outputs_at(p["H"], p["X0"], p["W_gate"], p["W_up"], p["W_down"], p["conv_w"],
                               p["W_target"], tokens=toks, **kw)
    np.testing.assert_allclose(got, full["O"][toks], rtol=1e-12, atol=1e-14)


# ----------------------------------------------------------------- backward

_GRAD_OF = {"H": "dH", "X0": "dX0", "W_gate": "dW_gate", "W_up": "dW_up", "W_down": "dW_down",
            "conv_w": "dconv_w", "W_target": "dW_target"}


def _fd_gradient(p, R, name, kw, h=1e-6):
    """Central differences of <O, R> with respect to every element of p[name]."""
    g = np.zeros_like(p[name])
    flat = g.reshape(-1)
    for j in range(flat.size):
        q = {k: v.copy() for k, v in p.items()}
        q[name].reshape(-1)[j] += h
        up = np.sum(_fwd(q, **kw)["O"] * R)
        q[name].reshape(-1)[j] -= 2 * h
        dn = np.sum(_fwd(q, **kw)["O"] * R)
        flat[j] = (up - dn) / (2 * h)
    return g


@pytest.mark.parametrize("tau", [0.0, 0.15])
def test_p18_backward_matches_finite_differences(tau):
    """Every input gradient of <O, dO> against central finite differences of
    the forward, on two ragged rows with documents inside chunks; with the
    clip on, some chunks are clipped and some are not."""
    rows, T, C = 2, 13, 4
    docs = [5, T + 7]
    p = _problem(rows=rows, T=T, C=C, d=4, f=6, seed=41)
    R = np.random.default_rng(9).standard_normal((rows * T, 4))
    kw = dict(rows=rows, T=T, C=C, eta=0.3, tau=tau, doc_starts=docs)
    alpha = _fwd(p, **kw)["alpha"]
    if tau > 0:
        assert np.any(alpha < 1) and np.any(alpha == 1)
    g = oracle.backward(p["H"], p["X0"], p["W_gate"], p["W_up"], p["W_down"], p["conv_w"], p["W_target"], R,
                        **kw)
    for name, key in _GRAD_OF.items():
        fd = _fd_gradient(p, R, name, kw)
        assert _rel(g[key], fd) < 1e-6, name
        assert np.linalg.norm(fd) > 0, name


@pytest.mark.parametrize("target", ["no_conv", "no_proj"])
def test_p18_backward_of_the_ablated_targets(target):
    rows, T, C = 1, 11, 4
    p = _problem(rows=rows, T=T, C=C, d=4, f=5, seed=43)
    R = np.random.default_rng(10).standard_normal((rows * T, 4))
    kw = dict(rows=rows, T=T, C=C, eta=0.3, tau=0.1, doc_starts=[6], target=target)
    g = oracle.backward(p["H"], p["X0"], p["W_gate"], p["W_up"], p["W_down"], p["conv_w"], p["W_target"], R,
                        **kw)
    for name in ("X0", "conv_w", "W_target"):
        key = _GRAD_OF[name]
        fd = _fd_gradient(p, R, name, kw)
        if (target, name) in (("no_conv", "conv_w"), ("no_proj", "W_target")):
            assert g[key] is None and np.all(fd == 0)
        else:
            assert _rel(g[key], fd) < 1e-6, name


def test_p19_backward_without_updates_is_the_gated_mlp_gradient():
    """eta = 0: the layer is the plain gated MLP, so dH, dW_gate, dW_up and
    dW_down equal torch autograd's gradients of it, and the target's inputs
    get exactly zero gradient."""
    rows, T, C = 1, 24, 8
    p = _problem(rows=rows, T=T, C=C, d=6, f=10, seed=44)
    R = np.random.default_rng(11).standard_normal((rows * T, 6))
    g = oracle.backward(p["H"], p["X0"], p["W_gate"], p["W_up"], p["W_down"], p["conv_w"], p["W_target"], R,
                        rows=rows, T=T, C=C, eta=0.0, tau=0.0, doc_starts=[11])
    t = {k: torch.from_numpy(p[k]).requires_grad_(True) for k in ("H", "W_gate", "W_up", "W_down")}
    F = torch.nn.functional
    O = F.linear(F.silu(F.linear(t["H"], t["W_gate"])) * F.linear(t["H"], t["W_up"]), t["W_down"])
    (O * torch.from_numpy(R)).sum().backward()
    for k in t:
        np.testing.assert_allclose(g[_GRAD_OF[k]], t[k].grad.numpy(), rtol=1e-12, atol=1e-14)
    for k in ("dX0", "dconv_w", "dW_target"):
        assert np.all(g[k] == 0)


def test_silu_grad_matches_autograd_and_is_finite():
    x = np.concatenate([RNG.standard_normal(500) * 8, [-800.0, -60.0, 0.0, 60.0, 800.0]])
    t = torch.from_numpy(x).requires_grad_(True)
    torch.nn.functional.silu(t).sum().backward()
    got = oracle.silu_grad(x)
    assert np.all(np.isfinite(got))
    np.testing.assert_allclose(got, t.grad.numpy(), rtol=1e-12, atol=1e-300)
