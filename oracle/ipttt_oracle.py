"""fp64 CPU oracle of the In-Place Test-Time Training (In-Place TTT) layer:
its forward and, for the backward pass, the gradients of its inputs.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module.  The HIP library
and its Python binding never do, and this module imports nothing from them:
the two implementations share no code.  Inputs arrive as numpy arrays that
already hold the rounded values the GPU receives; every step runs in fp64.

Sources, cited by page and section:
  [JX] lijianxiong.blog, "In-Place Test-Time Training" (ICLR 2026 Oral notes):
       方法 > 原地自适应 (gated MLP), 高效的块状更新机制 (chunks, 步骤一 apply,
       步骤二 update), 对齐语言模型的目标函数 (target, loss, update rule),
       理论分析 (Theorem 1), 工程实现 (unrolled sum, exclusive prefix).
  [TC] developer.cloud.tencent.com, "榨干MLP的剩余价值：大模型“即插即用”的动态记忆改造术":
       详细步骤 3 (k=5 conv, causal padding), 4 (deltas, prefix sum, 1e-5 norm
       clip), 验证模块一 (near-zero init), 验证模块三 (ablation of the target's
       conv and projection).
  [IP] iplexlaw.co.kr, In-Place Test-Time Training review: §3 (apply before
       update, per chunk), §6 (exclusive prefix scan, edge padding, reset at
       document end, 1e-5 clip, depthwise k=5 conv).
  [AD] admirer.cn, In-Place TTT article: 四 (parallel scan equals the
       sequential order; reset at document boundaries), 七 (padding isolates
       each delta to its chunk).

Readings taken where the pages are silent or disagree (each also listed in the
design notes): exclusive state per chunk; forward conv window t..t+4; clip of
the post-eta delta of each (chunk, document) segment to Frobenius norm tau;
loss without a 1/C factor; phi = SiLU; V_hat = Y @ W_target with W_target
stored [in, out]; a fixed row-relative chunk grid in which document starts cut
chunks into segments; a short last chunk when C does not divide T.

Document boundaries are given as ``doc_starts``: strictly increasing flat token
offsets in [0, rows*T).  Every row start is a document start whether listed or
not.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "silu", "intermediate", "row_starts", "window_end", "lm_target",
    "segment_table", "forward", "forward_prefix_scan", "plain_mlp", "outputs_at", "TARGETS",
    "silu_grad", "backward_z", "backward_target", "backward_scan_apply", "backward",
]


def silu(x):
    """SiLU(x) = x * sigmoid(x).

    The logistic function is evaluated on the branch where exp cannot
    overflow and 1 + e never cancels: 1/(1+e^-x) for x >= 0, e^x/(1+e^x) below.
    phi in the gated MLP ([JX] 方法 > 原地自适应); SiLU is the activation of the
    Qwen3 models the pages adapt ([TC] 验证模块一).
    """
    x = np.asarray(x, dtype=np.float64)
    e = np.exp(-np.abs(x))
    sig = np.where(x >= 0, 1.0 / (1.0 + e), e / (1.0 + e))
    return x * sig


def intermediate(H, W_gate, W_up):
    """Z = phi(H W_gate^T) * (H W_up^T)   ([JX] 高效的块状更新机制, definition of Z)."""
    H = np.asarray(H, dtype=np.float64)
    return silu(H @ np.asarray(W_gate, np.float64).T) * (H @ np.asarray(W_up, np.float64).T)


def plain_mlp(H, W_gate, W_up, W_down):
    """The unmodified gated MLP O = Z W_down^T ([JX] 方法 > 原地自适应)."""
    return intermediate(H, W_gate, W_up) @ np.asarray(W_down, np.float64).T


def row_starts(rows, T, doc_starts, continues=None):
    """Per row, the sorted row-relative document starts.

    0 is among them unless ``continues[b]`` is set: then the row's first
    tokens (up to its first listed start) belong to a document that began
    in an earlier call, whose state is carried in (streamed prefill of one
    long sequence in pieces, each a whole number of chunks)."""
    ds = np.asarray([] if doc_starts is None else doc_starts, dtype=np.int64)
    out = []
    for b in range(rows):
        sel = ds[(ds >= b * T) & (ds < (b + 1) * T)] - b * T
        if continues is not None and continues[b]:
            out.append(np.unique(sel))
        else:
            out.append(np.union1d(np.array([0], np.int64), sel))
    return out


def window_end(T, C, starts):
    """end(t) = min(end of t's chunk, start of the next document, T).

    The target of token t may read X0 only below end(t): padding at chunk and
    document edges keeps each chunk's delta free of later chunks and other
    documents ([TC] 详细步骤 3; [IP] §6; [AD] 七).
    """
    t = np.arange(T)
    chunk_end = np.minimum((t // C + 1) * C, T)
    if len(starts) == 0:
        return chunk_end
    nxt = np.searchsorted(starts, t, side="right")
    next_start = np.where(nxt < len(starts), starts[np.minimum(nxt, len(starts) - 1)], T)
    return np.minimum(chunk_end, next_start)


TARGETS = ("lm", "no_conv", "no_proj")


def lm_target(X0, conv_w, W_target, rows, T, C, doc_starts=None, target="lm"):
    """V_hat = Conv1D(X0) W_target  ([JX] 对齐语言模型的目标函数; [IP] §4, §6).

    Depthwise conv with k = 5 taps ([TC] 详细步骤 3; [IP] §6), read forward:
    Y[t, c] = sum_k w[c, k] * X0[t + k, c] over the taps with t + k < end(t),
    so the target of t mixes the current and the next four tokens, padded with
    zeros where the chunk or the document ends.  No bias.

    The ablation of the target's two parts ([TC] 验证模块三, objective
    decoupling, figure 3(c)): target="no_conv" drops the conv
    (V_hat = X0 W_target), "no_proj" drops the projection (V_hat = Y).
    """
    X0 = np.asarray(X0, np.float64)
    if target == "no_conv":
        return X0 @ np.asarray(W_target, np.float64)
    if target not in ("lm", "no_proj"):
        raise ValueError(target)
    w = np.asarray(conv_w, np.float64)
    Y = np.zeros_like(X0)
    for b, starts in enumerate(row_starts(rows, T, doc_starts)):
        Xb = X0[b * T:(b + 1) * T]
        end = window_end(T, C, starts)
        Yb = Y[b * T:(b + 1) * T]
        for t in range(T):
            for k in range(5):
                if t + k < end[t]:
                    Yb[t] += w[:, k] * Xb[t + k]
    if target == "no_proj":
        return Y
    return Y @ np.asarray(W_target, np.float64)


def segment_table(rows, T, C, doc_starts=None, continues=None):
    """Integer description of how document starts cut each chunk.

    For row b, chunk i covering row-relative tokens [iC, min((i+1)C, T)) of
    length L_i, returns (r0, l0, carry):
      r0    offset of the first document start inside the chunk, L_i if none
            (tokens at or after r0 use the freshly reset fast weight);
      l0    offset of the last document start inside the chunk, 0 if none
            (tokens from l0 on form the segment whose delta can carry on);
      carry 1 if chunk i+1 exists and does not begin a new document.
    Reset at document boundaries: [IP] §6 and §8; [AD] 四.  A row flagged in
    ``continues`` has no start at 0 (see row_starts).
    """
    N = -(-T // C)
    tbl = np.zeros((rows, N, 3), dtype=np.int64)
    for b, starts in enumerate(row_starts(rows, T, doc_starts, continues)):
        sset = set(int(s) for s in starts)
        for i in range(N):
            lo, hi = i * C, min((i + 1) * C, T)
            inside = [s - lo for s in range(lo, hi) if s in sset]
            tbl[b, i, 0] = inside[0] if inside else hi - lo
            tbl[b, i, 1] = inside[-1] if inside else 0
            tbl[b, i, 2] = 1 if (i + 1 < N and hi not in sset) else 0
    return tbl


def _clip(G, tau):
    """Rescale the delta to Frobenius norm tau when it is larger
    ([TC] 详细步骤 4 note; [IP] §6, "Appendix C.2" threshold 1e-5).
    Returns (scaled delta, scale).  tau <= 0 disables the clip."""
    if tau is None or tau <= 0:
        return G, 1.0
    n = float(np.sqrt(np.sum(G * G)))
    if n > tau:
        s = tau / n
        return G * s, s
    return G, 1.0


def forward(H, X0, W_gate, W_up, W_down, conv_w, W_target, *, rows, T, C, eta, tau=0.0,
            doc_starts=None, max_chunks=None, want_dW=False, target="lm", continues=None,
            S_in=None, want_state=False):
    """The strictly sequential apply-then-update loop, chunk by chunk.

    Initial fast weight W_down ([JX] 高效的块状更新机制).  For each chunk, first
    every token is mapped through the current fast weight of its document
    (步骤一, apply: O_[i] = Z_[i] W^T), then each document present in the chunk
    updates its own fast weight with the gradient step on the loss
    L = -<Z W^T, V_hat>_F, i.e. W += eta V_hat_[seg]^T Z_[seg] (步骤二 and
    对齐语言模型的目标函数), clipped per segment.  A document's fast weight starts
    at W_down when the document starts ([IP] §6, §8; [AD] 四).  Z and V_hat are
    computed chunk by chunk, which the edge padding allows.  The fast weight
    is kept as W_down + S with S the sum of the document's deltas so far (the
    unrolled form of [JX] 工程实现).

    Carrying state across calls (a long document read in pieces): a row
    flagged in ``continues`` begins inside a document whose S is S_in[b]
    (zero if S_in is None), up to its first listed start.  ``want_state``
    returns, per row, the S of the document open at the row's end after the
    update of the last processed chunk: the state the next piece continues
    from.  With pieces that are whole numbers of chunks, piecewise calls
    reproduce one call over the whole sequence.

    Returns a dict with Z, V, O ([rows*T', ...] for the processed chunks),
    alpha [rows, N'], if ``want_dW``, dW [rows, N', d, f]: the clip scale
    and the clipped delta of each chunk's last segment (the one whose state
    can continue into the next chunk), and if ``want_state``, S [rows, d, f].
    """
    H = np.asarray(H, np.float64)
    X0 = np.asarray(X0, np.float64)
    Wd = np.asarray(W_down, np.float64)
    d, f = Wd.shape
    N = -(-T // C)
    Nk = N if max_chunks is None else min(N, max_chunks)
    Tk = min(T, Nk * C)
    Z = np.zeros((rows * Tk, f))
    V = np.zeros((rows * Tk, d))
    O = np.zeros((rows * Tk, d))
    alpha = np.ones((rows, Nk))
    dW = np.zeros((rows, Nk, d, f)) if want_dW else None
    S_out = np.zeros((rows, d, f)) if want_state else None
    all_starts = row_starts(rows, T, doc_starts, continues)
    for b in range(rows):
        starts = all_starts[b]
        # document index of each token; -1 is the document carried in
        doc_of = np.searchsorted(starts, np.arange(T), side="right") - 1
        state = {}
        if continues is not None and continues[b]:
            state[-1] = np.zeros((d, f)) if S_in is None else np.array(S_in[b], np.float64)
        for i in range(Nk):
            lo, hi = i * C, min((i + 1) * C, T)
            g = slice(b * T + lo, b * T + hi)
            o = slice(b * Tk + lo, b * Tk + hi)
            Zc = intermediate(H[g], W_gate, W_up)
            # Target of this chunk only: padding stops the window at the chunk end.
            loc = starts[(starts >= lo) & (starts < hi)] - lo
            Vc = lm_target(X0[g], conv_w, W_target, 1, hi - lo, hi - lo, loc, target=target)
            Z[o], V[o] = Zc, Vc
            docs = doc_of[lo:hi]
            segs = [(int(dc), np.nonzero(docs == dc)[0]) for dc in np.unique(docs)]
            # Apply: every token of the chunk sees its document's pre-update state.
            for dc, idx in segs:
                S = state.setdefault(dc, np.zeros((d, f)))
                O[o][idx] = Zc[idx] @ (Wd + S).T
            # Update: one delta per document present in the chunk.  The last
            # segment is the one whose document can continue into chunk i+1.
            for dc, idx in segs:
                G = eta * (Vc[idx].T @ Zc[idx])
                G, s = _clip(G, tau)
                state[dc] = state[dc] + G
            alpha[b, i] = s
            if want_dW:
                dW[b, i] = G
        if want_state:
            S_out[b] = state[int(doc_of[Tk - 1])]
    return {"Z": Z, "V": V, "O": O, "alpha": alpha, "dW": dW, "S": S_out}


def forward_prefix_scan(Z, V, W_down, *, rows, T, C, eta, tau=0.0, doc_starts=None):
    """Second, independently written form: all segment deltas first, then an
    exclusive prefix sum per document, then one apply per chunk.

    This is the unrolled sum W^(i) = W^(0) + eta * sum_{j<i} V_hat_[j]^T Z_[j]
    with the prefix taken exclusively, Delta S_i = sum_{j<i} Delta W_j
    ([JX] 工程实现; [TC] 详细步骤 4; [IP] §6), restricted to one document.
    Takes Z and V_hat as inputs; returns O.
    """
    Z = np.asarray(Z, np.float64)
    V = np.asarray(V, np.float64)
    Wd = np.asarray(W_down, np.float64)
    N = -(-T // C)
    O = np.zeros((rows * T, Wd.shape[0]))
    for b, starts in enumerate(row_starts(rows, T, doc_starts)):
        doc_of = np.searchsorted(starts, np.arange(T), side="right") - 1
        # 1) deltas of every (chunk, document) segment, independent of each other
        delta = {}
        for i in range(N):
            lo, hi = i * C, min((i + 1) * C, T)
            for dc in np.unique(doc_of[lo:hi]):
                idx = lo + np.nonzero(doc_of[lo:hi] == dc)[0]
                G = eta * (V[b * T + idx].T @ Z[b * T + idx])
                delta[(i, int(dc))] = _clip(G, tau)[0]
        # 2) exclusive prefix per document and 3) apply
        for i in range(N):
            lo, hi = i * C, min((i + 1) * C, T)
            for dc in np.unique(doc_of[lo:hi]):
                idx = lo + np.nonzero(doc_of[lo:hi] == dc)[0]
                S = np.zeros_like(Wd)
                for j in range(i):
                    if (j, int(dc)) in delta:
                        S = S + delta[(j, int(dc))]
                O[b * T + idx] = Z[b * T + idx] @ (Wd + S).T
    return O


def outputs_at(H, X0, W_gate, W_up, W_down, conv_w, W_target, *, rows, T, C, eta, tau=0.0,
               doc_starts=None, tokens, target="lm", continues=None, S_in=None):
    """O at selected flat token indices, from the unrolled exclusive sum per
    document (the same definition as forward_prefix_scan, [JX] 工程实现):

      O[t] = Z[t] (W_down + sum_{j < chunk(t)} D_{j, doc(t)})^T,
      D_{j, doc} = clip(eta V_hat_[j, doc]^T Z_[j, doc])   (per segment)

    Only what the requested tokens need is computed: their own Z rows, and
    the segment deltas of earlier chunks of their documents.  A chunk whose
    rows of X0 are all zero has V_hat = 0 there (its conv window never leaves
    the chunk), so all its deltas are zero and it is skipped; with X0 zero
    outside a few chunks this makes outputs deep into a long sequence cheap.

    ``continues`` and ``S_in`` carry a document in from an earlier call, as
    in forward.

    Returns (O_rows [len(tokens), d], alpha) where alpha maps (row, chunk) to
    the clip scale of the chunk's last segment, for the chunks evaluated.
    """
    H = np.asarray(H, np.float64)
    X0 = np.asarray(X0, np.float64)
    Wd = np.asarray(W_down, np.float64)
    tokens = np.asarray(tokens, dtype=np.int64)
    all_starts = row_starts(rows, T, doc_starts, continues)
    out = np.zeros((len(tokens), Wd.shape[0]))
    alpha = {}
    delta = {}  # (row, chunk, doc) -> clipped delta of that segment

    def seg_deltas(b, j):
        lo, hi = j * C, min((j + 1) * C, T)
        g = slice(b * T + lo, b * T + hi)
        if (b, j) in alpha:
            return
        if not np.any(X0[g]):
            alpha[(b, j)] = 1.0
            return
        starts = all_starts[b]
        doc_of = np.searchsorted(starts, np.arange(lo, hi), side="right") - 1
        Zc = intermediate(H[g], W_gate, W_up)
        loc = starts[(starts >= lo) & (starts < hi)] - lo
        Vc = lm_target(X0[g], conv_w, W_target, 1, hi - lo, hi - lo, loc, target=target)
        s = 1.0
        for dc in np.unique(doc_of):
            idx = np.nonzero(doc_of == dc)[0]
            G, s = _clip(eta * (Vc[idx].T @ Zc[idx]), tau)
            delta[(b, j, int(dc))] = G
        alpha[(b, j)] = s  # the last segment's scale

    for n, t in enumerate(tokens):
        b, tt = int(t // T), int(t % T)
        i = tt // C
        starts = all_starts[b]
        dc = int(np.searchsorted(starts, tt, side="right") - 1)
        first = int(starts[dc]) // C if dc >= 0 else 0  # the document's first chunk
        W = Wd.copy()
        if dc < 0 and S_in is not None:
            W += np.asarray(S_in[b], np.float64)
        for j in range(first, i):
            seg_deltas(b, j)
            if (b, j, dc) in delta:
                W += delta[(b, j, dc)]
        out[n] = intermediate(H[t:t + 1], W_gate, W_up)[0] @ W.T
    return out, alpha


# ------------------------------------------------------------------ backward
#
# Reverse mode of the forward above: given the cotangent dO of the output O,
# the gradients of <O, dO> with respect to every input.  Each function
# follows the chain rule through the steps of the forward in reverse order;
# nothing here is fused or reordered beyond that.  The pages use these
# gradients when they train the layer further ([JX] 工程实现 and the pages'
# continued-pretraining setup); they give no formulas for them, so the
# formulas are the plain derivatives of the forward's definitions, pinned by
# finite differences of ``forward``.

def silu_grad(x):
    """d/dx SiLU(x) = s(x) (1 + x (1 - s(x))), s = the logistic function,
    evaluated on the same overflow-free branches as ``silu``."""
    x = np.asarray(x, dtype=np.float64)
    e = np.exp(-np.abs(x))
    s = np.where(x >= 0, 1.0 / (1.0 + e), e / (1.0 + e))
    return s * (1.0 + x * (1.0 - s))


def backward_z(H, W_gate, W_up, dZ):
    """Gradients through Z = SiLU(H W_gate^T) * (H W_up^T)
    ([JX] 方法 > 原地自适应).  Returns dH, dW_gate, dW_up."""
    H = np.asarray(H, np.float64)
    Wg = np.asarray(W_gate, np.float64)
    Wu = np.asarray(W_up, np.float64)
    dZ = np.asarray(dZ, np.float64)
    G = H @ Wg.T
    U = H @ Wu.T
    dG = dZ * U * silu_grad(G)
    dU = dZ * silu(G)
    return {"dH": dG @ Wg + dU @ Wu, "dW_gate": dG.T @ H, "dW_up": dU.T @ H}


def backward_target(X0, conv_w, W_target, dV, *, rows, T, C, doc_starts=None, target="lm"):
    """Gradients through V_hat = Conv1D(X0) W_target (and its ablations):
    dY = dV W_target^T, dW_target = Y^T dV, and through the windowed conv
    Y[t] = sum_{k < w(t)} w[:, k] * X0[t + k]: dconv[:, k] = sum_t dY[t] *
    X0[t + k] and dX0[t + k] += w[:, k] * dY[t] over the same taps
    ([JX] 对齐语言模型的目标函数; [TC] 详细步骤 3; [IP] §6).  Returns dX0,
    dconv_w (None without the conv) and dW_target (None without the
    projection)."""
    X0 = np.asarray(X0, np.float64)
    dV = np.asarray(dV, np.float64)
    if target not in TARGETS:
        raise ValueError(target)
    if target == "no_conv":
        Y = X0
    else:
        Y = lm_target(X0, conv_w, None, rows, T, C, doc_starts, target="no_proj")
    if target == "no_proj":
        dY, dWt = dV, None
    else:
        Wt = np.asarray(W_target, np.float64)
        dY, dWt = dV @ Wt.T, Y.T @ dV
    if target == "no_conv":
        return {"dX0": dY, "dconv_w": None, "dW_target": dWt}
    w = np.asarray(conv_w, np.float64)
    dX0 = np.zeros_like(X0)
    dw = np.zeros_like(w)
    for b, starts in enumerate(row_starts(rows, T, doc_starts)):
        end = window_end(T, C, starts)
        o = b * T
        for t in range(T):
            for k in range(5):
                if t + k < end[t]:
                    dw[:, k] += dY[o + t] * X0[o + t + k]
                    dX0[o + t + k] += w[:, k] * dY[o + t]
    return {"dX0": dX0, "dconv_w": dw, "dW_target": dWt}


def backward_scan_apply(Z, V, W_down, dO, *, rows, T, C, eta, tau=0.0, doc_starts=None):
    """Gradients through the chunk deltas, their clip, the exclusive
    segmented scan and the apply, given Z and V_hat: returns dZ, dV (d V_hat)
    and dW_down.

    The forward is replayed chunk by chunk as in ``forward`` (apply with the
    pre-update state of each token's document, then one clipped delta per
    document segment).  The reverse pass walks the chunks backwards, holding
    per document the adjoint of its state after the current chunk's update:
      - update: the delta's adjoint is that state adjoint g.  The delta is
        eta*D with D = V_seg^T Z_seg, or tau*D/|D| when clipped, so
        dD = eta*g, or (tau/|D|) (g - D <g, D>/|D|^2) when clipped; then
        dV_seg += Z_seg dD^T and dZ_seg += V_seg dD;
      - apply: O = Z (W_down + S)^T gives dZ += dO (W_down + S),
        dW_down += dO^T Z, and the state before the update gains dO^T Z.
    """
    Z = np.asarray(Z, np.float64)
    V = np.asarray(V, np.float64)
    dO = np.asarray(dO, np.float64)
    Wd = np.asarray(W_down, np.float64)
    d, f = Wd.shape
    N = -(-T // C)
    dZ = np.zeros_like(Z)
    dV = np.zeros_like(V)
    dWd = np.zeros_like(Wd)
    for b, starts in enumerate(row_starts(rows, T, doc_starts)):
        doc_of = np.searchsorted(starts, np.arange(T), side="right") - 1
        state, applied, updates = {}, [], []
        for i in range(N):
            lo, hi = i * C, min((i + 1) * C, T)
            docs = doc_of[lo:hi]
            segs = [(int(dc), b * T + lo + np.nonzero(docs == dc)[0]) for dc in np.unique(docs)]
            applied.append([(dc, idx, state.setdefault(dc, np.zeros((d, f))).copy()) for dc, idx in segs])
            up = []
            for dc, idx in segs:
                D = V[idx].T @ Z[idx]
                Gc, s = _clip(eta * D, tau)
                state[dc] = state[dc] + Gc
                up.append((dc, idx, D, s))
            updates.append(up)
        g = {}
        for i in reversed(range(N)):
            for dc, idx, D, s in updates[i]:
                a = g.get(dc)
                if a is None:
                    continue
                nD2 = float(np.sum(D * D))
                if s != 1.0:
                    dD = (tau / np.sqrt(nD2)) * (a - D * (float(np.sum(a * D)) / nD2))
                else:
                    dD = eta * a
                dV[idx] += Z[idx] @ dD.T
                dZ[idx] += V[idx] @ dD
            for dc, idx, S in applied[i]:
                dZ[idx] += dO[idx] @ (Wd + S)
                P = dO[idx].T @ Z[idx]
                dWd += P
                g[dc] = g.get(dc, 0.0) + P
    return {"dZ": dZ, "dV": dV, "dW_down": dWd}


def backward(H, X0, W_gate, W_up, W_down, conv_w, W_target, dO, *, rows, T, C, eta, tau=0.0,
             doc_starts=None, target="lm"):
    """Gradients of <O, dO> with respect to H, X0, W_gate, W_up, W_down,
    conv_w and W_target: the three backward steps in reverse order of the
    forward.  Also returns the intermediate dZ and dV."""
    Z = intermediate(H, W_gate, W_up)
    V = lm_target(X0, conv_w, W_target, rows, T, C, doc_starts, target=target)
    sa = backward_scan_apply(Z, V, W_down, dO, rows=rows, T=T, C=C, eta=eta, tau=tau, doc_starts=doc_starts)
    tg = backward_target(X0, conv_w, W_target, sa["dV"], rows=rows, T=T, C=C, doc_starts=doc_starts,
                         target=target)
    zz = backward_z(H, W_gate, W_up, sa["dZ"])
    out = dict(sa)
    out.update(tg)
    out.update(zz)
    return out
