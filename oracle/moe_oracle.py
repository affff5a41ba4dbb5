"""CPU oracle for the MoE layer forward and backward pass.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the package smoke check and
the CPU-baseline leg of the benchmark may import this module.  It shares no
code with the HIP path and must never be used to produce the product's
results.

What it computes (the plain definition of the layer):

    y_t = s(x_t) + sum_e m[t,e] * g[t,e] * FFN_e(x_t)
    FFN_e(z) = (silu(z W_g[e]^T) * (z W_u[e]^T)) W_d[e]^T

* The router picks, for each token, k of the E experts; only the picked
  experts run on that token, and their outputs are weighted by the gates and
  summed (Ultimate MoE Training Handbook, section 2.5 "First training of
  MoE": the router selects 8 of 64 smaller experts per token; tokens are sent
  to the selected experts and their outputs returned).
* Each expert is a SwiGLU feed-forward block without bias, i.e. three weight
  matrices (Handbook 2.5, "Calculation of activated parameters and total
  parameters").
* Router logits are computed in fp32 (Handbook 2.5, the fp32 router dtype
  flag).  Scores are either a softmax over the experts (top-k softmax router)
  or a per-expert sigmoid (DeepSeek-V3 style router); shared experts run on
  every token and are added ungated (KempnerForge README, "Features /
  Architecture" and "Sparse architecture research").
* Sigmoid routing adds a per-expert bias to the scores only to decide which
  experts are picked; the gate values use the unbiased scores (Apex-3 code
  page, "What's inside", row "Fine-grained MoE": the bias balances load
  without a loss term).
* Dropless: every assignment is computed (no capacity factor appears for the
  pages' MoE runs).

Readings taken where the pages are silent (each is a single switch here):
  - softmax gates are the full-softmax probabilities of the picked experts,
    renormalised over the top k only when ``renorm`` is set;
  - sigmoid gates are the picked scores divided by their sum;
  - ties in the selection key go to the lower expert index; slot j holds the
    j-th best expert;
  - inside an expert's segment, rows keep assignment order a = t*k + j;
  - no routed scaling factor (it is 1).

Precision: the router is fp32 as the pages state.  Logits are the fp64 product
rounded once to fp32; the sigmoid / softmax scores are evaluated in fp64 from
those fp32 logits and rounded once to fp32; a sigmoid selection key is the
fp32 sum of the fp32 score and the fp32 bias.  Gates are fp32.  Everything in
the expert path (GEMMs, activation, combine, backward) is fp64, computed from
the exact values of the stored inputs.

Parity pins (tests/test_oracle_pins.py): dense-masked brute force, torch fp64
autograd, central finite differences, single-expert == dense, granularity
identity, permutation invariants, gate renormalisation, bias-selects-only,
brute-force top-k, the softmax Jacobian special case and the Handbook's
parameter count; for the router training terms, torch fp64 autograd of each
loss, the single-expert loss of exactly 1, balanced loads, the z-loss closed
form and the bias update on balanced and skewed loads; for the fp8 mode, the
e4m3 format table and rounding, exactness of every product on the e4m3 grid,
the half-step error bound off it, power-of-two equivariance of the whole
layer, closeness to the exact layer and the bf16 rounding rule; for the e5m2
gradient format, its decode table and rounding, brute-force nearest search,
the row-wise half-step bound and exactness of the down data gradient on the
e5m2 grid; for the fp8 weight gradients, exactness on the grid by columns
(and of every weight gradient of a grid layer), the half-step bound and
power-of-two equivariance.  Every function below is covered by at least one
pin.
"""
from __future__ import annotations

import numpy as np

F32 = np.float32
F64 = np.float64


# ----------------------------------------------------------------------------- router
def router_logits(x, w_router):
    """logits = x W_r^T, fp64 product rounded once to fp32 (fp32 router).

    x: [T, d] (any float dtype, taken exactly); w_router: [E, d] fp32."""
    return (np.asarray(x, F64) @ np.asarray(w_router, F64).T).astype(F32)


def router_scores(logits32, score):
    """Per-expert scores from fp32 logits, evaluated in fp64, rounded to fp32.

    softmax: p = exp(l - max l) / sum exp(l - max l) over the E experts.
    sigmoid: s = 1 / (1 + exp(-l)), independently per expert."""
    l = np.asarray(logits32, F32).astype(F64)
    if score == "softmax":
        z = np.exp(l - l.max(axis=1, keepdims=True))
        return (z / z.sum(axis=1, keepdims=True)).astype(F32)
    if score == "sigmoid":
        return (1.0 / (1.0 + np.exp(-l))).astype(F32)
    raise ValueError(score)


def selection_keys(logits32, scores32, bias32, score):
    """The value experts are ranked by.

    softmax: the logit itself (same order as the probability, no exp rounding).
    sigmoid: score + bias, one fp32 addition; a missing bias means zero."""
    if score == "softmax":
        return np.asarray(logits32, F32).copy()
    s = np.asarray(scores32, F32)
    if bias32 is None:
        return s.copy()
    return (s + np.asarray(bias32, F32)[None, :]).astype(F32)


def select_topk(keys32, k):
    """Pick k experts per token: key descending, ties to the lower index.

    Returns idx [T, k] int32 (slot j = j-th best) and the selection margin
    key_(k) - key_(k+1) per token (inf when k == E)."""
    keys = np.asarray(keys32, F32)
    T, E = keys.shape
    # a stable sort of the negated key keeps equal keys in index order
    order = np.argsort(-keys, axis=1, kind="stable")
    idx = order[:, :k].astype(np.int32)
    if k < E:
        kth = np.take_along_axis(keys, order[:, k - 1:k], axis=1)[:, 0].astype(F64)
        nxt = np.take_along_axis(keys, order[:, k:k + 1], axis=1)[:, 0].astype(F64)
        margin = kth - nxt
    else:
        margin = np.full(T, np.inf)
    return idx, margin


def gates_from_scores(scores32, idx, score, renorm):
    """Gate values of the picked experts (fp32).

    softmax: the picked probabilities, divided by their sum if ``renorm``.
    sigmoid: the picked (unbiased) scores divided by their sum."""
    picked = np.take_along_axis(np.asarray(scores32, F32), idx, axis=1).astype(F64)
    if score == "softmax" and not renorm:
        return picked.astype(F32)
    return (picked / picked.sum(axis=1, keepdims=True)).astype(F32)


# ----------------------------------------------------------------------------- permutation
def permute_indices(idx, E):
    """Expert-contiguous order of the T*k assignments a = t*k + j.

    counts[e]: assignments routed to e; offsets: exclusive prefix sum
    (offsets[E] = T*k); src[p]: the assignment stored at permuted row p, rows
    of one expert in increasing a; pos[a]: the row that assignment a went to
    (pos and src are inverse permutations)."""
    expert_of_a = np.asarray(idx, np.int64).reshape(-1)
    A = expert_of_a.size
    counts = np.bincount(expert_of_a, minlength=E).astype(np.int32)
    offsets = np.zeros(E + 1, np.int64)
    offsets[1:] = np.cumsum(counts)
    src = np.argsort(expert_of_a, kind="stable").astype(np.int32)
    pos = np.empty(A, np.int32)
    pos[src] = np.arange(A, dtype=np.int32)
    return counts, offsets.astype(np.int32), pos, src


# ----------------------------------------------------------------------------- experts
def silu(z):
    return z / (1.0 + np.exp(-z))


def swiglu_ffn(z, w_gate, w_up, w_down):
    """One SwiGLU FFN on rows z: returns (G, U, H, Y) with
    G = z W_g^T, U = z W_u^T, H = silu(G) * U, Y = H W_d^T (fp64)."""
    G = z @ w_gate.T
    U = z @ w_up.T
    H = silu(G) * U
    return G, U, H, H @ w_down.T


def swiglu_ffn_backward(z, w_gate, w_up, w_down, G, U, H, dY):
    """Reverse of ``swiglu_ffn`` for upstream dY: returns
    (dz, dW_g, dW_u, dW_d) with dH = dY W_d, dG = dH * U * silu'(G),
    dU = dH * silu(G), silu'(g) = sig(g) (1 + g (1 - sig(g)))."""
    dH = dY @ w_down
    sg = 1.0 / (1.0 + np.exp(-G))
    dG = dH * U * sg * (1.0 + G * (1.0 - sg))
    dU = dH * (G * sg)
    dW_d = dY.T @ H
    dW_g = dG.T @ z
    dW_u = dU.T @ z
    dz = dG @ w_gate + dU @ w_up
    return dz, dW_g, dW_u, dW_d, dG, dU


def _split_gateup(w_gateup):
    f = w_gateup.shape[-2] // 2
    return w_gateup[..., :f, :], w_gateup[..., f:, :]


# ----------------------------------------------------------------------------- layer
def forward(x, w_router, bias, w_gateup, w_down, s_gateup=None, s_down=None, *,
            top_k, score, renorm=False, forced_idx=None, forced_gate=None, fp8=False, forced_h=None,
            forced_s_h=None):
    """Forward pass of the MoE layer on the tokens of ``x``.

    x: [T, d]; w_router: [E, d] fp32; bias: [E] fp32 or None (sigmoid only);
    w_gateup: [E, 2f, d] (gate rows, then up rows); w_down: [E, d, f];
    s_gateup: [2F, d], s_down: [d, F] for the shared experts (concatenated
    along their hidden width) or None.  Weights are taken exactly in fp64.

    ``forced_idx`` replaces the selection (used to follow another
    implementation's choice on near-tied tokens); gates are then recomputed
    from this oracle's own scores for the forced experts, unless
    ``forced_gate`` [T, k] (fp32) replaces them too: another implementation's
    rounding of the same gate values.

    ``fp8``: the expert products (routed and shared) run as e4m3 products
    with row-wise scales (``swiglu_ffn_fp8``); the router stays fp32.
    ``forced_h`` / ``forced_s_h`` replace the bf16 copy of H that the down
    products quantise (permuted rows / token rows): another implementation's
    rounding of the same H, used where its fp32 sums round the other way.

    Returns a dict with every intermediate of the layer."""
    x = np.asarray(x, F64)
    T, d = x.shape
    E = w_router.shape[0]
    k = int(top_k)
    logits = router_logits(x, w_router)
    scores = router_scores(logits, score)
    keys = selection_keys(logits, scores, bias if score == "sigmoid" else None, score)
    idx, margin = select_topk(keys, k)
    if forced_idx is not None:
        idx = np.asarray(forced_idx, np.int32).reshape(T, k)
    gate = gates_from_scores(scores, idx, score, renorm)
    if forced_gate is not None:
        gate = np.asarray(forced_gate, F32).reshape(T, k)
    counts, offsets, pos, src = permute_indices(idx, E)

    A = T * k
    f = w_gateup.shape[1] // 2
    tok_of_row = src // k
    x_perm = x[tok_of_row]
    preact = np.empty((A, 2 * f), F64)
    h = np.empty((A, f), F64)
    h_q = np.zeros((A, f), F64) if fp8 else None   # the bf16 H the fp8 down products quantised
    y_perm = np.empty((A, d), F64)
    wg_all, wu_all = _split_gateup(np.asarray(w_gateup))
    for e in range(E):
        r0, r1 = int(offsets[e]), int(offsets[e + 1])
        if r1 == r0:
            continue
        if fp8:
            G, U, H, Y, Hq = swiglu_ffn_fp8(x_perm[r0:r1], np.asarray(wg_all[e], F64),
                                            np.asarray(wu_all[e], F64), np.asarray(w_down[e], F64),
                                            None if forced_h is None else forced_h[r0:r1])
            h_q[r0:r1] = Hq
        else:
            G, U, H, Y = swiglu_ffn(x_perm[r0:r1], np.asarray(wg_all[e], F64),
                                    np.asarray(wu_all[e], F64), np.asarray(w_down[e], F64))
        preact[r0:r1, :f] = G
        preact[r0:r1, f:] = U
        h[r0:r1] = H
        y_perm[r0:r1] = Y

    out = dict(logits=logits, scores=scores, keys=keys, idx=idx, margin=margin, gate=gate,
               counts=counts, offsets=offsets, pos=pos, src=src, x_perm=x_perm,
               preact=preact, h=h, y_perm=y_perm, h_q=h_q)

    if s_gateup is not None:
        sg, su = _split_gateup(np.asarray(s_gateup, F64))
        Hsq = None
        if fp8:
            Gs, Us, Hs, ys, Hsq = swiglu_ffn_fp8(x, sg, su, np.asarray(s_down, F64), forced_s_h)
        else:
            Gs, Us, Hs, ys = swiglu_ffn(x, sg, su, np.asarray(s_down, F64))
        out.update(s_preact=np.concatenate([Gs, Us], axis=1), s_h=Hs, ys=ys, s_h_q=Hsq)
    else:
        ys = np.zeros((T, d), F64)
        out.update(s_preact=None, s_h=None, ys=None, s_h_q=None)

    out["y"] = combine(y_perm, gate, pos, ys)
    return out


def combine(y_perm, gate, pos, shared_y=None):
    """y[t] = sum_j gate[t,j] * y_perm[pos[t*k+j]] (+ shared_y[t]): slot order,
    shared output last (fp64)."""
    T, k = gate.shape
    y = np.zeros((T, y_perm.shape[1]), F64)
    g64 = np.asarray(gate, F32).astype(F64)
    rows = np.asarray(pos).reshape(T, k)
    for j in range(k):
        y += g64[:, j:j + 1] * np.asarray(y_perm, F64)[rows[:, j]]
    if shared_y is not None:
        y += shared_y
    return y


def combine_backward(dy, y_perm, gate, pos, src):
    """Reverse of ``combine``: d(y_perm)[p] = gate * dy[token of p] and
    dgate[t,j] = <dy[t], y_perm[pos[t*k+j]]>."""
    dy = np.asarray(dy, F64)
    T, k = gate.shape
    tok_of_row = np.asarray(src) // k
    slot_of_row = np.asarray(src) % k
    g64 = np.asarray(gate, F32).astype(F64)
    dy_perm = g64[tok_of_row, slot_of_row][:, None] * dy[tok_of_row]
    rows = np.asarray(pos).reshape(T, k)
    yp = np.asarray(y_perm, F64)
    dgate = np.stack([(dy * yp[rows[:, j]]).sum(axis=1) for j in range(k)], axis=1)
    return dy_perm, dgate


def unpermute_sum(dx_perm, pos, k, dx_shared=None, dx_router=None):
    """dx[t] = sum_j dx_perm[pos[t*k+j]] (+ dx_shared[t]) (+ dx_router[t])."""
    rows = np.asarray(pos).reshape(-1, k)
    T = rows.shape[0]
    dxp = np.asarray(dx_perm, F64)
    dx = np.zeros((T, dxp.shape[1]), F64)
    for j in range(k):
        dx += dxp[rows[:, j]]
    if dx_shared is not None:
        dx += dx_shared
    if dx_router is not None:
        dx += dx_router
    return dx


def router_backward(dgate, scores32, idx, score, renorm):
    """Gradient of the loss w.r.t. the fp32 logits, given dL/dgate [T, k].

    The selection is piecewise constant, so gradient reaches the router only
    through the gate values; the bias receives none.
      sigmoid:  g_i = s_i / S, S = sum of picked s  ->  ds_i = (dg_i - <g, dg>) / S
                on picked experts, dl = ds * s * (1 - s), zero elsewhere.
      softmax:  dp = dgate scattered onto the picked experts (through the
                renormalisation when it is on), then the softmax Jacobian
                dl = p * (dp - <p, dp>) over all experts."""
    s = np.asarray(scores32, F32).astype(F64)
    T, E = s.shape
    dg = np.asarray(dgate, F64)
    picked = np.take_along_axis(s, idx, axis=1)
    if score == "sigmoid" or renorm:
        S = picked.sum(axis=1, keepdims=True)
        g = picked / S
        dpicked = (dg - (g * dg).sum(axis=1, keepdims=True)) / S
    else:
        dpicked = dg
    dscore = np.zeros((T, E), F64)
    np.put_along_axis(dscore, idx.astype(np.int64), dpicked, axis=1)
    if score == "sigmoid":
        return dscore * s * (1.0 - s)
    return s * (dscore - (s * dscore).sum(axis=1, keepdims=True))


# ----------------------------------------------------------------------------- router training terms
# Apex-3 code page ("What's inside", "Fine-grained MoE"; "Run it yourself":
# router_bias_update=proportional, router_bias_rate 1e-3 in training and 0.01
# in the benchmark, seq_aux_alpha=1e-3); Ultimate MoE Training Handbook 2.5
# (an auxiliary load-balancing loss with coefficient 1e-3, equal to exactly 1
# with a single expert); KempnerForge README ("Features": router z-loss;
# "MoE roadmap": sequence aux loss, adaptive bias, z-loss).

def routing_distribution(logits32, score):
    """q[t, e]: the router's distribution over all E experts, fp64.
    softmax: the probabilities; sigmoid: the scores normalised to sum 1."""
    l = np.asarray(logits32, F32).astype(F64)
    if score == "softmax":
        z = np.exp(l - l.max(axis=1, keepdims=True))
        return z / z.sum(axis=1, keepdims=True)
    s = 1.0 / (1.0 + np.exp(-l))
    return s / s.sum(axis=1, keepdims=True)


def _dlogits_from_dq(logits32, score, dq):
    """Chain a gradient w.r.t. q (routing_distribution) back to the logits."""
    l = np.asarray(logits32, F32).astype(F64)
    if score == "softmax":
        q = routing_distribution(logits32, score)
        return q * (dq - (q * dq).sum(axis=1, keepdims=True))
    s = 1.0 / (1.0 + np.exp(-l))
    S = s.sum(axis=1, keepdims=True)
    q = s / S
    ds = (dq - (q * dq).sum(axis=1, keepdims=True)) / S
    return ds * s * (1.0 - s)


def aux_loss(logits32, counts, k, score, coeff):
    """Load-balancing loss over the whole batch: coeff * E * sum_e f_e P_e with
    f_e = counts_e / (T k) (share of the assignments, no gradient) and
    P_e = mean over tokens of q[t, e].  Returns (value, dlogits [T, E])."""
    q = routing_distribution(logits32, score)
    T, E = q.shape
    f = np.asarray(counts, F64) / (T * k)
    P = q.mean(axis=0)
    value = coeff * E * float((f * P).sum())
    dq = np.broadcast_to(coeff * E * f / T, (T, E))
    return value, _dlogits_from_dq(logits32, score, dq)


def seq_aux_loss(logits32, idx, k, score, coeff, seq_len):
    """The same balance measured per sequence of seq_len tokens and averaged
    over the sequences: f^s_e = E/(k S) * #(tokens of s that picked e),
    P^s_e = mean over the tokens of s of q[t, e]."""
    q = routing_distribution(logits32, score)
    T, E = q.shape
    S = seq_len if seq_len else T
    n = T // S
    value = 0.0
    dq = np.zeros((T, E))
    for sq in range(n):
        t0, t1 = sq * S, (sq + 1) * S
        c = np.bincount(np.asarray(idx[t0:t1]).reshape(-1), minlength=E).astype(F64)
        f = c * E / (k * S)
        P = q[t0:t1].mean(axis=0)
        value += float((f * P).sum())
        dq[t0:t1] = f / S
    value *= coeff / n
    return value, _dlogits_from_dq(logits32, score, dq * coeff / n)


def z_loss(logits32, coeff):
    """coeff * mean over tokens of logsumexp(l_t)^2; gradient
    coeff * 2/T * lse_t * softmax(l_t)."""
    l = np.asarray(logits32, F32).astype(F64)
    T = l.shape[0]
    m = l.max(axis=1, keepdims=True)
    z = np.exp(l - m)
    lse = (m + np.log(z.sum(axis=1, keepdims=True)))
    value = coeff * float((lse[:, 0] ** 2).mean())
    return value, coeff * 2.0 / T * lse * (z / z.sum(axis=1, keepdims=True))


def router_terms(logits32, idx, counts, k, score, terms):
    """Sum of the enabled terms: (values dict, dlogits [T, E]).  terms holds
    aux_coeff, seq_aux_coeff, z_coeff and seq_len (0: one sequence)."""
    T, E = np.asarray(logits32).shape
    dl = np.zeros((T, E))
    vals = {"aux": 0.0, "seq_aux": 0.0, "z": 0.0}
    if terms.get("aux_coeff", 0.0):
        vals["aux"], g = aux_loss(logits32, counts, k, score, terms["aux_coeff"])
        dl += g
    if terms.get("seq_aux_coeff", 0.0):
        vals["seq_aux"], g = seq_aux_loss(logits32, idx, k, score, terms["seq_aux_coeff"],
                                          terms.get("seq_len", 0))
        dl += g
    if terms.get("z_coeff", 0.0):
        vals["z"], g = z_loss(logits32, terms["z_coeff"])
        dl += g
    return vals, dl


def bias_update(bias32, counts, T, k, rate):
    """Proportional load-balancing bias update after a step: each expert's
    bias moves by rate * (mean load - its load) / mean load, mean load
    T k / E; evaluated in fp64 and rounded once to fp32."""
    b = np.asarray(bias32, F32).astype(F64)
    E = b.shape[0]
    mean = T * k / E
    c = np.asarray(counts, F64)
    return (b + F64(np.float32(rate)) * (mean - c) / mean).astype(F32)


def backward(x, w_router, w_gateup, w_down, s_gateup, s_down, fwd, dy, *, score, renorm=False,
             terms=None, fp8=False, forced_dgu=None, forced_s_dgu=None, fp8_grad_format="e4m3",
             fp8_wgrad=False):
    """Backward pass for upstream gradient dy [T, d], reusing ``forward``'s dict.

    Returns dict: dx [T,d], d_w_gateup [E,2f,d], d_w_down [E,d,f],
    d_s_gateup / d_s_down (or None), d_w_router [E,d], d_logits [T,E],
    dgate [T,k], plus the permuted intermediates dy_perm, dgu, dx_perm.

    ``fp8``: the expert data gradients (routed and shared) run as e4m3
    products (``swiglu_ffn_backward_fp8``); weight gradients stay exact.
    ``forced_dgu`` [A, 2f] / ``forced_s_dgu`` [T, 2F] replace the bf16 copies
    of dG | dU that the gate/up data gradients quantise (another
    implementation's rounding of the same values); the returned dgu / s_dgu
    are this oracle's own.  ``fp8_grad_format``: "e4m3" or "e5m2" for the
    gradient operands of the fp8 data gradients (the weights stay e4m3).
    ``fp8_wgrad`` (with fp8): the weight gradients are e4m3 products too, of
    operands quantised along each expert's rows (``wgrad_fp8``), H as the
    forward's down products quantised it."""
    x = np.asarray(x, F64)
    dy = np.asarray(dy, F64)
    T, d = x.shape
    E = w_router.shape[0]
    idx, gate, pos, src, offsets = fwd["idx"], fwd["gate"], fwd["pos"], fwd["src"], fwd["offsets"]
    k = idx.shape[1]
    A = T * k
    f = w_gateup.shape[1] // 2
    dy_perm, dgate = combine_backward(dy, fwd["y_perm"], gate, pos, src)

    wg_all, wu_all = _split_gateup(np.asarray(w_gateup))
    d_w_gateup = np.zeros((E, 2 * f, d), F64)
    d_w_down = np.zeros((E, d, f), F64)
    dgu = np.zeros((A, 2 * f), F64)
    dx_perm = np.zeros((A, d), F64)
    for e in range(E):
        r0, r1 = int(offsets[e]), int(offsets[e + 1])
        if r1 == r0:
            continue
        G = fwd["preact"][r0:r1, :f]
        U = fwd["preact"][r0:r1, f:]
        args = (fwd["x_perm"][r0:r1], np.asarray(wg_all[e], F64), np.asarray(wu_all[e], F64),
                np.asarray(w_down[e], F64), G, U, fwd["h"][r0:r1], dy_perm[r0:r1])
        if fp8:
            dz, dWg, dWu, dWd, dG, dU = swiglu_ffn_backward_fp8(
                *args, None if forced_dgu is None else forced_dgu[r0:r1], fp8_grad_format,
                fwd["h_q"][r0:r1] if fp8_wgrad else None)
        else:
            dz, dWg, dWu, dWd, dG, dU = swiglu_ffn_backward(*args)
        d_w_gateup[e, :f] = dWg
        d_w_gateup[e, f:] = dWu
        d_w_down[e] = dWd
        dgu[r0:r1, :f] = dG
        dgu[r0:r1, f:] = dU
        dx_perm[r0:r1] = dz

    out = dict(dgate=dgate, dy_perm=dy_perm, dgu=dgu, dx_perm=dx_perm,
               d_w_gateup=d_w_gateup, d_w_down=d_w_down)

    if s_gateup is not None:
        sg, su = _split_gateup(np.asarray(s_gateup, F64))
        Fs = sg.shape[0]
        Gs = fwd["s_preact"][:, :Fs]
        Us = fwd["s_preact"][:, Fs:]
        args = (x, sg, su, np.asarray(s_down, F64), Gs, Us, fwd["s_h"], dy)
        if fp8:
            dxs, dSg, dSu, dSd, dGs, dUs = swiglu_ffn_backward_fp8(*args, forced_s_dgu, fp8_grad_format,
                                                                    fwd["s_h_q"] if fp8_wgrad else None)
        else:
            dxs, dSg, dSu, dSd, dGs, dUs = swiglu_ffn_backward(*args)
        out["s_dgu"] = np.concatenate([dGs, dUs], axis=1)
        out["d_s_gateup"] = np.concatenate([dSg, dSu], axis=0)
        out["d_s_down"] = dSd
        out["dx_shared"] = dxs
    else:
        out["d_s_gateup"] = None
        out["d_s_down"] = None
        out["s_dgu"] = None
        dxs = np.zeros((T, d), F64)
        out["dx_shared"] = None

    dlogits = router_backward(dgate, fwd["scores"], idx, score, renorm)
    if terms is not None:
        out["router_terms"], dl_terms = router_terms(fwd["logits"], idx, fwd["counts"], k, score, terms)
        dlogits = dlogits + dl_terms
    wr = np.asarray(w_router, F32).astype(F64)
    out["d_logits"] = dlogits
    out["d_w_router"] = dlogits.T @ x
    dx_router = dlogits @ wr
    out["dx_router"] = dx_router

    # unpermute-sum: slot order, then shared, then router contribution
    out["dx"] = unpermute_sum(dx_perm, pos, k, dxs, dx_router)
    return out


def expert_parameter_count(d_model, d_ff):
    """Weights in one SwiGLU expert without bias: three d_model x d_ff matrices."""
    return 3 * int(d_model) * int(d_ff)


# ----------------------------------------------------------------------------- fp8 (e4m3) experts
# Apex-3 code page ("What's inside": FP8 through torchao; "Run it yourself":
# --precision fp8_rowwise); KempnerForge README ("MoE roadmap": FP8 mixed
# precision).  Format: OCP e4m3 -- 1 sign, 4 exponent (bias 7), 3 mantissa
# bits; exponent 0 holds the subnormals m/8 * 2^-6; 0x7f / 0xff are NaN; the
# largest finite value is 448 (no infinities).

def _e4m3_values():
    """Value of each of the 256 e4m3 codes (index = code), fp64."""
    c = np.arange(256, dtype=np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 15
    m = c & 7
    val = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e.astype(F64) - 7.0))
    val = np.where((e == 15) & (m == 7), np.nan, val)
    return sign * val


_E4M3_VALUES = _e4m3_values()


def e4m3_decode(codes):
    """Value of each e4m3 code (uint8 array) as fp64 (a lookup in the table of
    all 256 codes)."""
    return _E4M3_VALUES[np.asarray(codes, np.uint8)]


def _table(values):
    """(values, codes) of the non-negative finite codes of a format, ascending."""
    codes = np.arange(128, dtype=np.uint8)
    v = values[codes]
    ok = np.isfinite(v)
    order = np.argsort(v[ok], kind="stable")
    return v[ok][order], codes[ok][order]


def _encode_nearest(x, values, vmax):
    """Round values to the nearest value of a format whose non-negative codes
    0..127 hold ascending magnitudes (sign in bit 7), ties to the even code
    (the one with mantissa bit 0), magnitudes beyond vmax clamped to vmax."""
    vals, codes = _table(values)
    a = np.minimum(np.abs(np.asarray(x, F64)), vmax)
    hi = np.searchsorted(vals, a, side="left")      # first value >= a
    hi = np.minimum(hi, len(vals) - 1)
    lo = np.maximum(hi - 1, 0)
    exact = vals[hi] == a
    dlo = a - vals[lo]
    dhi = vals[hi] - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (codes[hi] % 2 == 0))
    c = np.where(exact | pick_hi, codes[hi], codes[lo])
    neg = np.signbit(np.asarray(x, F64))
    return (c | np.where(neg, 0x80, 0)).astype(np.uint8)


def e4m3_encode(x):
    """Round fp64/fp32 values to the nearest e4m3 value, ties to the even code
    (the one with mantissa bit 0), values beyond +-448 clamped to +-448."""
    return _encode_nearest(x, _E4M3_VALUES, 448.0)


# OCP e5m2 (KempnerForge README, "Features": FP8 in E4M3 and E5M2): 1 sign,
# 5 exponent (bias 15), 2 mantissa bits; exponent 0 holds the subnormals
# m/4 * 2^-14; exponent 31 holds infinity (mantissa 0) and NaN; the largest
# finite value is 57344.

def _e5m2_values():
    """Value of each of the 256 e5m2 codes (index = code), fp64."""
    c = np.arange(256, dtype=np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 2) & 31
    m = c & 3
    val = np.where(e == 0, m / 4.0 * 2.0 ** -14, (1.0 + m / 4.0) * np.exp2(e.astype(F64) - 15.0))
    val = np.where(e == 31, np.where(m == 0, np.inf, np.nan), val)
    return sign * val


_E5M2_VALUES = _e5m2_values()


def e5m2_decode(codes):
    """Value of each e5m2 code (uint8 array) as fp64."""
    return _E5M2_VALUES[np.asarray(codes, np.uint8)]


def e5m2_encode(x):
    """Round values to the nearest finite e5m2 value, ties to the even code,
    values beyond +-57344 clamped to +-57344."""
    return _encode_nearest(x, _E5M2_VALUES, 57344.0)


# the two formats: decoder, encoder, largest finite value
FP8_FORMATS = {"e4m3": (e4m3_decode, e4m3_encode, 448.0), "e5m2": (e5m2_decode, e5m2_encode, 57344.0)}


def quantize_rowwise(x, fmt="e4m3"):
    """Row-wise scaling: s_r = amax_r / vmax (fp32; 1 for an all-zero row;
    vmax = 448 for e4m3, 57344 for e5m2), q = fmt(x / s_r) with the division
    in fp32.  Returns (codes uint8, s fp32)."""
    _, encode, vmax = FP8_FORMATS[fmt]
    x32 = np.asarray(x, F32)
    amax = np.abs(x32).max(axis=1)
    s = np.where(amax > 0, (amax / np.float32(vmax)).astype(F32), np.float32(1.0)).astype(F32)
    q = encode((x32 / s[:, None]).astype(F32))
    return q, s


def quantize_tensorwise(x):
    """Tensor-wise scaling: one scale s = amax / 448 over every element (fp32;
    1 for an all-zero tensor), q = e4m3(x / s) with the division in fp32.
    Returns (codes uint8, s as an fp32 scalar)."""
    x32 = np.asarray(x, F32)
    amax = np.float32(np.abs(x32).max()) if x32.size else np.float32(0.0)
    s = np.float32(amax / np.float32(448.0)) if amax > 0 else np.float32(1.0)
    q = e4m3_encode((x32 / s).astype(F32))
    return q, s


def quantize_rowwise_transposed(w):
    """Row-wise quantisation along the first axis of each matrix: for
    w [G, R, C], codes [G, C, R] and scales [G, C], the codes of column c of
    w[g] stored as row c (its transpose), one scale per column:
    s[g, c] = amax_r |w[g, r, c]| / 448.  A product that reduces over R (the
    data gradient dX = dGU . W with W [2f, d]) then runs in the forward
    layout with the weight operand as rows (FP2: one scale per row along the
    reduction dimension)."""
    w = np.asarray(w, F32)
    G, R, C = w.shape
    codes = np.empty((G, C, R), np.uint8)
    scales = np.empty((G, C), F32)
    for g in range(G):
        codes[g], scales[g] = quantize_rowwise(w[g].T)
    return codes, scales


def grouped_gemm_fp8_nt(a_codes, a_scale, b_codes, b_scale, offsets, a_fmt="e4m3"):
    """C[m, n] = a_scale[m] * b_scale[g, n] * sum_k A[m, k] B[g, n, k] over the
    decoded codes (A in a_fmt, B in e4m3), for the rows m of group g; fp64."""
    A = FP8_FORMATS[a_fmt][0](a_codes)
    B = e4m3_decode(b_codes)
    G, N, _ = B.shape
    C = np.zeros((A.shape[0], N))
    for g in range(G):
        r0, r1 = int(offsets[g]), int(offsets[g + 1])
        if r1 > r0:
            C[r0:r1] = (A[r0:r1] @ B[g].T) * np.asarray(a_scale, F64)[r0:r1, None] * \
                np.asarray(b_scale, F64)[g][None, :]
    return C


# ----------------------------------------------------------------------------- fp8 layer
# The expert products of the layer in e4m3 (Apex-3 code page, "Run it
# yourself": the fp8_rowwise precision; KempnerForge README, "MoE roadmap":
# FP8 mixed precision).  Readings, where the pages name only the recipe:
#   - every product quantises both operands row-wise along its reduction
#     dimension, from the operands' current values (activations per row,
#     weights per output row in the forward, per reduction-dimension column for
#     the data gradients);
#   - an activation is quantised from its bf16 copy, the copy the bf16 layer
#     stores (H, the gate-weighted dY, dG | dU), so that the rounding to bf16
#     precedes the quantisation as it does on a device that keeps bf16
#     activations; dG | dU are formed from the bf16 copies of G and U, the
#     pre-activations the layer saves; the router stays fp32;
#   - weight gradients stay in the layer's own precision (exact here), the
#     row-wise recipe with high-precision weight gradients; or, with
#     ``fp8_wgrad``, they are e4m3 products whose operands are quantised along
#     their reduction dimension, the rows of one expert: one scale per
#     (expert, column) of dY~, H, dG | dU and the token rows.

def round_bf16(v):
    """The bf16 value a stored fp32 result takes: v rounded to fp32, then to
    the nearest bf16 (8 significand bits), ties to the even one (fp64 out)."""
    v32 = np.ascontiguousarray(np.asarray(v, F64).astype(F32))
    b = v32.view(np.uint32).astype(np.uint64)
    b = ((b + 0x7FFF + ((b >> 16) & 1)) >> 16) << 16
    return b.astype(np.uint32).view(F32).astype(F64)


def fp8_product(a, b, a_fmt="e4m3"):
    """a [M, K] times b [N, K]^T with each operand quantised row-wise along K
    (``quantize_rowwise``; a in a_fmt, b in e4m3) and the scaled product
    taken exactly (fp64)."""
    a = np.asarray(a, F64)
    qa, sa = quantize_rowwise(a, a_fmt)
    qb, sb = quantize_rowwise(b)
    return grouped_gemm_fp8_nt(qa, sa, qb[None], sb[None], np.array([0, a.shape[0]]), a_fmt)


def swiglu_ffn_fp8(z, w_gate, w_up, w_down, forced_h=None):
    """``swiglu_ffn`` with both products in e4m3: G | U = fp8(z) . fp8(W_g | W_u)^T,
    H = silu(G) U (fp64), Y = fp8(bf16(H)) . fp8(W_d)^T; ``forced_h`` replaces
    bf16(H) as the down product's input.  Returns (G, U, H, Y, Hb) like
    ``swiglu_ffn`` with H unrounded, plus the bf16 H the down product
    quantised."""
    f = w_gate.shape[0]
    GU = fp8_product(z, np.concatenate([w_gate, w_up], axis=0))
    G, U = GU[:, :f], GU[:, f:]
    H = silu(G) * U
    Hb = round_bf16(H) if forced_h is None else np.asarray(forced_h, F64)
    return G, U, H, fp8_product(Hb, w_down), Hb


def swiglu_ffn_backward_fp8(z, w_gate, w_up, w_down, G, U, H, dY, forced_dgu=None, grad_fmt="e4m3",
                            Hq=None):
    """``swiglu_ffn_backward`` with the two data gradients in e4m3:
    dH = fp8(bf16(dY)) . fp8 of W_d along its rows d (W_d^T quantised
    row-wise), dz = fp8(bf16(dG | dU)) . fp8 of W_g | W_u along 2f; the
    weight gradients are exact (fp64).  dG | dU, which the second product
    quantises, come from the pre-activations as the layer stores them (bf16),
    so that this quantisation sees the values a bf16 layer holds;
    ``forced_dgu`` replaces that bf16 copy as the second product's input.
    ``grad_fmt``: the format of the gradient operands (dY, dG | dU); the
    weights stay e4m3.  ``Hq`` (the bf16 H the forward's down product
    quantised) given: the weight gradients are e4m3 products too
    (``wgrad_fp8``: dW_d from bf16(dY) and Hq, dW_g | dW_u from the quantised
    dG | dU copy and z).  Same return values."""
    dH = fp8_product(round_bf16(dY), np.asarray(w_down, F64).T, grad_fmt)
    Gb, Ub = round_bf16(G), round_bf16(U)
    sg = 1.0 / (1.0 + np.exp(-Gb))
    dG = dH * Ub * sg * (1.0 + Gb * (1.0 - sg))
    dU = dH * (Gb * sg)
    w_gu = np.concatenate([w_gate, w_up], axis=0)
    dgu_b = round_bf16(np.concatenate([dG, dU], axis=1)) if forced_dgu is None else np.asarray(forced_dgu, F64)
    dz = fp8_product(dgu_b, w_gu.T, grad_fmt)
    if Hq is None:
        dW_d = dY.T @ H
        dW_g = dG.T @ z
        dW_u = dU.T @ z
    else:
        f = w_gate.shape[0]
        dW_d = wgrad_fp8(round_bf16(dY), Hq)
        dW_gu = wgrad_fp8(dgu_b, z)
        dW_g, dW_u = dW_gu[:f], dW_gu[f:]
    return dz, dW_g, dW_u, dW_d, dG, dU


def quantize_colwise(x, fmt="e4m3"):
    """Column-wise scaling over the rows of x [M, C]: s_c = amax_c / vmax (1
    for an all-zero column), q = fmt(x / s_c); the row-wise scheme applied to
    x^T.  Returns (codes [M, C], s [C])."""
    q, s = quantize_rowwise(np.asarray(x, F64).T, fmt)
    return q.T, s


def wgrad_fp8(a, b):
    """The weight gradient a^T b (a [M, N], b [M, K], reduction over the M
    rows) in e4m3: both operands quantised column-wise, i.e. row-wise along
    their reduction dimension (``quantize_colwise``), and the scaled product
    C[n, k] = s_a[n] s_b[k] sum_m q_a[m, n] q_b[m, k] taken exactly (fp64)."""
    qa, sa = quantize_colwise(a)
    qb, sb = quantize_colwise(b)
    return grouped_gemm_fp8_nt(qa.T, sa, qb.T[None], sb[None], np.array([0, qa.shape[1]]))
