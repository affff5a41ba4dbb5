"""Pins of the CPU oracle against things other than itself.

Each test checks the oracle against torch fp64 autograd, a brute force written
differently, a closed form, a special case that reduces to a textbook routine,
or numbers printed on the pages (tests/golden).  None of these tests needs a
GPU."""
import json
import os

import numpy as np
import pytest
import torch

from oracle import moe_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
F64 = np.float64


def _rand_layer(seed, T, d, E, k, f, Fs, score, renorm, bias=True, wr_std=0.5):
    g = np.random.default_rng(seed)
    x = g.standard_normal((T, d))
    wr = (g.standard_normal((E, d)) * wr_std).astype(np.float32)
    b = (g.uniform(-0.3, 0.3, E).astype(np.float32) if (bias and score == "sigmoid") else None)
    wgu = g.standard_normal((E, 2 * f, d)) / np.sqrt(d)
    wd = g.standard_normal((E, d, f)) / np.sqrt(f)
    if Fs:
        sgu = g.standard_normal((2 * Fs, d)) / np.sqrt(d)
        sd = g.standard_normal((d, Fs)) / np.sqrt(Fs)
    else:
        sgu = sd = None
    dy = g.standard_normal((T, d))
    return dict(x=x, w_router=wr, bias=b, w_gateup=wgu, w_down=wd, s_gateup=sgu, s_down=sd, dy=dy,
                k=k, score=score, renorm=renorm)


def _fwd(L, **kw):
    return O.forward(L["x"], L["w_router"], L["bias"], L["w_gateup"], L["w_down"], L["s_gateup"],
                     L["s_down"], top_k=L["k"], score=L["score"], renorm=L["renorm"], **kw)


def _bwd(L, fwd):
    return O.backward(L["x"], L["w_router"], L["w_gateup"], L["w_down"], L["s_gateup"], L["s_down"],
                      fwd, L["dy"], score=L["score"], renorm=L["renorm"])


def _rel(a, b):
    a = np.asarray(a, F64)
    b = np.asarray(b, F64)
    return np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300)


# --------------------------------------------------------------------------- independent reference
def _brute_select(keys32, k):
    """Top-k by an explicit python sort of (-key, index) tuples."""
    out = []
    for row in np.asarray(keys32, np.float32):
        order = sorted(range(len(row)), key=lambda e: (-float(row[e]), e))
        out.append(order[:k])
    return np.array(out, np.int32)


def _torch_keys(L):
    """Selection keys recomputed with torch (fp64 math, rounded like an fp32 router)."""
    x = torch.tensor(L["x"], dtype=torch.float64)
    wr = torch.tensor(L["w_router"], dtype=torch.float64)
    logits32 = (x @ wr.T).to(torch.float32)
    if L["score"] == "softmax":
        return logits32.numpy()
    s32 = torch.sigmoid(logits32.to(torch.float64)).to(torch.float32)
    if L["bias"] is not None:
        s32 = s32 + torch.tensor(L["bias"])
    return s32.numpy()


def _dense_masked_torch(L, mask_idx):
    """All E experts on all T tokens in torch fp64, masked by the selection and
    weighted by gates recomputed from the logits; returns y and a closure for
    autograd.  The selection is fixed (it is piecewise constant)."""
    T, d = L["x"].shape
    E = L["w_router"].shape[0]
    f = L["w_gateup"].shape[1] // 2
    t = {n: torch.tensor(np.asarray(L[n], F64), dtype=torch.float64, requires_grad=True)
         for n in ("x", "w_router", "w_gateup", "w_down")}
    if L["s_gateup"] is not None:
        for n in ("s_gateup", "s_down"):
            t[n] = torch.tensor(L[n], dtype=torch.float64, requires_grad=True)
    M = torch.zeros(T, E, dtype=torch.float64)
    M[torch.arange(T)[:, None], torch.tensor(mask_idx, dtype=torch.long)] = 1.0
    logits = t["x"] @ t["w_router"].T
    if L["score"] == "softmax":
        p = torch.softmax(logits, dim=1)
        g = M * p
        if L["renorm"]:
            g = g / g.sum(dim=1, keepdim=True)
    else:
        s = torch.sigmoid(logits)
        g = M * s
        g = g / g.sum(dim=1, keepdim=True)
    y = torch.zeros(T, d, dtype=torch.float64)
    for e in range(E):
        G = t["x"] @ t["w_gateup"][e, :f].T
        U = t["x"] @ t["w_gateup"][e, f:].T
        Y = (torch.nn.functional.silu(G) * U) @ t["w_down"][e].T
        y = y + g[:, e:e + 1] * Y
    if "s_gateup" in t:
        Fs = t["s_gateup"].shape[0] // 2
        Gs = t["x"] @ t["s_gateup"][:Fs].T
        Us = t["x"] @ t["s_gateup"][Fs:].T
        y = y + (torch.nn.functional.silu(Gs) * Us) @ t["s_down"].T
    return y, t


CASES = [
    # seed, T, d, E, k, f, Fs, score, renorm
    (1, 24, 16, 8, 2, 12, 0, "softmax", False),
    (2, 20, 16, 8, 3, 8, 0, "softmax", True),
    (3, 32, 16, 8, 4, 8, 8, "sigmoid", True),
    (4, 16, 8, 6, 6, 4, 4, "sigmoid", True),      # k == E
    (5, 17, 12, 5, 1, 8, 0, "sigmoid", True),     # k == 1
]


@pytest.mark.parametrize("case", CASES)
def test_p1_dense_masked_brute_force_forward(case):
    """Sparse oracle forward == all-experts dense compute masked by the selection."""
    L = _rand_layer(*case)
    fw = _fwd(L)
    sel = _brute_select(_torch_keys(L), L["k"])
    assert np.array_equal(fw["idx"], sel)
    y, _ = _dense_masked_torch(L, sel)
    assert _rel(fw["y"], y.detach().numpy()) < 1e-6


@pytest.mark.parametrize("case", CASES)
def test_p2_backward_matches_torch_autograd(case):
    """Hand-written oracle backward == torch fp64 autograd of the dense-masked layer."""
    L = _rand_layer(*case)
    fw = _fwd(L)
    bw = _bwd(L, fw)
    y, t = _dense_masked_torch(L, fw["idx"])
    (y * torch.tensor(L["dy"])).sum().backward()
    assert _rel(bw["dx"], t["x"].grad.numpy()) < 1e-6
    assert _rel(bw["d_w_gateup"], t["w_gateup"].grad.numpy()) < 1e-6
    assert _rel(bw["d_w_down"], t["w_down"].grad.numpy()) < 1e-6
    ref = t["w_router"].grad.numpy()
    # top-1 sigmoid: the exact gradient is zero and autograd leaves ~1e-16 noise
    assert np.linalg.norm(bw["d_w_router"] - ref) <= 1e-5 * np.linalg.norm(ref) + 1e-12
    if L["s_gateup"] is not None:
        assert _rel(bw["d_s_gateup"], t["s_gateup"].grad.numpy()) < 1e-6
        assert _rel(bw["d_s_down"], t["s_down"].grad.numpy()) < 1e-6


def test_p2_finite_differences_expert_weights():
    """Central differences of L = <dy, y> w.r.t. expert and shared weights.
    These perturbations leave the router untouched, so y is smooth in fp64."""
    L = _rand_layer(7, 12, 8, 4, 2, 6, 4, "sigmoid", True)
    fw = _fwd(L)
    bw = _bwd(L, fw)
    g = np.random.default_rng(0)
    h = 1e-6
    for name, grad in (("w_gateup", bw["d_w_gateup"]), ("w_down", bw["d_w_down"]),
                       ("s_gateup", bw["d_s_gateup"]), ("s_down", bw["d_s_down"])):
        for _ in range(6):
            i = tuple(int(g.integers(0, s)) for s in L[name].shape)
            Lp = dict(L); Lp[name] = L[name].copy(); Lp[name][i] += h
            Lm = dict(L); Lm[name] = L[name].copy(); Lm[name][i] -= h
            num = ((_fwd(Lp)["y"] - _fwd(Lm)["y"]) * L["dy"]).sum() / (2 * h)
            assert abs(num - grad[i]) <= 1e-6 * max(1.0, abs(num)), (name, i, num, grad[i])


def test_p3_single_expert_top1_equals_dense():
    """One expert with top-1 routing is the dense FFN it came from (Handbook 2.5)."""
    for score in ("softmax", "sigmoid"):
        L = _rand_layer(11, 16, 8, 1, 1, 12, 0, score, score == "sigmoid")
        fw = _fwd(L)
        assert np.all(fw["gate"] == 1.0)
        x = torch.tensor(L["x"])
        f = L["w_gateup"].shape[1] // 2
        W = torch.tensor(L["w_gateup"][0])
        dense = (torch.nn.functional.silu(x @ W[:f].T) * (x @ W[f:].T)) @ torch.tensor(L["w_down"][0]).T
        assert _rel(fw["y"], dense.numpy()) < 1e-13


def test_p4_single_expert_router_gets_no_gradient():
    """With one expert the router weight receives exactly zero gradient
    (Handbook 2.5: the ~32,770 zero-gradient parameters are the router)."""
    gold = json.load(open(os.path.join(GOLDEN, "handbook_param_count.json")))
    for score in ("softmax", "sigmoid"):
        L = _rand_layer(12, 16, 8, 1, 1, 12, 0, score, score == "sigmoid")
        fw = _fwd(L)
        bw = _bwd(L, fw)
        assert np.all(bw["d_logits"] == 0.0)
        assert np.all(bw["d_w_router"] == 0.0)
        # 16 layers x (1 expert x hidden 2048) router weights, all zero-gradient
        zero_router = gold["layers"] * 1 * gold["hidden_size"]
        assert zero_router <= gold["single_expert_zero_grad_params"] <= zero_router + gold["dense_zero_grad_params_max"]
    # sigmoid top-1 with many experts: the renormalised gate is exactly 1
    L = _rand_layer(13, 16, 8, 6, 1, 4, 0, "sigmoid", True)
    bw = _bwd(L, _fwd(L))
    assert np.all(bw["d_logits"] == 0.0)


def test_p5_granularity_identity():
    """A dense SwiGLU of width F cut into E experts of width F/E: routing every
    token to every expert and summing the expert outputs gives the dense FFN
    (Handbook 2.5: eight 1024-wide experts == the 8192-wide dense layer)."""
    g = np.random.default_rng(5)
    T, d, E, fe = 20, 16, 4, 6
    F = E * fe
    Wg = g.standard_normal((F, d)); Wu = g.standard_normal((F, d)); Wd = g.standard_normal((d, F))
    wgu = np.stack([np.concatenate([Wg[e * fe:(e + 1) * fe], Wu[e * fe:(e + 1) * fe]]) for e in range(E)])
    wd = np.stack([Wd[:, e * fe:(e + 1) * fe] for e in range(E)])
    x = g.standard_normal((T, d))
    wr = g.standard_normal((E, d)).astype(np.float32)
    fw = O.forward(x, wr, None, wgu, wd, top_k=E, score="softmax", renorm=False)
    summed = fw["y_perm"][fw["pos"].reshape(T, E)].sum(axis=1)
    xt = torch.tensor(x)
    dense = (torch.nn.functional.silu(xt @ torch.tensor(Wg).T) * (xt @ torch.tensor(Wu).T)) @ torch.tensor(Wd).T
    assert _rel(summed, dense.numpy()) < 1e-13


def test_p5_handbook_parameter_accounting():
    """Parameter counts printed in the Handbook (sections 2.4 and 2.5)."""
    gold = json.load(open(os.path.join(GOLDEN, "handbook_param_count.json")))
    d, fe, F, k, E, Lyr = (gold[n] for n in ("hidden_size", "moe_ffn_hidden_size", "dense_ffn_hidden_size",
                                             "router_topk", "num_experts", "layers"))
    per_expert = O.expert_parameter_count(d, fe)
    assert per_expert == 6_291_456
    assert k * per_expert == O.expert_parameter_count(d, F) == 50_331_648
    dense_ffn = Lyr * O.expert_parameter_count(d, F)
    router = Lyr * E * d
    rest = gold["dense_total_params_B"] * 1e9 - dense_ffn
    active = rest + Lyr * k * per_expert + router
    total = rest + Lyr * E * per_expert + router
    assert abs(active / 1e9 - gold["moe_active_params_B"]) < 0.0015
    assert abs(total / 1e9 - gold["moe_total_params_B"]) < 0.006


@pytest.mark.parametrize("case", CASES)
def test_p6_p7_p11_permutation_invariants(case):
    L = _rand_layer(*case)
    fw = _fwd(L)
    T, k, E = L["x"].shape[0], L["k"], L["w_router"].shape[0]
    A = T * k
    assert fw["counts"].sum() == A and fw["offsets"][-1] == A and fw["offsets"][0] == 0
    assert np.array_equal(fw["src"][fw["pos"]], np.arange(A))
    # brute-force stable grouping: per expert, assignments in increasing order
    flat = fw["idx"].reshape(-1)
    expect = [a for e in range(E) for a in range(A) if flat[a] == e]
    assert np.array_equal(fw["src"], np.array(expect))
    for e in range(E):
        assert fw["counts"][e] == fw["offsets"][e + 1] - fw["offsets"][e] == int((flat == e).sum())
    # permuted rows are copies of the token rows; unpermute-combine with
    # renormalised weights gives x back
    xp = fw["x_perm"]
    assert np.array_equal(xp[fw["pos"]], np.repeat(L["x"], k, axis=0))
    w = np.full((T, k), 1.0 / k)
    back = sum(w[:, j:j + 1] * xp[fw["pos"].reshape(T, k)[:, j]] for j in range(k))
    assert _rel(back, L["x"]) < 1e-15


def test_p8_sigmoid_gates_renormalise():
    L = _rand_layer(21, 64, 16, 16, 4, 4, 0, "sigmoid", True)
    g = _fwd(L)["gate"].astype(F64)
    assert np.all(np.abs(g.sum(axis=1) - 1.0) < 4 * 2.0 ** -24 * 4)


def test_p9_bias_selects_but_does_not_scale():
    L = _rand_layer(22, 64, 16, 12, 3, 4, 0, "sigmoid", True)
    fw = _fwd(L)
    s = torch.sigmoid(torch.tensor(fw["logits"], dtype=torch.float64)).to(torch.float32).numpy().astype(F64)
    picked = np.take_along_axis(s, fw["idx"], axis=1)
    assert np.array_equal(fw["gate"], (picked / picked.sum(axis=1, keepdims=True)).astype(np.float32))
    # a +10 bias on a fixed set S of size k forces I_t = S for every token
    S = [7, 2, 9]
    L2 = dict(L); L2["bias"] = L["bias"].copy(); L2["bias"][S] += 10.0
    fw2 = _fwd(L2)
    assert all(set(r) == set(S) for r in fw2["idx"].tolist())
    s_S = s[:, S]
    for t in range(s.shape[0]):
        for j, e in enumerate(fw2["idx"][t]):
            assert fw2["gate"][t, j] == np.float32(s[t, e] / s_S[t].sum())
    # the bias changes the selection on the unbiased layer
    assert not np.array_equal(fw["idx"], fw2["idx"])


def test_p10_topk_brute_force_with_ties():
    g = np.random.default_rng(3)
    keys = g.integers(-3, 4, size=(200, 9)).astype(np.float32)   # many exact ties
    keys[0, :] = 0.0
    keys[1, :] = -0.0
    keys[1, 4] = 0.0
    for k in (1, 2, 5, 9):
        idx, margin = O.select_topk(keys, k)
        assert np.array_equal(idx, _brute_select(keys, k))
        if k == 9:
            assert np.all(np.isinf(margin))
            assert all(sorted(r) == list(range(9)) for r in idx.tolist())
    # the sigmoid scores agree with an independent library evaluation
    l = g.standard_normal((50, 7)).astype(np.float32) * 4
    s = O.router_scores(l, "sigmoid")
    ref = torch.sigmoid(torch.tensor(l, dtype=torch.float64)).to(torch.float32).numpy()
    assert np.array_equal(s, ref)
    p = O.router_scores(l, "softmax")
    refp = torch.softmax(torch.tensor(l, dtype=torch.float64), dim=1).to(torch.float32).numpy()
    assert np.max(np.abs(p.astype(F64) - refp)) <= 2.0 ** -24


def test_p13_softmax_backward_is_the_softmax_jacobian():
    """k = E, no renormalisation: dl = p * (dp - <p, dp>), checked against torch autograd."""
    g = np.random.default_rng(8)
    l = g.standard_normal((10, 6)).astype(np.float32)
    p32 = O.router_scores(l, "softmax")
    idx, _ = O.select_topk(l, 6)
    dg = g.standard_normal((10, 6))
    dl = O.router_backward(dg, p32, idx, "softmax", False)
    pt = torch.tensor(p32.astype(F64), requires_grad=True)
    # the Jacobian of softmax at p: d p_i / d l_j = p_i (delta_ij - p_j)
    J = torch.diag_embed(pt) - pt[:, :, None] * pt[:, None, :]
    dp = np.zeros((10, 6)); np.put_along_axis(dp, idx.astype(np.int64), dg, axis=1)
    ref = torch.einsum("ti,tij->tj", torch.tensor(dp), J).detach().numpy()
    assert _rel(dl, ref) < 1e-14
    # and against autograd through torch.softmax at fp64 logits
    lt = torch.tensor(l.astype(F64), requires_grad=True)
    (torch.softmax(lt, 1) * torch.tensor(dp)).sum().backward()
    assert _rel(dl, lt.grad.numpy()) < 1e-6


# --------------------------------------------------------------------------- router training terms
def _torch_terms(l32, idx, counts, k, score, aux, seq_aux, zc, seq_len):
    """The three losses written directly in torch fp64 (autograd gives the
    reference dlogits): switch-style balance, per-sequence balance, z-loss."""
    l = torch.tensor(l32.astype(F64), requires_grad=True)
    T, E = l.shape
    if score == "softmax":
        q = torch.softmax(l, dim=1)
    else:
        s = torch.sigmoid(l)
        q = s / s.sum(dim=1, keepdim=True)
    f = torch.tensor(np.asarray(counts, F64)) / (T * k)
    L_aux = aux * E * (f * q.mean(dim=0)).sum()
    S = seq_len or T
    n = T // S
    L_seq = 0.0
    for sq in range(n):
        onehot = torch.zeros(S, E, dtype=torch.float64)
        onehot.scatter_(1, torch.tensor(idx[sq * S:(sq + 1) * S].astype(np.int64)), 1.0)
        fs = onehot.sum(dim=0) * E / (k * S)
        L_seq = L_seq + (fs * q[sq * S:(sq + 1) * S].mean(dim=0)).sum()
    L_seq = seq_aux * L_seq / n
    L_z = zc * (torch.logsumexp(l, dim=1) ** 2).mean()
    total = L_aux + L_seq + L_z
    total.backward()
    return float(L_aux), float(L_seq), float(L_z), l.grad.numpy()


@pytest.mark.parametrize("score", ["softmax", "sigmoid"])
def test_router_terms_match_torch_autograd(score):
    g = np.random.default_rng(21)
    T, E, k, S = 96, 8, 2, 32
    l = (g.standard_normal((T, E)) * 1.5).astype(np.float32)
    idx, _ = O.select_topk(l, k)
    counts = np.bincount(idx.reshape(-1), minlength=E)
    terms = dict(aux_coeff=1e-3, seq_aux_coeff=2e-3, z_coeff=3e-3, seq_len=S)
    vals, dl = O.router_terms(l, idx, counts, k, score, terms)
    ra, rs, rz, rg = _torch_terms(l, idx, counts, k, score, 1e-3, 2e-3, 3e-3, S)
    assert abs(vals["aux"] - ra) <= 1e-15 + 1e-13 * abs(ra)
    assert abs(vals["seq_aux"] - rs) <= 1e-15 + 1e-13 * abs(rs)
    assert abs(vals["z"] - rz) <= 1e-15 + 1e-13 * abs(rz)
    assert _rel(dl, rg) < 1e-12


def test_router_terms_single_expert_balance_loss_is_one():
    """One expert (E = k = 1): both balance losses equal their coefficient
    exactly (the Handbook's load balance loss of exactly 1), with zero
    gradient; the z-loss is mean(l^2) with gradient 2 l / T."""
    g = np.random.default_rng(22)
    l = g.standard_normal((40, 1)).astype(np.float32)
    idx = np.zeros((40, 1), np.int32)
    for score in ("softmax", "sigmoid"):
        v, dl = O.aux_loss(l, [40], 1, score, 1.0)
        assert v == 1.0 and np.all(dl == 0.0)
        v, dl = O.seq_aux_loss(l, idx, 1, score, 1.0, 8)
        assert abs(v - 1.0) < 1e-15 and np.all(dl == 0.0)
    v, dl = O.z_loss(l, 1.0)
    l64 = l.astype(F64)
    assert abs(v - float((l64 ** 2).mean())) < 1e-14
    assert np.max(np.abs(dl - 2.0 * l64 / 40)) < 1e-15


def test_router_terms_closed_forms():
    """Uniform routing and perfectly balanced loads give a balance loss equal to
    its coefficient; equal logits c give z = (c + ln E)^2 and a gradient of
    2 (c + ln E) / (T E) on every logit."""
    T, E, k = 64, 8, 2
    l = np.full((T, E), 0.75, np.float32)
    counts = np.full(E, T * k // E)
    for score in ("softmax", "sigmoid"):
        v, _ = O.aux_loss(l, counts, k, score, 1.0)
        assert abs(v - 1.0) < 1e-14
    c = F64(np.float32(0.75))
    v, dl = O.z_loss(l, 1.0)
    assert abs(v - (c + np.log(E)) ** 2) < 1e-13
    assert np.max(np.abs(dl - 2.0 * (c + np.log(E)) / (T * E))) < 1e-15


def test_bias_update_moves_toward_balance():
    """The proportional bias update (reading of the Apex-3 page's
    router_bias_update=proportional) pinned by what "proportional to the
    relative load error" fixes, without writing the rule out again:
    balanced loads leave the bias unchanged; the step is linear in the load
    error (doubling every expert's excess load doubles every step, exactly:
    a power-of-two scaling); it depends on the loads only relative to the
    mean (T and the counts scaled together give the same step); the steps
    sum to zero (the loads always sum to T k); an expert with no load moves
    up by the rate and one at twice the mean load down by the rate; and the
    step grows with the overload (monotone)."""
    T, k, E, rate = 1024, 4, 8, 0.01
    m = T * k // E
    b = np.linspace(-0.1, 0.1, E).astype(np.float32)
    z = np.zeros(E, np.float32)
    # balanced loads: no change at all
    assert np.array_equal(O.bias_update(b, np.full(E, m), T, k, rate), b)
    # linear in the load error (Sum of the error is zero, so both are valid loads)
    err = np.array([256, -128, 64, -64, 0, -32, -32, -64])
    assert err.sum() == 0
    s1 = O.bias_update(z, m + err, T, k, rate)
    s2 = O.bias_update(z, m + 2 * err, T, k, rate)
    assert np.array_equal(s2, 2 * s1)
    # relative loads only: T and the counts doubled together, same step
    assert np.array_equal(O.bias_update(b, m + err, T, k, rate), O.bias_update(b, 2 * (m + err), 2 * T, k, rate))
    # the steps balance out
    assert abs(float(s1.astype(F64).sum())) <= E * 2.0 ** -24 * float(np.abs(s1).max())
    # no load: up by the rate; twice the mean: down by the rate
    c = np.array([0, 2 * m, m, m, m, m, m, m])
    s = O.bias_update(z, c, T, k, rate)
    assert s[0] == np.float32(rate) and s[1] == -np.float32(rate) and np.all(s[2:] == 0)
    # monotone: more load, lower bias
    c = np.array([1024, 768, 640, 512, 384, 320, 256, 192])
    assert c.sum() == T * k
    nb = O.bias_update(z, c, T, k, rate)
    assert np.all(np.diff(nb.astype(F64)) > 0)


def test_balance_loss_values_independent_of_their_formula():
    """Values of the balance losses fixed without retyping them: the
    per-sequence loss over one sequence equals the batch loss (both measure
    the same loads); over n copies of one sequence it equals that sequence's
    loss; and with every token on expert 0 (k = 1) and a router certain of it
    the batch loss is coeff * E (the most unbalanced case)."""
    g = np.random.default_rng(23)
    T, E, k = 64, 8, 2
    l = (g.standard_normal((T, E)) * 1.5).astype(np.float32)
    idx, _ = O.select_topk(l, k)
    counts = np.bincount(idx.reshape(-1), minlength=E)
    for score in ("softmax", "sigmoid"):
        va, _ = O.aux_loss(l, counts, k, score, 1.0)
        vs, _ = O.seq_aux_loss(l, idx, k, score, 1.0, T)
        assert abs(va - vs) <= 1e-14 * abs(va)
        l3, i3 = np.tile(l, (3, 1)), np.tile(idx, (3, 1))
        v3, _ = O.seq_aux_loss(l3, i3, k, score, 1.0, T)
        assert abs(v3 - vs) <= 1e-14 * abs(vs)
    l1 = np.zeros((T, E), np.float32)
    l1[:, 0] = 60.0
    v, _ = O.aux_loss(l1, np.array([T] + [0] * (E - 1)), 1, "softmax", 1.0)
    assert abs(v - E) <= 1e-12


# --------------------------------------------------------------------------- fp8 (e4m3)
def test_e4m3_decode_table_against_the_format():
    """Every code against the format written out by hand: the named values of
    the OCP e4m3 definition."""
    v = O.e4m3_decode(np.arange(256, dtype=np.uint8))
    assert v[0x00] == 0.0 and v[0x80] == 0.0 and np.signbit(v[0x80])
    assert v[0x01] == 2.0 ** -9                 # smallest subnormal
    assert v[0x07] == 7 * 2.0 ** -9             # largest subnormal
    assert v[0x08] == 2.0 ** -6                 # smallest normal
    assert v[0x38] == 1.0 and v[0xb8] == -1.0
    assert v[0x7e] == 448.0 and v[0xfe] == -448.0
    assert np.isnan(v[0x7f]) and np.isnan(v[0xff])
    finite = v[~np.isnan(v)]
    assert len(finite) == 254 and len(np.unique(finite)) == 253     # +0 and -0 compare equal


def test_e4m3_encode_rounding():
    vals = O.e4m3_decode(np.arange(0x7f, dtype=np.uint8))
    # every finite value encodes to itself
    assert np.array_equal(O.e4m3_decode(O.e4m3_encode(vals)), vals)
    # midpoints go to the even code; a hair either side goes to the nearest
    lo, hi = vals[:-1], vals[1:]
    mid = (lo + hi) / 2
    enc = O.e4m3_encode(mid)
    codes_lo = np.arange(0x7e, dtype=np.uint8)
    want = np.where(codes_lo % 2 == 0, codes_lo, codes_lo + 1)
    assert np.array_equal(enc, want)
    assert np.array_equal(O.e4m3_encode(np.nextafter(mid, 0)), codes_lo)
    assert np.array_equal(O.e4m3_encode(np.nextafter(mid, np.inf)), codes_lo + 1)
    # clamping and sign
    assert O.e4m3_encode([1000.0])[0] == 0x7e and O.e4m3_encode([-1000.0])[0] == 0xfe
    assert O.e4m3_encode([-1.0])[0] == 0xb8


def test_fp8_rowwise_gemm_factorises():
    """The scaled product equals the product of the dequantised operands, and
    quantisation error per element is at most half a step of e4m3 (relative
    2^-4 of the value, or 2^-10 of the row scale in the subnormal range)."""
    g = np.random.default_rng(31)
    x = g.standard_normal((40, 64)).astype(np.float32)
    w = (g.standard_normal((3, 24, 64)) / 8).astype(np.float32)
    qx, sx = O.quantize_rowwise(x)
    qw, sw = O.quantize_rowwise(w.reshape(-1, 64))
    qw = qw.reshape(3, 24, 64)
    sw = sw.reshape(3, 24)
    off = np.array([0, 10, 10, 40])
    C = O.grouped_gemm_fp8_nt(qx, sx, qw, sw, off)
    xd = O.e4m3_decode(qx) * sx[:, None]
    wd = O.e4m3_decode(qw) * sw[:, :, None]
    ref = np.zeros_like(C)
    ref[0:10] = xd[0:10] @ wd[0].T
    ref[10:40] = xd[10:40] @ wd[2].T
    assert np.max(np.abs(C - ref)) <= 1e-12 * np.max(np.abs(ref))
    assert np.all(C[0:10].shape == (10, 24))
    err = np.abs(xd - x.astype(np.float64))
    bound = np.maximum(np.abs(x) * 2.0 ** -4, sx[:, None].astype(np.float64) * 2.0 ** -10)
    assert np.all(err <= bound * (1 + 1e-12))
    # the row maximum maps to 448 exactly
    assert np.all(np.max(np.abs(O.e4m3_decode(qx)), axis=1) == 448.0)


def test_fp8_transposed_quantisation():
    """Codes [G, C, R] of w [G, R, C] quantised along R: every code decodes,
    times its column's scale, to within half an e4m3 step of w[g, r, c] (so
    the transposed index mapping is right), every column's maximum maps to
    exactly 448, an all-zero column gets scale 1 and zero codes, and the
    data-gradient product dX = A . W computed in the forward layout with
    these codes equals the product of the dequantised operands."""
    g = np.random.default_rng(37)
    w = (g.standard_normal((2, 48, 16)) * np.exp(g.standard_normal(16))[None, None, :]).astype(np.float32)
    w[1, :, 5] = 0.0
    q, s = O.quantize_rowwise_transposed(w)
    assert q.shape == (2, 16, 48) and s.shape == (2, 16)
    wd = O.e4m3_decode(q) * s[:, :, None]                  # [G, C, R]
    ref = np.swapaxes(w, 1, 2).astype(np.float64)
    bound = np.maximum(np.abs(ref) * 2.0 ** -4, s[:, :, None].astype(np.float64) * 2.0 ** -10)
    assert np.all(np.abs(wd - ref) <= bound * (1 + 1e-12))
    nz = np.ones((2, 16), bool)
    nz[1, 5] = False
    assert np.all(np.max(np.abs(O.e4m3_decode(q)), axis=2)[nz] == 448.0)
    assert s[1, 5] == 1.0 and np.all(q[1, 5] == 0)
    # A [M, R] quantised row-wise, W as [G, C, R] rows: C[m, c] = sum_r A[m, r] W[g, r, c]
    a = g.standard_normal((30, 48)).astype(np.float32)
    qa, sa = O.quantize_rowwise(a)
    off = np.array([0, 12, 30])
    C = O.grouped_gemm_fp8_nt(qa, sa, q, s, off)
    ad = O.e4m3_decode(qa) * sa[:, None]
    exp = np.concatenate([ad[0:12] @ np.swapaxes(wd[0], 0, 1), ad[12:30] @ np.swapaxes(wd[1], 0, 1)])
    assert np.max(np.abs(C - exp)) <= 1e-12 * np.max(np.abs(exp))


def test_e4m3_encode_matches_brute_force_nearest():
    """Random values against a nearest-value search over all finite codes
    written independently (ties to the even code)."""
    g = np.random.default_rng(32)
    x = np.concatenate([g.standard_normal(3000) * 40, g.standard_normal(1000) * 0.01])
    codes = np.arange(0x7f, dtype=np.uint8)
    table = O.e4m3_decode(codes)
    for v in x:
        a = min(abs(v), 448.0)
        d = np.abs(table - a)
        best = np.where(d == d.min())[0]
        c = best[0] if len(best) == 1 else [b for b in best if b % 2 == 0][0]
        want = c | (0x80 if v < 0 else 0)
        assert O.e4m3_encode([v])[0] == want, v


def test_fp8_tensorwise_quantisation():
    """One scale for the whole tensor: the largest magnitude maps to 448
    exactly, every element is reproduced within half an e4m3 step, a
    one-row tensor quantises as the row-wise scheme does, a power-of-two
    rescaling of x rescales s and leaves the codes unchanged, and an all-zero
    tensor gets s = 1 and zero codes."""
    g = np.random.default_rng(5)
    x = (g.standard_normal((40, 96)) * np.exp(g.uniform(-3, 3, (40, 1)))).astype(np.float32)
    q, s = O.quantize_tensorwise(x)
    assert s.dtype == np.float32 and q.shape == x.shape
    v = O.e4m3_decode(q)
    assert np.max(np.abs(v)) == 448.0
    i = np.unravel_index(np.argmax(np.abs(x)), x.shape)
    assert abs(v[i]) == 448.0
    # half a step: 2^-4 relative for normal values, 2^-10 absolute in the
    # subnormal range (values below 2^-6), both in units of s, plus the fp32
    # rounding of the quotient
    y = x.astype(np.float64) / np.float64(s)
    err = np.abs(v - y)
    assert np.all(err <= np.maximum(np.abs(y) * 2.0 ** -4, 2.0 ** -10) * (1 + 1e-6))
    q1, s1 = O.quantize_tensorwise(x[3:4])
    qr, sr = O.quantize_rowwise(x[3:4])
    assert s1 == sr[0] and np.array_equal(q1, qr)
    q2, s2 = O.quantize_tensorwise(x * np.float32(8.0))
    assert s2 == s * np.float32(8.0) and np.array_equal(q2, q)
    qz, sz = O.quantize_tensorwise(np.zeros((3, 64), np.float32))
    assert sz == 1.0 and not qz.any()


# --------------------------------------------------------------------------- fp8 layer
def _e4m3_grid(g, R, C, p, cols=False):
    """[R, C] values on the e4m3 grid times 2^-p, every row's largest magnitude
    exactly 448 * 2^-p (with ``cols`` every column's too), so that row-wise
    quantisation (of the matrix, and with ``cols`` of its transpose) is exact:
    scale 2^-p, codes equal to the values."""
    codes = g.integers(0, 0x7e, size=(R, C)).astype(np.uint8)       # 0 .. 416
    m = O.e4m3_decode(codes) * np.where(g.random((R, C)) < 0.5, -1.0, 1.0)
    r = np.arange(R)
    m[r, r % C] = 448.0 * np.where(r % 2, -1.0, 1.0)
    if cols:
        c = np.arange(C)
        m[c % R, c] = 448.0
    return m * 2.0 ** -p


def _grid_layer(seed, T, d, E, k, f, Fs, score, renorm, one_hot=False):
    """A layer on the e4m3 grid.  one_hot: each token row has one nonzero
    element (448 * 2^-7), so that every pre-activation is one product of two
    e4m3 values (at most 8 significant bits): exact in bf16."""
    g = np.random.default_rng(seed)
    L = _rand_layer(seed, T, d, E, k, f, Fs, score, renorm)
    L["x"] = _e4m3_grid(g, T, d, 7)
    if one_hot:
        L["x"] = np.zeros((T, d))
        L["x"][np.arange(T), g.integers(0, d, T)] = 448.0 * 2.0 ** -7
    L["w_gateup"] = np.stack([_e4m3_grid(g, 2 * f, d, 10, cols=True) for _ in range(E)])
    L["w_down"] = np.stack([_e4m3_grid(g, d, f, 10, cols=True) for _ in range(E)])
    if Fs:
        L["s_gateup"] = _e4m3_grid(g, 2 * Fs, d, 10, cols=True)
        L["s_down"] = _e4m3_grid(g, d, Fs, 10, cols=True)
    L["dy"] = _e4m3_grid(g, T, d, 6)
    return L


def test_fp8_product_exact_on_the_grid_and_bounded_off_it():
    """fp8_product equals the exact product when both operands are on the
    e4m3 grid with row maxima 448 * 2^-p, and off the grid stays within the
    half-step bound: each quantised element is within 2^-4 of its value
    relative (normal range) plus half the smallest subnormal step."""
    g = np.random.default_rng(71)
    a = _e4m3_grid(g, 40, 96, 5)
    b = _e4m3_grid(g, 24, 96, 9)
    assert np.array_equal(O.fp8_product(a, b), a @ b.T)
    a = g.standard_normal((40, 96))
    b = g.standard_normal((24, 96))
    sa = np.abs(a).max(1) / 448.0
    sb = np.abs(b).max(1) / 448.0
    ea = np.abs(a) * 2.0 ** -4 + sa[:, None] * 2.0 ** -10
    eb = np.abs(b) * 2.0 ** -4 + sb[:, None] * 2.0 ** -10
    bound = ea @ np.abs(b).T + np.abs(a) @ eb.T + ea @ eb.T
    err = np.abs(O.fp8_product(a, b) - a @ b.T)
    assert np.all(err <= bound * (1 + 1e-6))
    assert err.max() > 0


def test_round_bf16_against_the_format():
    """round_bf16: exact bf16 values stay, the midpoint between two bf16
    neighbours goes to the one with an even last significand bit, one fp32
    ulp either side of it goes to the nearer; fp64 input is rounded to fp32
    first."""
    one, nxt = 1.0, 1.0 + 2.0 ** -7                       # neighbours; 1.0 has the even bit
    assert O.round_bf16([one, nxt, -nxt, 0.0])[1] == nxt
    mid = 1.0 + 2.0 ** -8
    assert O.round_bf16([mid])[0] == one
    assert O.round_bf16([mid + 2.0 ** -23])[0] == nxt
    assert O.round_bf16([mid - 2.0 ** -23])[0] == one
    mid2 = nxt + 2.0 ** -8                                 # between nxt (odd) and 1 + 2^-6 (even)
    assert O.round_bf16([mid2])[0] == 1.0 + 2.0 ** -6
    # within half an fp32 ulp below the midpoint: fp32 rounding lands on it first
    assert O.round_bf16([mid2 - 2.0 ** -26])[0] == 1.0 + 2.0 ** -6
    v = np.random.default_rng(3).standard_normal(1000) * 1e3
    r = O.round_bf16(v)
    assert np.all(np.abs(r - v) <= np.abs(v) * 2.0 ** -8 * (1 + 1e-6))
    bits = r.astype(np.float32).view(np.uint32)
    assert not np.any(bits & 0xFFFF)


@pytest.mark.parametrize("score,Fs,one_hot", [("softmax", 8, False), ("sigmoid", 0, False),
                                              ("softmax", 8, True), ("sigmoid", 0, True)])
def test_fp8_layer_exact_on_the_e4m3_grid(score, Fs, one_hot):
    """Tokens and weights on the e4m3 grid (row maxima 448 * 2^-p): the fp8
    layer's gate/up pre-activations equal the exact layer's bit for bit, and
    so do its down outputs when the down products take a bf16 H that is on the
    grid (forced).  With one-hot token rows (pre-activations exact in bf16),
    top-1 routing (gate exactly 1) and dy on the grid, the down data gradient
    is exact too: dG | dU and dW_down equal the exact backward's."""
    T, d, E, k, f = 24, 48, 4, 1, 32
    L = _grid_layer(5, T, d, E, k, f, Fs, score, True, one_hot)
    ex = _fwd(L)
    g = np.random.default_rng(9)
    fh = _e4m3_grid(g, T * k, f, 3)
    fsh = _e4m3_grid(g, T, Fs, 3) if Fs else None
    f8 = _fwd(L, fp8=True, forced_h=fh, forced_s_h=fsh)
    assert np.array_equal(f8["idx"], ex["idx"])
    assert np.array_equal(f8["preact"], ex["preact"])
    assert np.array_equal(f8["h"], ex["h"])
    for e in range(E):
        r0, r1 = ex["offsets"][e], ex["offsets"][e + 1]
        assert np.array_equal(f8["y_perm"][r0:r1], fh[r0:r1] @ L["w_down"][e].T)
    if Fs:
        assert np.array_equal(f8["s_preact"], ex["s_preact"])
        assert np.array_equal(f8["ys"], fsh @ L["s_down"].T)
    assert np.all(ex["gate"] == 1.0)
    if not one_hot:
        return
    assert np.array_equal(O.round_bf16(ex["preact"]), ex["preact"])
    b_ex = _bwd(L, ex)
    b_8 = O.backward(L["x"], L["w_router"], L["w_gateup"], L["w_down"], L["s_gateup"], L["s_down"],
                     f8, L["dy"], score=L["score"], renorm=L["renorm"], fp8=True)
    assert np.array_equal(b_8["dgu"], b_ex["dgu"])
    assert np.array_equal(b_8["d_w_down"][:, :, :], b_ex["d_w_down"])
    # a forced dG | dU on the grid: the gate/up data gradient is its exact
    # product with W_g | W_u (every column of which is on the grid too)
    fd = _e4m3_grid(g, T * k, 2 * f, 4)
    fsd = _e4m3_grid(g, T, 2 * Fs, 4) if Fs else None
    b_f = O.backward(L["x"], L["w_router"], L["w_gateup"], L["w_down"], L["s_gateup"], L["s_down"],
                     f8, L["dy"], score=L["score"], renorm=L["renorm"], fp8=True, forced_dgu=fd,
                     forced_s_dgu=fsd)
    assert np.array_equal(b_f["dgu"], b_8["dgu"])
    for e in range(E):
        r0, r1 = ex["offsets"][e], ex["offsets"][e + 1]
        assert np.array_equal(b_f["dx_perm"][r0:r1], fd[r0:r1] @ L["w_gateup"][e])
    if Fs:
        assert np.array_equal(b_f["dx_shared"], fsd @ L["s_gateup"])


def test_fp8_layer_power_of_two_equivariance():
    """Scaling W_down (routed and shared) by 2^3 scales y exactly by 2^3, and
    scaling dy by 2^-2 scales dx and every weight gradient exactly by 2^-2:
    each quantisation scale follows its operand, so a dropped or misplaced
    scale breaks the identity (random layer, off the grid)."""
    L = _rand_layer(11, 40, 32, 6, 2, 16, 16, "sigmoid", True)
    f1 = _fwd(L, fp8=True)
    L2 = dict(L, w_down=L["w_down"] * 8.0, s_down=L["s_down"] * 8.0)
    f2 = _fwd(L2, fp8=True)
    assert np.array_equal(f2["y"], 8.0 * f1["y"])
    b1 = O.backward(L["x"], L["w_router"], L["w_gateup"], L["w_down"], L["s_gateup"], L["s_down"],
                    f1, L["dy"], score=L["score"], renorm=L["renorm"], fp8=True)
    b2 = O.backward(L["x"], L["w_router"], L["w_gateup"], L["w_down"], L["s_gateup"], L["s_down"],
                    f1, L["dy"] * 0.25, score=L["score"], renorm=L["renorm"], fp8=True)
    for key in ("dx", "d_w_gateup", "d_w_down", "d_s_gateup", "d_s_down", "d_w_router"):
        assert np.array_equal(b2[key], 0.25 * b1[key]), key


@pytest.mark.parametrize("case", CASES[:4])
def test_fp8_layer_close_to_the_exact_layer(case):
    """Off the grid the fp8 layer is the exact layer up to e4m3 rounding: y, dx
    and the weight gradients within a few per cent (rel-L2) of the exact
    layer, and not equal to it.  A transposed operand, a wrong expert's
    weights or a lost term would be off by order one."""
    L = _rand_layer(*case)
    ex = _fwd(L)
    f8 = _fwd(L, fp8=True, forced_idx=ex["idx"])
    b_ex = _bwd(L, ex)
    b_8 = O.backward(L["x"], L["w_router"], L["w_gateup"], L["w_down"], L["s_gateup"], L["s_down"],
                     f8, L["dy"], score=L["score"], renorm=L["renorm"], fp8=True)
    checks = [(f8["y"], ex["y"]), (b_8["dx"], b_ex["dx"]), (b_8["d_w_gateup"], b_ex["d_w_gateup"]),
              (b_8["d_w_down"], b_ex["d_w_down"])]
    if L["s_gateup"] is not None:
        checks += [(b_8["d_s_gateup"], b_ex["d_s_gateup"]), (b_8["d_s_down"], b_ex["d_s_down"])]
    for got, want in checks:
        assert 1e-4 < _rel(got, want) < 0.08, _rel(got, want)


def test_forced_gate_replaces_the_gates():
    """forward's forced_gate: doubling every gate doubles the routed output
    exactly (a layer without shared experts), and the routing stays."""
    L = _rand_layer(13, 30, 16, 6, 2, 8, 0, "sigmoid", True)
    f1 = _fwd(L)
    f2 = _fwd(L, forced_idx=f1["idx"], forced_gate=2.0 * f1["gate"])
    assert np.array_equal(f2["idx"], f1["idx"])
    assert np.array_equal(f2["y"], 2.0 * f1["y"])


# --------------------------------------------------------------------------- e5m2
def test_e5m2_decode_table_against_the_format():
    """Every code against the OCP e5m2 definition written out by hand."""
    v = O.e5m2_decode(np.arange(256, dtype=np.uint8))
    assert v[0x00] == 0.0 and v[0x80] == 0.0 and np.signbit(v[0x80])
    assert v[0x01] == 2.0 ** -16                # smallest subnormal
    assert v[0x03] == 3 * 2.0 ** -16            # largest subnormal
    assert v[0x04] == 2.0 ** -14                # smallest normal
    assert v[0x3c] == 1.0 and v[0xbc] == -1.0
    assert v[0x3d] == 1.25 and v[0x3e] == 1.5 and v[0x3f] == 1.75
    assert v[0x7b] == 57344.0 and v[0xfb] == -57344.0
    assert v[0x7c] == np.inf and v[0xfc] == -np.inf
    assert all(np.isnan(v[c]) for c in (0x7d, 0x7e, 0x7f, 0xfd, 0xfe, 0xff))
    finite = v[np.isfinite(v)]
    assert len(finite) == 248 and len(np.unique(finite)) == 247


def test_e5m2_encode_rounding_and_brute_force():
    """Finite values encode to themselves; midpoints go to the even code and a
    hair either side to the nearer; magnitudes beyond 57344 clamp to it; and
    random values match a nearest-value search over the finite codes written
    independently."""
    codes = np.arange(0x7c, dtype=np.uint8)
    vals = O.e5m2_decode(codes)
    assert np.array_equal(O.e5m2_decode(O.e5m2_encode(vals)), vals)
    mid = (vals[:-1] + vals[1:]) / 2
    lo = codes[:-1]
    assert np.array_equal(O.e5m2_encode(mid), np.where(lo % 2 == 0, lo, lo + 1))
    assert np.array_equal(O.e5m2_encode(np.nextafter(mid, 0)), lo)
    assert np.array_equal(O.e5m2_encode(np.nextafter(mid, np.inf)), lo + 1)
    assert O.e5m2_encode([1e6])[0] == 0x7b and O.e5m2_encode([-1e6])[0] == 0xfb
    g = np.random.default_rng(33)
    x = np.concatenate([g.standard_normal(2000) * 3000, g.standard_normal(1000) * 1e-4])
    for v in x:
        a = min(abs(v), 57344.0)
        dd = np.abs(vals - a)
        best = np.where(dd == dd.min())[0]
        c = best[0] if len(best) == 1 else [b for b in best if b % 2 == 0][0]
        assert O.e5m2_encode([v])[0] == (c | (0x80 if v < 0 else 0)), v


def test_e5m2_rowwise_quantisation_and_product():
    """Row-wise e5m2: every row maximum maps to 57344 exactly, every element is
    reproduced within half an e5m2 step (2^-3 of the value, or 2^-17 of the
    row scale in the subnormal range), and the product with an e4m3 operand
    equals the product of the two dequantised operands."""
    g = np.random.default_rng(34)
    x = (g.standard_normal((30, 64)) * np.exp(g.uniform(-4, 4, (30, 1)))).astype(np.float32)
    q, s = O.quantize_rowwise(x, "e5m2")
    xd = O.e5m2_decode(q) * s[:, None].astype(np.float64)
    bound = np.maximum(np.abs(x) * 2.0 ** -3, s[:, None].astype(np.float64) * 2.0 ** -17)
    assert np.all(np.abs(xd - x) <= bound * (1 + 1e-12))
    assert np.all(np.max(np.abs(O.e5m2_decode(q)), axis=1) == 57344.0)
    w = g.standard_normal((20, 64)).astype(np.float32)
    qw, sw = O.quantize_rowwise(w)
    C = O.grouped_gemm_fp8_nt(q, s, qw[None], sw[None], np.array([0, 30]), "e5m2")
    ref = xd @ (O.e4m3_decode(qw) * sw[:, None].astype(np.float64)).T
    assert np.max(np.abs(C - ref)) <= 1e-12 * np.max(np.abs(ref))


def _e5m2_grid(g, R, C, p):
    """[R, C] values on the e5m2 grid times 2^-p, each row's largest magnitude
    exactly 57344 * 2^-p: row-wise e5m2 quantisation is then exact."""
    codes = g.integers(0x10, 0x78, size=(R, C)).astype(np.uint8)     # moderate magnitudes
    m = O.e5m2_decode(codes) * np.where(g.random((R, C)) < 0.5, -1.0, 1.0)
    m[np.arange(R), np.arange(R) % C] = 57344.0
    return m * 2.0 ** -p


def test_fp8_layer_e5m2_gradients():
    """The fp8 backward with e5m2 gradient operands: with one-hot tokens and
    weights on the e4m3 grid, top-1 routing and dy on the e5m2 grid, the down
    data gradient is exact (dG | dU equal the exact backward's); scaling dy by
    2^-2 scales dx and every gradient by exactly 2^-2; off the grid it stays
    close to the exact layer, further from it than the e4m3 gradients (one
    mantissa bit fewer)."""
    T, d, E, k, f = 24, 48, 4, 1, 32
    L = _grid_layer(5, T, d, E, k, f, 8, "softmax", True, one_hot=True)
    L["dy"] = _e5m2_grid(np.random.default_rng(8), T, d, 12)
    ex = _fwd(L)
    f8 = _fwd(L, fp8=True)
    b_ex = _bwd(L, ex)
    b_5 = O.backward(L["x"], L["w_router"], L["w_gateup"], L["w_down"], L["s_gateup"], L["s_down"],
                     f8, L["dy"], score=L["score"], renorm=L["renorm"], fp8=True, fp8_grad_format="e5m2")
    assert np.array_equal(b_5["dgu"], b_ex["dgu"])
    L2 = _rand_layer(11, 40, 32, 6, 2, 16, 16, "sigmoid", True)
    fw = _fwd(L2, fp8=True)
    bw = lambda dy, fmt: O.backward(L2["x"], L2["w_router"], L2["w_gateup"], L2["w_down"],  # noqa: E731
                                    L2["s_gateup"], L2["s_down"], fw, dy, score=L2["score"],
                                    renorm=L2["renorm"], fp8=True, fp8_grad_format=fmt)
    b1, b2 = bw(L2["dy"], "e5m2"), bw(L2["dy"] * 0.25, "e5m2")
    for key in ("dx", "d_w_gateup", "d_w_down", "d_s_gateup", "d_s_down", "d_w_router"):
        assert np.array_equal(b2[key], 0.25 * b1[key]), key
    fx = _fwd(L2)
    bx = _bwd(L2, fx)
    b4 = bw(L2["dy"], "e4m3")
    r5, r4 = _rel(b1["dx"], bx["dx"]), _rel(b4["dx"], bx["dx"])
    assert 1e-4 < r4 < r5 < 0.15, (r4, r5)


# --------------------------------------------------------------------------- fp8 weight gradients
def test_wgrad_fp8_exact_on_the_grid_and_bounded():
    """wgrad_fp8(a, b) = a^T b when every column of both operands is on the
    e4m3 grid with column maxima 448 * 2^-p (exact column-wise quantisation),
    stays within the half-step bound off the grid, and follows a power-of-two
    scaling of either operand exactly."""
    g = np.random.default_rng(72)
    a = _e4m3_grid(g, 20, 50, 6).T            # [50, 20]: columns on the grid
    b = _e4m3_grid(g, 12, 50, 9).T            # [50, 12]
    assert np.array_equal(O.wgrad_fp8(a, b), a.T @ b)
    a = g.standard_normal((70, 20))
    b = g.standard_normal((70, 12))
    sa = np.abs(a).max(0) / 448.0
    sb = np.abs(b).max(0) / 448.0
    ea = np.abs(a) * 2.0 ** -4 + sa[None, :] * 2.0 ** -10
    eb = np.abs(b) * 2.0 ** -4 + sb[None, :] * 2.0 ** -10
    bound = ea.T @ np.abs(b) + np.abs(a).T @ eb + ea.T @ eb
    err = np.abs(O.wgrad_fp8(a, b) - a.T @ b)
    assert np.all(err <= bound * (1 + 1e-6)) and err.max() > 0
    assert np.array_equal(O.wgrad_fp8(a * 4.0, b), 4.0 * O.wgrad_fp8(a, b))
    q, s = O.quantize_colwise(a)
    assert np.all(np.max(np.abs(O.e4m3_decode(q)), axis=0) == 448.0) and s.shape == (20,)


def test_fp8_layer_weight_gradients():
    """The fp8 backward with e4m3 weight gradients: one expert, top-1 (gate 1),
    one-hot tokens, dy and the forced H and dG | dU on the grid by rows and by
    columns -- every weight gradient is then the exact product of those
    operands; off the grid the weight gradients stay within a few per cent of
    the exact layer's and scale exactly with a power-of-two dy."""
    T, d, E, k, f, Fs = 40, 48, 1, 1, 32, 16
    L = _grid_layer(6, T, d, E, k, f, Fs, "softmax", True, one_hot=True)
    g = np.random.default_rng(10)
    L["dy"] = _e4m3_grid(g, T, d, 6, cols=True)
    fh = _e4m3_grid(g, T, f, 3, cols=True)
    fsh = _e4m3_grid(g, T, Fs, 3, cols=True)
    fw = _fwd(L, fp8=True, forced_h=fh, forced_s_h=fsh)
    assert np.array_equal(fw["h_q"], fh) and np.array_equal(fw["s_h_q"], fsh)
    fd = _e4m3_grid(g, T, 2 * f, 4, cols=True)
    fsd = _e4m3_grid(g, T, 2 * Fs, 4, cols=True)
    bw = O.backward(L["x"], L["w_router"], L["w_gateup"], L["w_down"], L["s_gateup"], L["s_down"], fw, L["dy"],
                    score=L["score"], renorm=L["renorm"], fp8=True, forced_dgu=fd, forced_s_dgu=fsd,
                    fp8_wgrad=True)
    x_perm = fw["x_perm"]
    assert np.all(fw["gate"] == 1.0)
    dyp = L["dy"][fw["src"] // k]
    assert np.array_equal(bw["d_w_down"][0], dyp.T @ fh)
    assert np.array_equal(bw["d_w_gateup"][0], fd.T @ x_perm)
    assert np.array_equal(bw["d_s_down"], L["dy"].T @ fsh)
    assert np.array_equal(bw["d_s_gateup"], fsd.T @ L["x"])
    # off the grid
    L2 = _rand_layer(12, 48, 32, 6, 2, 16, 16, "sigmoid", True)
    f2 = _fwd(L2, fp8=True)
    b = lambda dy, wg: O.backward(L2["x"], L2["w_router"], L2["w_gateup"], L2["w_down"],  # noqa: E731
                                  L2["s_gateup"], L2["s_down"], f2, dy, score=L2["score"], renorm=L2["renorm"],
                                  fp8=True, fp8_wgrad=wg)
    b8, bh, b8q = b(L2["dy"], True), b(L2["dy"], False), b(L2["dy"] * 0.25, True)
    for key in ("d_w_gateup", "d_w_down", "d_s_gateup", "d_s_down"):
        assert 1e-4 < _rel(b8[key], bh[key]) < 0.08, key
        assert np.array_equal(b8q[key], 0.25 * b8[key]), key
    assert np.array_equal(b8["dx"], bh["dx"])
