"""Per-call GPU parity: each C-ABI call against the CPU oracle.

Routing, counts, offsets and the permutation are compared bit-exactly on
identical fp32 logits; GEMM and combine outputs within the stated tolerance
(fp32: rel-L2 <= 1e-5; bf16: rel-L2 <= 1e-2 and max-abs <= 5e-2 * RMS)."""
import zlib

import numpy as np
import pytest
import torch

import synth
from oracle import moe_oracle as O
from tests.gpu_util import assert_rounded, dev, host, ulp_f32

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import mixture_experts_layer_18_amd as M


def _logits_for(cfg):
    inp = synth.make_inputs(cfg, parts=("x", "router"))
    logits = O.router_logits(synth.as_f64(inp["x"], cfg.dtype), inp["w_router"])
    return inp, logits


def _route_gpu(cfg, logits, bias, T=None):
    T = cfg.T if T is None else T
    desc = M.desc_from_config(cfg, T=T)
    idx = torch.empty(T, cfg.k, dtype=torch.int32, device="cuda")
    gate = torch.empty(T, cfg.k, dtype=torch.float32, device="cuda")
    hist = torch.empty(max(M.route_hist_elems(desc), 1), dtype=torch.int32, device="cuda")
    M.moe_route(desc, dev(logits), dev(bias), idx, gate, hist)
    torch.cuda.synchronize()
    return desc, idx, gate, hist


def _oracle_route(cfg, logits, bias):
    scores = O.router_scores(logits, cfg.score)
    keys = O.selection_keys(logits, scores, bias, cfg.score)
    idx, margin = O.select_topk(keys, cfg.k)
    gate = O.gates_from_scores(scores, idx, cfg.score, cfg.renorm)
    return idx, gate, margin


def _check_route(cfg, logits, bias, T=None):
    desc, idx, gate, hist = _route_gpu(cfg, logits, bias, T)
    oidx, ogate, _ = _oracle_route(cfg, logits, bias)
    gidx = idx.cpu().numpy()
    assert np.array_equal(gidx, oidx), f"idx mismatch on {(gidx != oidx).any(axis=1).sum()} tokens"
    g = gate.cpu().numpy()
    assert np.all(np.abs(g.astype(np.float64) - ogate) <= 2 * ulp_f32(ogate)), "gates beyond 2 ulp"
    # per-block expert histogram
    T_ = logits.shape[0]
    nblk = -(-T_ // 32)
    h = hist.cpu().numpy()[: cfg.E * nblk].reshape(cfg.E, nblk)
    for b in range(nblk):
        ref = np.bincount(oidx[b * 32:(b + 1) * 32].reshape(-1), minlength=cfg.E)
        assert np.array_equal(h[:, b], ref)
    return desc, idx, gate, hist


@pytest.mark.parametrize("cfg", synth.CONFIGS, ids=[c.name for c in synth.CONFIGS])
def test_route_bit_exact_on_identical_logits(cfg):
    print(f"[route] {cfg.name}", flush=True)
    inp, logits = _logits_for(cfg)
    _check_route(cfg, logits, inp["bias"])


@pytest.mark.parametrize("E,k,score,renorm,T", [
    (8, 8, "softmax", False, 45),      # k == E, ragged block
    (1, 1, "sigmoid", True, 33),       # single expert
    (256, 16, "sigmoid", True, 100),   # maximum E and k
    (128, 3, "softmax", True, 64),
    (100, 7, "sigmoid", True, 70),     # E not a power of two
])
def test_route_edge_shapes(E, k, score, renorm, T):
    print(f"[route-edge] E={E} k={k} {score} T={T}", flush=True)
    cfg = synth.CONFIGS[0].replace(E=E, k=k, score=score, renorm=renorm, T=T)
    g = np.random.default_rng(E * 1000 + k)
    logits = g.standard_normal((T, E)).astype(np.float32)
    bias = g.uniform(-0.1, 0.1, E).astype(np.float32) if score == "sigmoid" else None
    _check_route(cfg, logits, bias)


def test_route_exact_ties_go_to_lower_index():
    cfg = synth.CONFIGS[0].replace(E=16, k=4, score="sigmoid", renorm=True, T=64)
    g = np.random.default_rng(5)
    logits = g.integers(-2, 3, size=(64, 16)).astype(np.float32)   # many equal keys
    logits[0] = 0.0
    bias = np.zeros(16, np.float32)
    _check_route(cfg, logits, bias)
    cfg2 = cfg.replace(score="softmax", renorm=False)
    _check_route(cfg2, logits, None)


@pytest.mark.parametrize("cfg", synth.CONFIGS, ids=[c.name for c in synth.CONFIGS])
def test_permute_bit_exact(cfg):
    print(f"[permute] {cfg.name}", flush=True)
    inp, logits = _logits_for(cfg)
    desc, idx, gate, hist = _check_route(cfg, logits, inp["bias"])
    T, k, E, d = cfg.T, cfg.k, cfg.E, cfg.d
    x = dev(inp["x"])
    counts = torch.empty(E, dtype=torch.int32, device="cuda")
    offsets = torch.empty(E + 1, dtype=torch.int32, device="cuda")
    pos = torch.empty(T * k, dtype=torch.int32, device="cuda")
    src = torch.empty(T * k, dtype=torch.int32, device="cuda")
    x_perm = torch.empty(T * k, d, dtype=x.dtype, device="cuda")
    ws = M.alloc_workspace(desc, "permute")
    tok = torch.empty(T * k, dtype=torch.int32, device="cuda")
    M.moe_permute(desc, x, idx, hist, counts, offsets, pos, src, x_perm, ws, tok=tok)
    torch.cuda.synchronize()
    oc, oo, op, os_ = O.permute_indices(idx.cpu().numpy(), E)
    assert np.array_equal(tok.cpu().numpy(), os_ // k)
    # without the row copy: the same indices
    pos2, src2, tok2 = torch.full_like(pos, -1), torch.full_like(src, -1), torch.full_like(tok, -1)
    M.moe_permute(desc, x, idx, hist, counts, offsets, pos2, src2, None, ws, tok=tok2)
    torch.cuda.synchronize()
    assert torch.equal(pos2, pos) and torch.equal(src2, src) and torch.equal(tok2, tok)
    assert np.array_equal(counts.cpu().numpy(), oc)
    assert np.array_equal(offsets.cpu().numpy(), oo)
    assert oo[-1] == T * k
    assert np.array_equal(pos.cpu().numpy(), op)
    assert np.array_equal(src.cpu().numpy(), os_)
    # rows are exact copies: compare raw bits
    xb = x_perm.view(torch.int16) if x.dtype == torch.bfloat16 else x_perm.view(torch.int32)
    xs = x.view(torch.int16) if x.dtype == torch.bfloat16 else x.view(torch.int32)
    src_t = torch.from_numpy((os_ // k).astype(np.int64)).cuda()
    assert torch.equal(xb, xs[src_t])


def test_permute_then_combine_is_the_identity():
    """Permuted copies of the token rows, combined with renormalised gates
    (1/k each, k = 4 so that every step is exact), give x back bit for bit."""
    cfg = synth.CONFIG_BY_NAME["moe7b_bf16"].replace(T=777, d=256, E=16, k=4)
    inp, logits = _logits_for(cfg)
    desc, idx, gate, hist = _route_gpu(cfg, logits, inp["bias"])
    T, k, E, d = cfg.T, cfg.k, cfg.E, cfg.d
    x = dev(inp["x"])
    counts = torch.empty(E, dtype=torch.int32, device="cuda")
    offsets = torch.empty(E + 1, dtype=torch.int32, device="cuda")
    pos = torch.empty(T * k, dtype=torch.int32, device="cuda")
    src = torch.empty(T * k, dtype=torch.int32, device="cuda")
    x_perm = torch.empty(T * k, d, dtype=x.dtype, device="cuda")
    M.moe_permute(desc, x, idx, hist, counts, offsets, pos, src, x_perm, M.alloc_workspace(desc, "permute"))
    y = torch.empty_like(x)
    M.moe_combine(desc, x_perm, torch.full((T, k), 0.25, dtype=torch.float32, device="cuda"), pos, None, y)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), x.view(torch.int16))


# ----------------------------------------------------------------------------- grouped GEMM
def _groups(seed, G, mean, empty=(), big=None):
    g = np.random.default_rng(seed)
    m = g.integers(max(1, mean // 2), mean * 3 // 2 + 1, size=G)
    for e in empty:
        m[e] = 0
    if big is not None:
        m[big] = mean * 4 + 37
    off = np.zeros(G + 1, np.int32)
    off[1:] = np.cumsum(m)
    return off


def _rand(g, shape, dtype, scale=1.0):
    v = (g.standard_normal(shape) * scale).astype(np.float32)
    if dtype == "bf16":
        return synth.f32_to_bf16_bits(v)
    return v


GEMM_CASES = [
    # dtype, G, mean rows, N-dim, K-dim (as in the call)
    ("bf16", 6, 150, 256, 192),
    ("bf16", 5, 40, 384, 128),
    ("f32", 4, 70, 192, 128),
    ("bf16", 3, 300, 128, 256),   # data gradient on 128 x 256 tiles
    ("bf16", 4, 90, 64, 192),     # NN reduction of two 32-deep k-steps (dSwiGLU: G | U staged after the loop)
]


@pytest.mark.parametrize("dtype,G,mean,N,K", GEMM_CASES)
@pytest.mark.parametrize("layout,epi", [("NT", "none"), ("NT", "swiglu"), ("NN", "none"),
                                        ("NN", "dswiglu"), ("TN", "none")])
def test_grouped_gemm_against_oracle(dtype, G, mean, N, K, layout, epi):
    if epi == "swiglu" and N % 128:
        N += 64      # SwiGLU tiles pair 64 gate columns with 64 up columns
    print(f"[gemm] {layout}/{epi} {dtype} G={G} N={N} K={K}", flush=True)
    g = np.random.default_rng(zlib.crc32(f"{layout}{epi}{dtype}{G}".encode()))
    off = _groups(G * 7 + N, G, mean, empty=(1,), big=G - 1)
    Mt = int(off[-1])
    f64 = lambda a: synth.as_f64(a, dtype)  # noqa: E731
    if layout == "NT":
        A = _rand(g, (Mt, K), dtype)
        B = _rand(g, (G, N, K), dtype, 1 / np.sqrt(K))
        F = N // 2
        Cw = F if epi == "swiglu" else N
        C = torch.empty(Mt, Cw, dtype=torch.bfloat16 if dtype == "bf16" else torch.float32, device="cuda")
        aux = torch.empty(Mt, N, dtype=C.dtype, device="cuda") if epi == "swiglu" else None
        M.moe_grouped_gemm(layout, epi, dtype, G, Mt, N, K, dev(off), dev(A), dev(B), C, aux)
        torch.cuda.synchronize()
        ref = np.zeros((Mt, Cw))
        refaux = np.zeros((Mt, N))
        for e in range(G):
            a0, a1 = off[e], off[e + 1]
            if epi == "swiglu":
                Gm, U, H, _ = O.swiglu_ffn(f64(A[a0:a1]), f64(B[e, :F]), f64(B[e, F:]), np.zeros((1, F)))
                ref[a0:a1] = H
                refaux[a0:a1, :F] = Gm
                refaux[a0:a1, F:] = U
            else:
                ref[a0:a1] = f64(A[a0:a1]) @ f64(B[e]).T
        assert_rounded(host(C), ref, dtype, "C")
        if epi == "swiglu":
            assert_rounded(host(aux), refaux, dtype, "aux")
    elif layout == "NN":
        A = _rand(g, (Mt, N), dtype)
        B = _rand(g, (G, N, K), dtype, 1 / np.sqrt(N))
        Cw = 2 * K if epi == "dswiglu" else K
        C = torch.empty(Mt, Cw, dtype=torch.bfloat16 if dtype == "bf16" else torch.float32, device="cuda")
        aux_h = _rand(g, (Mt, 2 * K), dtype) if epi == "dswiglu" else None
        M.moe_grouped_gemm(layout, epi, dtype, G, Mt, N, K, dev(off), dev(A), dev(B), C, dev(aux_h))
        torch.cuda.synchronize()
        ref = np.zeros((Mt, Cw))
        for e in range(G):
            a0, a1 = off[e], off[e + 1]
            if epi == "dswiglu":
                # the down projection's data gradient through the oracle's SwiGLU backward
                Gm, U = f64(aux_h[a0:a1, :K]), f64(aux_h[a0:a1, K:])
                dG, dU = _dswiglu_ref(f64(A[a0:a1]), f64(B[e]), Gm, U)
                ref[a0:a1, :K] = dG
                ref[a0:a1, K:] = dU
            else:
                ref[a0:a1] = f64(A[a0:a1]) @ f64(B[e])
        assert_rounded(host(C), ref, dtype, "C")
    else:
        A = _rand(g, (Mt, N), dtype)
        B = _rand(g, (Mt, K), dtype)
        C = torch.full((G, N, K), float("nan"), dtype=torch.bfloat16 if dtype == "bf16" else torch.float32,
                       device="cuda")
        ws_n = M.grouped_gemm_workspace_bytes(layout, dtype, G, Mt, N, K)
        ws = torch.empty(max(ws_n, 256), dtype=torch.uint8, device="cuda")
        M.moe_grouped_gemm(layout, epi, dtype, G, Mt, N, K, dev(off), dev(A), dev(B), C, None, ws)
        torch.cuda.synchronize()
        ref = np.zeros((G, N, K))
        for e in range(G):
            a0, a1 = off[e], off[e + 1]
            ref[e] = f64(A[a0:a1]).T @ f64(B[a0:a1])
        out = host(C)
        assert np.all(out[1] == 0.0), "empty group must give zero"
        assert_rounded(out, ref, dtype, "C")


@pytest.mark.parametrize("G,N,K", [(64, 1024, 1024), (128, 1024, 320)], ids=["whole-tiles", "partial-columns"])
def test_weight_gradient_many_groups(G, N, K):
    """A weight gradient with enough 256 x 256 output tiles for the persistent
    kernel: ragged groups, an empty group and one group four times the mean;
    K = 320 leaves a partial last column tile."""
    mean = 100
    print(f"[gemm] TN persistent G={G} N={N} K={K}", flush=True)
    off = _groups(91, G, mean, empty=(3, 40), big=17)
    Mt = int(off[-1])
    g = np.random.default_rng(92)
    A = _rand(g, (Mt, N), "bf16")
    B = _rand(g, (Mt, K), "bf16")
    assert M.grouped_gemm_workspace_bytes("TN", "bf16", G, Mt, N, K) == 0
    C = torch.full((G, N, K), float("nan"), dtype=torch.bfloat16, device="cuda")
    M.moe_grouped_gemm("TN", "none", "bf16", G, Mt, N, K, dev(off), dev(A), dev(B), C)
    torch.cuda.synchronize()
    f64 = lambda a: synth.as_f64(a, "bf16")  # noqa: E731
    ref = np.stack([f64(A[off[e]:off[e + 1]]).T @ f64(B[off[e]:off[e + 1]]) for e in range(G)])
    out = host(C)
    assert np.all(out[3] == 0.0) and np.all(out[40] == 0.0), "empty groups must give zero"
    assert_rounded(out, ref, "bf16", "C")


@pytest.mark.parametrize("rows", [[4096], [4000], [5000, 37]], ids=["one-4096", "one-4000", "big-small"])
def test_weight_gradient_row_slices(rows):
    """Weight gradients with few output tiles and long groups run as row
    slices with fp32 partials summed in order (empty slices included)."""
    print(f"[gemm] TN slices rows={rows}", flush=True)
    G, N, K = len(rows), 256, 384
    off = np.zeros(G + 1, np.int32)
    off[1:] = np.cumsum(rows)
    Mt = int(off[-1])
    g = np.random.default_rng(sum(rows))
    A = _rand(g, (Mt, N), "bf16")
    B = _rand(g, (Mt, K), "bf16")
    ws_n = M.grouped_gemm_workspace_bytes("TN", "bf16", G, Mt, N, K)
    assert ws_n > 0, "this shape is expected to use row slices"
    ws = torch.empty(ws_n, dtype=torch.uint8, device="cuda")
    C = torch.full((G, N, K), float("nan"), dtype=torch.bfloat16, device="cuda")
    M.moe_grouped_gemm("TN", "none", "bf16", G, Mt, N, K, dev(off), dev(A), dev(B), C, None, ws)
    torch.cuda.synchronize()
    f64 = lambda a: synth.as_f64(a, "bf16")  # noqa: E731
    ref = np.stack([f64(A[off[e]:off[e + 1]]).T @ f64(B[off[e]:off[e + 1]]) for e in range(G)])
    assert_rounded(host(C), ref, "bf16", "C")
    with pytest.raises(M.MoeError):
        M.moe_grouped_gemm("TN", "none", "bf16", G, Mt, N, K, dev(off), dev(A), dev(B), C, None,
                           ws[: ws_n // 2])


@pytest.mark.parametrize("Mt,N,K,slices", [(8195, 1024, 1280, 8), (4100, 2048, 2816, 2), (1000, 4096, 2048, 1)],
                         ids=["20-tiles", "88-tiles", "128-tiles"])
def test_one_group_weight_gradient_persistent(Mt, N, K, slices):
    """A one-group weight gradient (the shared experts' shape) with fewer than
    1024 output tiles on the persistent kernel: cut into equal row slices of
    whole k-steps (the last one ragged) until 128 tiles run, fp32 partials
    summed in slice order; with 128 tiles of its own, unsliced."""
    print(f"[gemm] TN one group M={Mt} N={N} K={K} slices={slices}", flush=True)
    ws_n = M.grouped_gemm_workspace_bytes("TN", "bf16", 1, Mt, N, K)
    assert ws_n == (slices * N * K * 4 if slices > 1 else 0)
    g = np.random.default_rng(Mt + N + K)
    A = _rand(g, (Mt, N), "bf16")
    B = _rand(g, (Mt, K), "bf16")
    ws = torch.empty(max(ws_n, 256), dtype=torch.uint8, device="cuda")
    C = torch.full((1, N, K), float("nan"), dtype=torch.bfloat16, device="cuda")
    off = np.array([0, Mt], np.int32)
    M.moe_grouped_gemm("TN", "none", "bf16", 1, Mt, N, K, dev(off), dev(A), dev(B), C, None, ws)
    torch.cuda.synchronize()
    f64 = lambda a: synth.as_f64(a, "bf16")  # noqa: E731
    ref = (f64(A).T @ f64(B))[None]
    assert_rounded(host(C), ref, "bf16", "C")
    # no offset table (one group) gives the same bits
    C2 = torch.full_like(C, float("nan"))
    M.moe_grouped_gemm("TN", "none", "bf16", 1, Mt, N, K, None, dev(A), dev(B), C2, None, ws)
    torch.cuda.synchronize()
    assert torch.equal(C.view(torch.int16), C2.view(torch.int16))
    if slices > 1:
        with pytest.raises(M.MoeError):
            M.moe_grouped_gemm("TN", "none", "bf16", 1, Mt, N, K, dev(off), dev(A), dev(B), C, None,
                               ws[: ws_n // 2])


def _dswiglu_ref(dY, Wd_e, Gm, U):
    """dG | dU of the oracle's SwiGLU backward with upstream dY through the
    down weight Wd_e [N, K] (here the product dH = dY Wd_e)."""
    # swiglu_ffn_backward takes the down weight as [d, f] and forms dH = dY @ w_down
    _, _, _, _, dG, dU = O.swiglu_ffn_backward(np.zeros((dY.shape[0], 1)), np.zeros((Gm.shape[1], 1)),
                                               np.zeros((Gm.shape[1], 1)), Wd_e, Gm, U, O.silu(Gm) * U, dY)
    return dG, dU


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_combine_against_oracle(dtype):
    print(f"[combine] {dtype}", flush=True)
    g = np.random.default_rng(11)
    T, d, k = 300, 256, 3
    E = 8
    idx = np.stack([g.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    _, _, pos, _ = O.permute_indices(idx, E)
    y_perm = _rand(g, (T * k, d), dtype)
    shared = _rand(g, (T, d), dtype)
    gate = g.uniform(0, 1, (T, k)).astype(np.float32)
    cfg = synth.CONFIGS[0].replace(T=T, d=d, k=k, E=E, dtype=dtype)
    desc = M.desc_from_config(cfg)
    for sh in (None, shared):
        y = torch.empty(T, d, dtype=torch.bfloat16 if dtype == "bf16" else torch.float32, device="cuda")
        M.moe_combine(desc, dev(y_perm), dev(gate), dev(pos), dev(sh), y)
        torch.cuda.synchronize()
        ref = O.combine(synth.as_f64(y_perm, dtype), gate, pos, None if sh is None else synth.as_f64(sh, dtype))
        assert_rounded(host(y), ref, dtype, "y")


FUSED_ROUTE = [
    ("moe7b_bf16", dict(T=1000)),                                    # E = 64, ragged last block
    ("finegrained_bf16", dict(T=4096)),                              # E = 64, top-8
    ("moe7b_bf16", dict(name="e16_softmax", T=300, d=256, E=16, k=4, f=128, n_shared=0, f_shared=0,
                        score="softmax", renorm=True, bias=None)),   # E < 64, softmax renormalised
    ("moe7b_bf16", dict(name="e64_softmax", T=777, d=256, E=64, k=2, f=128, n_shared=0, f_shared=0,
                        score="softmax", renorm=False, bias=None)),  # softmax without renormalisation
]


@pytest.mark.parametrize("base,kw", FUSED_ROUTE, ids=[f"{b}-{kw.get('name', kw['T'])}" for b, kw in FUSED_ROUTE])
def test_forward_routing_matches_moe_route(base, kw):
    """The forward pass routes its own logits inside the router kernel (bf16
    tokens, E <= 64); moe_route and moe_permute on those same logits must
    give the same indices, gates, counts, offsets and permutation bit for bit."""
    cfg = synth.CONFIG_BY_NAME[base].replace(**kw)
    inp = synth.make_inputs(cfg)
    desc = M.desc_from_config(cfg)
    w = {n: dev(inp.get(n)) for n in ("w_router", "bias", "w_gateup", "w_down", "s_gateup", "s_down")}
    x = dev(inp["x"])
    y = torch.empty_like(x)
    saved = M.alloc_saved(desc, training=False, gather=True)
    M.moe_forward(desc, w, x, y, saved, M.alloc_workspace(desc, "forward"))
    torch.cuda.synchronize()
    T, k, E = cfg.T, cfg.k, cfg.E
    idx = torch.empty(T, k, dtype=torch.int32, device="cuda")
    gate = torch.empty(T, k, dtype=torch.float32, device="cuda")
    hist = torch.empty(max(M.route_hist_elems(desc), 1), dtype=torch.int32, device="cuda")
    M.moe_route(desc, saved["logits"], w["bias"] if cfg.score == "sigmoid" else None, idx, gate, hist)
    A = T * k
    counts = torch.empty(E, dtype=torch.int32, device="cuda")
    offsets = torch.empty(E + 1, dtype=torch.int32, device="cuda")
    pos = torch.empty(A, dtype=torch.int32, device="cuda")
    src = torch.empty(A, dtype=torch.int32, device="cuda")
    tok = torch.empty(A, dtype=torch.int32, device="cuda")
    M.moe_permute(desc, x, idx, hist, counts, offsets, pos, src, None, M.alloc_workspace(desc, "permute"), tok=tok)
    torch.cuda.synchronize()
    for name, a, b in (("idx", saved["idx"], idx), ("gate", saved["gate"], gate), ("counts", saved["counts"], counts),
                       ("offsets", saved["offsets"], offsets), ("pos", saved["pos"], pos), ("src", saved["src"], src),
                       ("tok", saved["tok"], tok)):
        assert torch.equal(a.view(torch.int32), b.view(torch.int32)), f"{cfg.name}: {name} differs"


def test_hbm_ceiling_copies_bytes():
    """The streaming-copy measurement aid moves every byte unchanged (a size
    that is not a multiple of 256 vectors leaves a partial last workgroup)."""
    print("[hbm ceiling] copy", flush=True)
    n = (1 << 20) + 48
    src = torch.randint(0, 256, (n,), dtype=torch.uint8, device="cuda")
    dst = torch.zeros_like(src)
    M.hbm_ceiling(src, dst)
    torch.cuda.synchronize()
    assert torch.equal(src, dst)
