"""Whole-layer parity at the full sizes of the benchmark layers, in the launch
configuration the benchmark times.

The oracle cannot run a full 16k- or 64k-token layer in seconds, so:
  * routing is checked on every token (logits are cheap);
  * the oracle follows the GPU's routing (its expert indices forced, gates
    from its own scores), so a near-tie that chose differently is compared,
    not dropped;
  * up to 16384 tokens the oracle runs the whole batch: y, dx and every
    gradient are compared on every token;
  * at 65536 tokens, y and dx are compared on 4096 tokens, among them the
    tokens at the first and last permuted row of every 256-row tile of every
    expert (each output depends only on its own token); the weight gradients
    come from a second backward pass whose upstream gradient is zero outside
    a uniform quarter of the tokens: every weight gradient is then a sum over
    that sample alone, which the oracle computes exactly, while the GPU still
    runs every kernel over all tokens and all experts.
"""
import numpy as np
import pytest
import torch

import synth
from oracle import moe_oracle as O
from tests.gpu_util import assert_close, assert_rounded, dev, host, max_abs_over_rms

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import mixture_experts_layer_18_amd as M
    from tests import layer_runner as R

FULL = [c for c in synth.CONFIGS if c.backward] + [synth.CONFIG_BY_NAME["finegrained_bf16"]]
# the benchmark's launch configuration gathers the token rows (no permuted
# copy); the 7B-style layer also runs with the permuted copy
CASES = [(c, True) for c in FULL] + [(synth.CONFIG_BY_NAME["moe7b_bf16"], False)]


def _sample(T, n, seed, must=()):
    """n tokens (at least): the tokens in `must`, then random others."""
    g = np.random.default_rng(seed)
    must = np.unique(np.asarray(must, np.int64))
    rest = np.setdiff1d(np.arange(T), must)
    extra = g.choice(rest, size=max(0, min(n - must.size, rest.size)), replace=False)
    return np.sort(np.concatenate([must, extra]))


def _tile_edge_tokens(offsets, tok, tile=256):
    """Tokens at the first and last permuted row of every 256-row tile of
    every expert (the rows where the grouped GEMM's tiles and ragged tails
    begin and end)."""
    rows = []
    for e in range(offsets.size - 1):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        for r0 in range(lo, hi, tile):
            rows += [r0, min(r0 + tile, hi) - 1]
    return tok[np.asarray(rows, np.int64)] if rows else np.zeros(0, np.int64)


@pytest.mark.parametrize("cfg,gather", CASES,
                         ids=[c.name + ("" if gth else "-permuted-copy") for c, gth in CASES])
def test_full_size_layer(cfg, gather):
    print(f"[full] {cfg.name} gather={gather}: generating inputs", flush=True)
    inp = synth.make_inputs(cfg, with_dy=True)
    desc = M.desc_from_config(cfg)
    w = R.upload_layer(cfg, inp)
    x = dev(inp["x"])
    dy = dev(inp["dy"])
    print(f"[full] {cfg.name}: GPU forward+backward", flush=True)
    g = R.run_gpu(cfg, inp, backward=True, weights=w, x=x, dy=dy, keep_device=True, gather=gather)
    g_logits = g["saved"]["logits"].cpu().numpy()
    g_idx = g["saved"]["idx"].cpu().numpy()
    counts = g["saved"]["counts"].cpu().numpy()
    offsets = g["saved"]["offsets"].cpu().numpy().astype(np.int64)
    tok = g["saved"]["tok"].cpu().numpy().astype(np.int64)
    assert counts.sum() == cfg.T * cfg.k
    assert torch.isfinite(g["y"].float()).all() and torch.isfinite(g["dx"].float()).all()

    # --- routing on every token
    print(f"[full] {cfg.name}: oracle router on all tokens", flush=True)
    xf = synth.as_f64(inp["x"], cfg.dtype)
    logits = O.router_logits(xf, inp["w_router"])
    scores = O.router_scores(logits, cfg.score)
    keys = O.selection_keys(logits, scores, inp["bias"], cfg.score)
    oidx, margin = O.select_topk(keys, cfg.k)
    fw_r = dict(logits=logits, keys=keys, idx=oidx, margin=margin)
    R.check_routing(cfg, g_logits, g_idx, fw_r)
    flips = int(np.sum(np.any(g_idx != oidx, axis=1)))
    print(f"[full] {cfg.name}: tokens on a near-tie choice other than the oracle's {flips}, margin<1e-3 "
          f"{int((margin < R.MARGIN).sum())}", flush=True)
    if cfg.bias == "zipf":
        assert (counts == 0).sum() >= 4

    oi = R.oracle_inputs(cfg, inp)
    if cfg.T <= 16384:
        # --- the whole batch: the oracle on every token (on the GPU's
        # routing), y, dx and every gradient compared in full
        print(f"[full] {cfg.name}: oracle forward+backward on all {cfg.T} tokens", flush=True)
        fw = O.forward(oi["x"], oi["w_router"], oi["bias"], oi["w_gateup"], oi["w_down"], oi["s_gateup"],
                       oi["s_down"], top_k=cfg.k, score=cfg.score, renorm=cfg.renorm, forced_idx=g_idx)
        bw = O.backward(oi["x"], oi["w_router"], oi["w_gateup"], oi["w_down"], oi["s_gateup"], oi["s_down"], fw,
                        oi["dy"], score=cfg.score, renorm=cfg.renorm)
        assert_close(host(g["y"]), fw["y"], cfg.dtype, "y")
        assert_close(host(g["dx"]), bw["dx"], cfg.dtype, "dx")
        _compare_grads(cfg, g["grads"], bw)
        return

    # --- 64k tokens: a token sample S with every expert's tile-edge rows plus
    # random tokens (4096), the oracle on the GPU's routing (indices forced:
    # no token excluded) for y and dx
    edges = _tile_edge_tokens(offsets, tok)
    S = _sample(cfg.T, max(4096, np.unique(edges).size), 1, must=edges)
    print(f"[full] {cfg.name}: oracle on {S.size} sampled tokens ({np.unique(edges).size} at tile edges)",
          flush=True)
    fw = O.forward(oi["x"][S], oi["w_router"], oi["bias"], oi["w_gateup"], oi["w_down"], oi["s_gateup"],
                   oi["s_down"], top_k=cfg.k, score=cfg.score, renorm=cfg.renorm, forced_idx=g_idx[S])
    bw = O.backward(oi["x"][S], oi["w_router"], oi["w_gateup"], oi["w_down"], oi["s_gateup"], oi["s_down"], fw,
                    oi["dy"][S], score=cfg.score, renorm=cfg.renorm)
    assert_close(host(g["y"])[S], fw["y"], cfg.dtype, "y")
    assert_close(host(g["dx"])[S], bw["dx"], cfg.dtype, "dx")
    del fw, bw

    # --- weight gradients: a second backward whose upstream gradient is zero
    # outside a uniform sample S2 of a quarter of the tokens, so every weight
    # gradient is a sum over S2 alone (each expert keeps its share of rows)
    S2 = _sample(cfg.T, cfg.T // 4, 2)
    print(f"[full] {cfg.name}: oracle forward+backward on {S2.size} uniformly sampled tokens", flush=True)
    fw = O.forward(oi["x"][S2], oi["w_router"], oi["bias"], oi["w_gateup"], oi["w_down"], oi["s_gateup"],
                   oi["s_down"], top_k=cfg.k, score=cfg.score, renorm=cfg.renorm, forced_idx=g_idx[S2])
    bw = O.backward(oi["x"][S2], oi["w_router"], oi["w_gateup"], oi["w_down"], oi["s_gateup"], oi["s_down"], fw,
                    oi["dy"][S2], score=cfg.score, renorm=cfg.renorm)
    del fw
    mask = torch.zeros(cfg.T, 1, dtype=dy.dtype, device="cuda")
    mask[torch.from_numpy(S2).cuda()] = 1
    dy2 = (dy * mask).contiguous()
    grads = M.alloc_grads(desc)
    dx2 = torch.empty_like(x)
    wsb = M.alloc_workspace(desc, "backward")
    print(f"[full] {cfg.name}: GPU backward with masked upstream gradient", flush=True)
    M.moe_backward(desc, w, x, g["saved"], dy2, dx2, grads, wsb)
    torch.cuda.synchronize()
    _compare_grads(cfg, grads, bw)
    out_dx2 = host(dx2)
    assert np.all(out_dx2[np.setdiff1d(np.arange(cfg.T), S2)] == 0.0)
    assert_close(out_dx2[S2], bw["dx"], cfg.dtype, "dx (masked)")


def _compare_grads(cfg, grads, bw):
    for name in ("d_w_gateup", "d_w_down", "d_s_gateup", "d_s_down"):
        if grads[name] is None:
            continue
        gv = host(grads[name])
        ref = bw[name]
        rms = np.sqrt(np.mean(ref * ref))
        big = np.abs(ref) >= rms
        print(f"[full] {cfg.name}: {name} rel-L2 {R.rel_l2(gv, ref):.2e} max-abs/RMS "
              f"{max_abs_over_rms(gv, ref):.2e} (max|ref|/RMS {np.abs(ref).max() / rms:.1f}, worst relative "
              f"error where |ref| >= RMS {np.max(np.abs(gv[big] - ref[big]) / np.abs(ref[big])):.2e})", flush=True)
        assert_close(gv, ref, cfg.dtype, name)
    # the router gradient is fp32; its reference runs through bf16-rounded
    # expert outputs on the GPU, so it is held to the bf16 layer bar
    assert_close(grads["d_w_router"].cpu().numpy(), bw["d_w_router"], cfg.dtype, "d_w_router")


def test_full_size_fp8_gate_up():
    """The fp8 forward gate/up product in the configuration the benchmark times
    (7B-style layer, 98304 routed rows, row-wise e4m3 scales, SwiGLU
    epilogue), checked on sampled rows of six experts: the largest, the
    smallest non-empty one and four more.  The oracle quantises the sampled
    token rows and those experts' weights from the bf16 inputs itself; the
    GPU's codes and scales must equal its codes and scales bit for bit, and
    its pre-activations and h must be within one bf16 rounding of the
    oracle's fp8 product."""
    cfg = synth.CONFIG_BY_NAME["moe7b_bf16"]
    print(f"[full] {cfg.name} fp8 gate/up: generating inputs", flush=True)
    inp = synth.make_inputs(cfg, with_dy=False)
    w = R.upload_layer(cfg, inp)
    x = dev(inp["x"])
    g = R.run_gpu(cfg, inp, backward=False, weights=w, x=x, keep_device=True, gather=True)
    saved = g["saved"]
    A, d, E, f = cfg.T * cfg.k, cfg.d, cfg.E, cfg.f
    x_perm = x[saved["tok"].long()].contiguous()
    xq = torch.empty(A, d, dtype=torch.uint8, device="cuda")
    xs = torch.empty(A, dtype=torch.float32, device="cuda")
    wq = torch.empty(E * 2 * f, d, dtype=torch.uint8, device="cuda")
    ws = torch.empty(E * 2 * f, dtype=torch.float32, device="cuda")
    h = torch.empty(A, f, dtype=torch.bfloat16, device="cuda")
    aux = torch.empty(A, 2 * f, dtype=torch.bfloat16, device="cuda")
    print(f"[full] {cfg.name} fp8 gate/up: GPU quantisation and grouped GEMM", flush=True)
    M.moe_quantize_fp8(w["w_gateup"].reshape(E * 2 * f, d), wq, ws)
    M.moe_quantize_fp8(x_perm, xq, xs)
    M.moe_grouped_gemm_fp8("swiglu", E, A, 2 * f, d, saved["offsets"], xq, xs, wq, ws, h, aux)
    torch.cuda.synchronize()

    off = saved["offsets"].cpu().numpy().astype(np.int64)
    tok = saved["tok"].cpu().numpy().astype(np.int64)
    counts = np.diff(off)
    nz = np.where(counts > 0)[0]
    rng = np.random.default_rng(7)
    experts = [int(nz[np.argmax(counts[nz])]), int(nz[np.argmin(counts[nz])])]
    experts += [int(e) for e in rng.choice(np.setdiff1d(nz, experts), size=4, replace=False)]
    h_all, aux_all = host(h), host(aux)
    xq_h, xs_h = xq.cpu().numpy(), xs.cpu().numpy()
    wq_h, ws_h = wq.cpu().numpy(), ws.cpu().numpy()
    for e in experts:
        lo, hi = int(off[e]), int(off[e + 1])
        rows = np.unique(np.concatenate([[lo, hi - 1], rng.integers(lo, hi, size=min(30, hi - lo))]))
        print(f"[full] fp8 gate/up: expert {e} ({hi - lo} rows), {rows.size} sampled", flush=True)
        qa, sa = O.quantize_rowwise(synth.as_f64(inp["x"][tok[rows]], "bf16"))
        qb, sb = O.quantize_rowwise(synth.as_f64(inp["w_gateup"][e], "bf16"))
        assert np.array_equal(xq_h[rows], qa) and np.array_equal(xs_h[rows], sa), "token row codes/scales"
        wr = slice(e * 2 * f, (e + 1) * 2 * f)
        assert np.array_equal(wq_h[wr], qb) and np.array_equal(ws_h[wr], sb), "weight codes/scales"
        ref = O.grouped_gemm_fp8_nt(qa, sa, qb[None], sb[None], np.array([0, rows.size]))
        assert_rounded(aux_all[rows], ref, "bf16", f"pre-activations, expert {e}")
        Gm, U = ref[:, :f], ref[:, f:]
        err = 1e-4 * np.sqrt(np.mean(ref * ref))
        sg = 1.0 / (1.0 + np.exp(-Gm))
        inherited = (np.abs(sg * (1.0 + Gm * (1.0 - sg)) * U) + np.abs(O.silu(Gm))) * err
        assert_rounded(h_all[rows], O.silu(Gm) * U, "bf16", f"h, expert {e}", extra=inherited)


def test_full_size_fp8_gate_up_data_gradient():
    """The fp8 gate/up data gradient dX = dGU . W_gu as the benchmark times it
    (7B-style layer routing, 98304 rows, dGU ~ N(0, 0.01^2) drawn on the
    host, W_gu quantised along 2f and stored transposed), checked on sampled
    rows of six experts: codes and scales bit-exact, products within one
    bf16 rounding of the oracle's fp8 product."""
    cfg = synth.CONFIG_BY_NAME["moe7b_bf16"]
    print(f"[full] {cfg.name} fp8 data gradient: generating inputs", flush=True)
    inp = synth.make_inputs(cfg, with_dy=False)
    w = R.upload_layer(cfg, inp)
    x = dev(inp["x"])
    g = R.run_gpu(cfg, inp, backward=False, weights=w, x=x, keep_device=True, gather=True)
    A, d, E, f = cfg.T * cfg.k, cfg.d, cfg.E, cfg.f
    rng = np.random.default_rng(12)
    dgu = synth.f32_to_bf16_bits((rng.standard_normal((A, 2 * f), dtype=np.float32) * 0.01).astype(np.float32))
    aq = torch.empty(A, 2 * f, dtype=torch.uint8, device="cuda")
    asc = torch.empty(A, dtype=torch.float32, device="cuda")
    wq = torch.empty(E, d, 2 * f, dtype=torch.uint8, device="cuda")
    wsc = torch.empty(E, d, dtype=torch.float32, device="cuda")
    dx = torch.empty(A, d, dtype=torch.bfloat16, device="cuda")
    print(f"[full] {cfg.name} fp8 data gradient: GPU quantisation and grouped GEMM", flush=True)
    M.moe_quantize_fp8(dev(dgu), aq, asc)
    M.moe_quantize_fp8_transposed(w["w_gateup"].reshape(E, 2 * f, d), wq, wsc)
    M.moe_grouped_gemm_fp8("none", E, A, d, 2 * f, g["saved"]["offsets"], aq, asc, wq, wsc, dx)
    torch.cuda.synchronize()

    off = g["saved"]["offsets"].cpu().numpy().astype(np.int64)
    counts = np.diff(off)
    nz = np.where(counts > 0)[0]
    experts = [int(nz[np.argmax(counts[nz])]), int(nz[np.argmin(counts[nz])])]
    experts += [int(e) for e in rng.choice(np.setdiff1d(nz, experts), size=4, replace=False)]
    dx_all, aq_h, asc_h = host(dx), aq.cpu().numpy(), asc.cpu().numpy()
    for e in experts:
        lo, hi = int(off[e]), int(off[e + 1])
        rows = np.unique(np.concatenate([[lo, hi - 1], rng.integers(lo, hi, size=min(30, hi - lo))]))
        print(f"[full] fp8 data gradient: expert {e} ({hi - lo} rows), {rows.size} sampled", flush=True)
        qa, sa = O.quantize_rowwise(synth.bf16_bits_to_f32(dgu[rows]))
        qw, sw = O.quantize_rowwise_transposed(synth.as_f64(inp["w_gateup"][e], "bf16")[None])
        assert np.array_equal(aq_h[rows], qa) and np.array_equal(asc_h[rows], sa), "dGU row codes/scales"
        assert np.array_equal(wq[e].cpu().numpy(), qw[0]) and np.array_equal(wsc[e].cpu().numpy(), sw[0]), \
            "transposed weight codes/scales"
        ref = O.grouped_gemm_fp8_nt(qa, sa, qw, sw, np.array([0, rows.size]))
        assert_rounded(dx_all[rows], ref, "bf16", f"dX, expert {e}")


def test_full_size_fp8_down_data_gradient():
    """The fp8 down data gradient with the dSwiGLU epilogue as the benchmark
    times it (7B-style routing, 98304 rows, dY~ ~ N(0, 0.2^2) and the
    pre-activations G | U ~ N(0, 1) drawn on the host, W_d quantised along d
    and stored transposed), checked on sampled rows of six experts: codes and
    scales bit-exact, dG | dU within one bf16 rounding plus the noise dH may
    carry through the dSwiGLU factors."""
    cfg = synth.CONFIG_BY_NAME["moe7b_bf16"]
    print(f"[full] {cfg.name} fp8 down data gradient: generating inputs", flush=True)
    inp = synth.make_inputs(cfg, with_dy=False)
    w = R.upload_layer(cfg, inp)
    x = dev(inp["x"])
    g = R.run_gpu(cfg, inp, backward=False, weights=w, x=x, keep_device=True, gather=True)
    A, d, E, f = cfg.T * cfg.k, cfg.d, cfg.E, cfg.f
    rng = np.random.default_rng(14)
    dyb = synth.f32_to_bf16_bits((rng.standard_normal((A, d), dtype=np.float32) * 0.2).astype(np.float32))
    preb = synth.f32_to_bf16_bits(rng.standard_normal((A, 2 * f), dtype=np.float32))
    aq = torch.empty(A, d, dtype=torch.uint8, device="cuda")
    asc = torch.empty(A, dtype=torch.float32, device="cuda")
    wq = torch.empty(E, f, d, dtype=torch.uint8, device="cuda")
    wsc = torch.empty(E, f, dtype=torch.float32, device="cuda")
    dgu = torch.empty(A, 2 * f, dtype=torch.bfloat16, device="cuda")
    print(f"[full] {cfg.name} fp8 down data gradient: GPU quantisation and grouped GEMM", flush=True)
    M.moe_quantize_fp8(dev(dyb), aq, asc)
    M.moe_quantize_fp8_transposed(w["w_down"].reshape(E, d, f), wq, wsc)
    M.moe_grouped_gemm_fp8("dswiglu", E, A, f, d, g["saved"]["offsets"], aq, asc, wq, wsc, dgu, dev(preb))
    torch.cuda.synchronize()

    off = g["saved"]["offsets"].cpu().numpy().astype(np.int64)
    counts = np.diff(off)
    nz = np.where(counts > 0)[0]
    experts = [int(nz[np.argmax(counts[nz])]), int(nz[np.argmin(counts[nz])])]
    experts += [int(e) for e in rng.choice(np.setdiff1d(nz, experts), size=4, replace=False)]
    out, aq_h, asc_h = host(dgu), aq.cpu().numpy(), asc.cpu().numpy()
    z, zw = None, np.zeros((f, 1))
    for e in experts:
        lo, hi = int(off[e]), int(off[e + 1])
        rows = np.unique(np.concatenate([[lo, hi - 1], rng.integers(lo, hi, size=min(30, hi - lo))]))
        print(f"[full] fp8 down data gradient: expert {e} ({hi - lo} rows), {rows.size} sampled", flush=True)
        qa, sa = O.quantize_rowwise(synth.bf16_bits_to_f32(dyb[rows]))
        qw, sw = O.quantize_rowwise_transposed(synth.as_f64(inp["w_down"][e], "bf16")[None])
        assert np.array_equal(aq_h[rows], qa) and np.array_equal(asc_h[rows], sa), "dY~ row codes/scales"
        assert np.array_equal(wq[e].cpu().numpy(), qw[0]) and np.array_equal(wsc[e].cpu().numpy(), sw[0]), \
            "transposed weight codes/scales"
        dH = O.grouped_gemm_fp8_nt(qa, sa, qw, sw, np.array([0, rows.size]))
        pre = synth.bf16_bits_to_f32(preb[rows]).astype(np.float64)
        Gm, U = pre[:, :f], pre[:, f:]
        z = np.zeros((rows.size, 1))
        _, _, _, _, dG, dU = O.swiglu_ffn_backward(z, zw, zw, np.eye(f), Gm, U, O.silu(Gm) * U, dH)
        err = 1e-4 * np.sqrt(np.mean(dH * dH))
        sg = 1.0 / (1.0 + np.exp(-Gm))
        inherited = np.concatenate([np.abs(U * sg * (1.0 + Gm * (1.0 - sg))), np.abs(O.silu(Gm))], axis=1) * err
        assert_rounded(out[rows], np.concatenate([dG, dU], axis=1), "bf16", f"dG | dU, expert {e}",
                       extra=inherited)
