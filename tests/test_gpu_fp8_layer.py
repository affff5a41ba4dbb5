"""The fp8 layer calls (moe_fp8_weights_quantize, moe_forward_fp8,
moe_backward_fp8) and the gathered fp8 grouped GEMM on the GPU against the
oracle's fp8 mode.

Protocol for the layer.  A quantised product is sensitive to which way
its bf16 input rounded: two correct evaluations whose fp32 (GPU) and fp64
(oracle) sums straddle a bf16 rounding boundary hold inputs one bf16 step
apart, and where that element is a row's largest the row's scale moves and
with it every code of the row (measured: a few per cent of dx on single
tokens).  So every quantised input is taken from the GPU after it is checked
to be a correct rounding of the oracle's own value, and the oracle then runs
on it, as it follows the GPU's expert choice on near-ties:
  * routing is checked on every token against the oracle's router and the
    oracle follows the GPU's expert indices (no token is dropped) and its
    fp32 gates (checked against the oracle's to 1e-5);
  * H = silu(G) U (and the shared H): the GPU's bf16 copy is checked element
    by element to be one bf16 rounding of the oracle's H plus the fp32 noise
    G and U may carry, then forced as the down products' input;
  * dG | dU (routed and shared), the operand of the gate/up data gradients:
    formed by the same kernels through the public calls (shown to be
    moe_backward_fp8's own by the weight gradients, which read them and must
    agree bit for bit), checked to be one rounding of the oracle's values on
    the GPU's stored pre-activations (which are themselves checked), then
    forced; the gate-weighted dY~ needs no forcing: with the same gates it is
    one fp32 product rounded once on both sides;
  * pre-activations, H, dG | dU and the routed down outputs are one bf16
    rounding of the oracle's values (assert_rounded, plus the fp32 summation
    bound); y, dx and every gradient meet the bf16 bar (rel-L2 <= 1e-2,
    max-abs <= 5e-2 RMS).
"""
import numpy as np
import pytest
import torch

import synth
from oracle import moe_oracle as O
from tests.gpu_util import assert_close, assert_rounded, dev, host

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import mixture_experts_layer_18_amd as M
    from tests import layer_runner as R

SMALL = synth.CONFIG_BY_NAME["finegrained_bf16"].replace(
    name="fp8_small", T=600, d=256, E=8, k=2, f=256, n_shared=1, f_shared=256, backward=True, seed=3)
FINE = synth.CONFIG_BY_NAME["finegrained_bf16"].replace(backward=True)


def _bf16(g, shape, scale=1.0):
    return synth.f32_to_bf16_bits((g.standard_normal(shape) * scale).astype(np.float32))


def _h_noise(preact, f):
    """Bound on what H = silu(G) U inherits from the fp32 noise of G and U
    (1e-4 of their RMS each), through |dH/dG| and |dH/dU|."""
    Gm, U = preact[:, :f], preact[:, f:]
    e = 1e-4 * np.sqrt(np.mean(preact * preact))
    sg = 1.0 / (1.0 + np.exp(-Gm))
    return (np.abs(sg * (1.0 + Gm * (1.0 - sg)) * U) + np.abs(O.silu(Gm))) * e


def _fp8_sum_bound(a, b):
    """K u sum_k |a'_k b'_k| with a', b' the values of the row-wise e4m3 copies
    of a [M, K] and b [N, K] and u = 2^-24: the standard bound on what fp32
    summation of the K exact products, in any order, adds to their sum."""
    qa, sa = O.quantize_rowwise(a)
    qb, sb = O.quantize_rowwise(b)
    A = np.abs(O.e4m3_decode(qa)) * sa[:, None].astype(np.float64)
    B = np.abs(O.e4m3_decode(qb)) * sb[:, None].astype(np.float64)
    return a.shape[1] * 2.0 ** -24 * (A @ B.T)


def test_fp8_weights_quantize_bit_exact():
    """moe_fp8_weights_quantize writes the oracle's codes and scales bit for
    bit: forward layout row-wise along d (gate/up) and f (down), data-gradient
    layout along 2f and d stored transposed, shared experts alike."""
    cfg = SMALL
    inp = synth.make_inputs(cfg, with_dy=False)
    desc = M.desc_from_config(cfg)
    w = R.upload_layer(cfg, inp)
    w8 = M.alloc_fp8_weights(desc)
    M.moe_fp8_weights_quantize(desc, w, w8)
    torch.cuda.synchronize()
    oi = R.oracle_inputs(cfg, inp)
    E, f, d = cfg.E, cfg.f, cfg.d
    F = cfg.F_shared
    gu, dn = oi["w_gateup"], oi["w_down"]
    q, s = O.quantize_rowwise(gu.reshape(E * 2 * f, d))
    assert np.array_equal(w8["gateup_q"].cpu().numpy().reshape(E * 2 * f, d), q)
    assert np.array_equal(w8["gateup_s"].cpu().numpy().ravel(), s)
    q, s = O.quantize_rowwise(dn.reshape(E * d, f))
    assert np.array_equal(w8["down_q"].cpu().numpy().reshape(E * d, f), q)
    assert np.array_equal(w8["down_s"].cpu().numpy().ravel(), s)
    q, s = O.quantize_rowwise_transposed(gu)
    assert np.array_equal(w8["gateup_tq"].cpu().numpy(), q) and np.array_equal(w8["gateup_ts"].cpu().numpy(), s)
    q, s = O.quantize_rowwise_transposed(dn)
    assert np.array_equal(w8["down_tq"].cpu().numpy(), q) and np.array_equal(w8["down_ts"].cpu().numpy(), s)
    sg, sd = oi["s_gateup"].astype(np.float32), oi["s_down"].astype(np.float32)
    q, s = O.quantize_rowwise(sg)
    assert np.array_equal(w8["s_gateup_q"].cpu().numpy(), q) and np.array_equal(w8["s_gateup_s"].cpu().numpy(), s)
    q, s = O.quantize_rowwise(sd)
    assert np.array_equal(w8["s_down_q"].cpu().numpy(), q) and np.array_equal(w8["s_down_s"].cpu().numpy(), s)
    q, s = O.quantize_rowwise_transposed(sg[None])
    assert np.array_equal(w8["s_gateup_tq"].cpu().numpy(), q[0])
    assert np.array_equal(w8["s_gateup_ts"].cpu().numpy(), s[0])
    q, s = O.quantize_rowwise_transposed(sd[None])
    assert np.array_equal(w8["s_down_tq"].cpu().numpy(), q[0]) and np.array_equal(w8["s_down_ts"].cpu().numpy(), s[0])
    assert F == 256


@pytest.mark.parametrize("epi,N", [("none", 384), ("swiglu", 512)])
def test_grouped_gemm_fp8_gather_against_oracle(epi, N):
    """The gathered fp8 product: token rows quantised once per token, routed
    row m reading the codes and scale of token rows[m] (tokens repeated across
    groups, a ragged tail, an empty group), against the oracle's product of
    the gathered codes and scales."""
    g = np.random.default_rng(50 + N)
    G, K, S = 5, 320, 700
    m = g.integers(40, 300, size=G)
    m[2] = 0
    off = np.zeros(G + 1, np.int32)
    off[1:] = np.cumsum(m)
    Mt = int(off[-1])
    rows = g.integers(0, S, size=Mt).astype(np.int32)
    rows[:3] = [S - 1, 0, S - 1]
    xb = _bf16(g, (S, K))
    bb = _bf16(g, (G * N, K), 1 / np.sqrt(K))
    xq = torch.empty(S, K, dtype=torch.uint8, device="cuda")
    xs = torch.empty(S, dtype=torch.float32, device="cuda")
    M.moe_quantize_fp8(dev(xb), xq, xs)
    bq = torch.empty(G * N, K, dtype=torch.uint8, device="cuda")
    bs = torch.empty(G * N, dtype=torch.float32, device="cuda")
    M.moe_quantize_fp8(dev(bb), bq, bs)
    qxo, sxo = O.quantize_rowwise(synth.bf16_bits_to_f32(xb))
    qbo, sbo = O.quantize_rowwise(synth.bf16_bits_to_f32(bb))
    ref = O.grouped_gemm_fp8_nt(qxo[rows], sxo[rows], qbo.reshape(G, N, K), sbo.reshape(G, N), off)
    print(f"[fp8 gather] {epi} G={G} M={Mt} N={N} K={K} tokens={S}", flush=True)
    r = torch.from_numpy(rows).cuda()
    if epi == "none":
        C = torch.empty(Mt, N, dtype=torch.bfloat16, device="cuda")
        M.moe_grouped_gemm_fp8_gather("none", G, Mt, N, K, dev(off), xq, xs, bq, bs, C, r, S)
        torch.cuda.synchronize()
        assert_rounded(host(C), ref, "bf16", "C")
    else:
        F = N // 2
        C = torch.empty(Mt, F, dtype=torch.bfloat16, device="cuda")
        aux = torch.empty(Mt, N, dtype=torch.bfloat16, device="cuda")
        M.moe_grouped_gemm_fp8_gather("swiglu", G, Mt, N, K, dev(off), xq, xs, bq, bs, C, r, S, aux=aux)
        torch.cuda.synchronize()
        assert_rounded(host(aux), ref, "bf16", "aux")
        assert_rounded(host(C), O.silu(ref[:, :F]) * ref[:, F:], "bf16", "h", extra=_h_noise(ref, F))


def _dswiglu_noise(dh_rms, pre, F):
    """Bound on what dG | dU inherit from the fp32 noise of dH (1e-4 of its
    RMS), through |U silu'(G)| and |silu(G)|, with G | U the bf16 pre-activations."""
    Gm, U = pre[:, :F], pre[:, F:]
    e = 1e-4 * dh_rms
    sg = 1.0 / (1.0 + np.exp(-Gm))
    return np.concatenate([np.abs(U * sg * (1.0 + Gm * (1.0 - sg))), np.abs(O.silu(Gm))], axis=1) * e


def _gpu_dgu(cfg, sv, w8, dy, fmt="e4m3"):
    """dG | dU as moe_backward_fp8 forms them, from the same kernels through
    the public calls: the gate-weighted rows dY~ = bf16(gate * dy) (one fp32
    product, rounded to nearest even), their row-wise e4m3 copy, and the fp8
    down data gradient with the dSwiGLU epilogue on the saved
    pre-activations; the shared experts' from dy itself.  Also the RMS of the
    data gradients dH themselves (the same products without the epilogue)."""
    T, d, E, k, f, F = cfg.T, cfg.d, cfg.E, cfg.k, cfg.f, cfg.F_shared
    A = T * k
    src = sv["src"].long()
    dyp = (sv["gate"].reshape(-1)[src].unsqueeze(1) * dy.float()[src // k]).to(torch.bfloat16)
    q = torch.empty(A, d, dtype=torch.uint8, device="cuda")
    qs = torch.empty(A, dtype=torch.float32, device="cuda")
    M.moe_quantize_fp8(dyp, q, qs, fmt=fmt)
    dgu = torch.empty(A, 2 * f, dtype=torch.bfloat16, device="cuda")
    M.moe_grouped_gemm_fp8("dswiglu", E, A, f, d, sv["offsets"], q, qs, w8["down_tq"], w8["down_ts"], dgu,
                           sv["preact"], a_fmt=fmt)
    dh = torch.empty(A, f, dtype=torch.bfloat16, device="cuda")
    M.moe_grouped_gemm_fp8("none", E, A, f, d, sv["offsets"], q, qs, w8["down_tq"], w8["down_ts"], dh,
                           a_fmt=fmt)
    rms = [float(dh.float().pow(2).mean().sqrt())]
    s_dgu = None
    if F:
        M.moe_quantize_fp8(dy, q[:T], qs[:T], fmt=fmt)
        s_dgu = torch.empty(T, 2 * F, dtype=torch.bfloat16, device="cuda")
        M.moe_grouped_gemm_fp8("dswiglu", 1, T, F, d, None, q[:T], qs[:T], w8["s_down_tq"], w8["s_down_ts"], s_dgu,
                               sv["s_preact"], a_fmt=fmt)
        sdh = torch.empty(T, F, dtype=torch.bfloat16, device="cuda")
        M.moe_grouped_gemm_fp8("none", 1, T, F, d, None, q[:T], qs[:T], w8["s_down_tq"], w8["s_down_ts"], sdh,
                               a_fmt=fmt)
        rms.append(float(sdh.float().pow(2).mean().sqrt()))
    return dgu, s_dgu, rms


def _fp8_wgrad_gpu(G, offsets, a, b, b_rows=None):
    """An fp8 weight gradient C[g] = a_g^T b_g through the public calls: both
    operands quantised column-wise over each group's rows (b read through
    b_rows when given), then the scaled product.  Returns C [G, N, K] bf16."""
    Mrows = a.shape[0]
    N, K = a.shape[1], b.shape[1]
    pad = torch.empty(G + 1, dtype=torch.int32, device="cuda")
    qa = torch.empty(M.quantize_fp8_colwise_bytes(G, Mrows, N), dtype=torch.uint8, device="cuda")
    qb = torch.empty(M.quantize_fp8_colwise_bytes(G, Mrows, K), dtype=torch.uint8, device="cuda")
    sa = torch.empty(G, N, dtype=torch.float32, device="cuda")
    sb = torch.empty(G, K, dtype=torch.float32, device="cuda")
    M.moe_quantize_fp8_colwise(a, G, offsets, pad, qa, sa)
    M.moe_quantize_fp8_colwise(b, G, offsets, pad, qb, sb, rows=b_rows, M=Mrows)
    C = torch.empty(G, N, K, dtype=torch.bfloat16, device="cuda")
    M.moe_grouped_gemm_fp8_wgrad(G, N, K, pad, qa, sa, qb, sb, C)
    return C


def _compare_fp8_layer(cfg, gather, grad_format="e4m3", wgrad_fp8=False, paired=False):
    print(f"[fp8 layer] {cfg.name} gather={gather} gradients {grad_format} fp8 weight gradients {wgrad_fp8}: inputs",
          flush=True)
    inp = synth.make_inputs(cfg, with_dy=True)
    desc = M.desc_from_config(cfg)
    w = R.upload_layer(cfg, inp)
    x, dy = dev(inp["x"]), dev(inp["dy"])
    print(f"[fp8 layer] {cfg.name}: GPU fp8 forward+backward", flush=True)
    g = R.run_gpu(cfg, inp, backward=True, weights=w, x=x, dy=dy, keep_device=True, gather=gather, fp8=True,
                  grad_format=grad_format, wgrad_fp8=wgrad_fp8)
    sv, w8 = g["saved"], g["w8"]
    g_idx = sv["idx"].cpu().numpy()
    g_gate = sv["gate"].cpu().numpy()
    oi = R.oracle_inputs(cfg, inp)
    rt = R.oracle_routing(cfg, oi)
    R.check_routing(cfg, sv["logits"].cpu().numpy(), g_idx, rt)
    # the GPU's gates on its own routing: the oracle's gate values up to the
    # logits' fp32 noise
    o_gate = O.gates_from_scores(rt["scores"], g_idx, cfg.score, cfg.renorm)
    assert np.max(np.abs(g_gate.astype(np.float64) - o_gate)) <= 1e-5
    f, F = cfg.f, cfg.F_shared
    gh = host(sv["h"])
    gsh = host(sv["s_h"]) if F else None
    print(f"[fp8 layer] {cfg.name}: oracle fp8 forward on the GPU's routing", flush=True)
    fw = O.forward(oi["x"], oi["w_router"], oi["bias"], oi["w_gateup"], oi["w_down"], oi["s_gateup"],
                   oi["s_down"], top_k=cfg.k, score=cfg.score, renorm=cfg.renorm, forced_idx=g_idx,
                   forced_gate=g_gate, fp8=True, forced_h=gh, forced_s_h=gsh)
    # the forced copies are correct roundings of the oracle's own values
    gpre = host(sv["preact"])
    assert_rounded(gpre, fw["preact"], "bf16", "preact")
    assert_rounded(gh, fw["h"], "bf16", "h", extra=_h_noise(fw["preact"], f))
    flips = int(np.sum(gh != O.round_bf16(fw["h"])))
    print(f"[fp8 layer] {cfg.name}: H elements whose bf16 rounding differs from the oracle's: {flips} of {gh.size}",
          flush=True)
    gspre = None
    if F:
        gspre = host(sv["s_preact"])
        assert_rounded(gspre, fw["s_preact"], "bf16", "s_preact")
        assert_rounded(gsh, fw["s_h"], "bf16", "s_h", extra=_h_noise(fw["s_preact"], F))
    # the routed down outputs: one rounding of the product of identical
    # codes, plus what fp32 summation over f may add
    off = fw["offsets"]
    acc = np.zeros_like(fw["y_perm"])
    for e in range(cfg.E):
        r0, r1 = int(off[e]), int(off[e + 1])
        if r1 > r0:
            acc[r0:r1] = _fp8_sum_bound(gh[r0:r1], oi["w_down"][e])
    assert_rounded(host(sv["y_perm"]), fw["y_perm"], "bf16", "y_perm", extra=acc)
    assert_close(host(g["y"]), fw["y"], cfg.dtype, "y")

    # --- backward: the operands the gate/up data gradients quantise, formed
    # by the same kernels through the public calls; the weight gradients that
    # read them show they are the ones moe_backward_fp8 formed (bit for bit)
    print(f"[fp8 layer] {cfg.name}: dG | dU through the public calls", flush=True)
    dgu, s_dgu, dh_rms = _gpu_dgu(cfg, sv, w8, dy, grad_format)
    T, d, E, k = cfg.T, cfg.d, cfg.E, cfg.k
    A = T * k
    if wgrad_fp8:
        dwg = _fp8_wgrad_gpu(E, sv["offsets"], dgu, x if gather else sv["x_perm"], sv["tok"] if gather else None)
    else:
        dwg = torch.empty(E, 2 * f, d, dtype=torch.bfloat16, device="cuda")
        if gather:
            M.moe_grouped_gemm_gather("TN", "none", E, A, 2 * f, d, sv["offsets"], dgu, x, dwg, sv["tok"], T)
        else:
            M.moe_grouped_gemm("TN", "none", "bf16", E, A, 2 * f, d, sv["offsets"], dgu, sv["x_perm"], dwg,
                               ws=torch.empty(max(M.grouped_gemm_workspace_bytes("TN", "bf16", E, A, 2 * f, d), 16),
                                              dtype=torch.uint8, device="cuda"))
    torch.cuda.synchronize()
    assert torch.equal(dwg.view(torch.int16), g["grads"]["d_w_gateup"].view(torch.int16))
    if F:
        if wgrad_fp8:
            dsg = _fp8_wgrad_gpu(1, None, s_dgu, x)[0]
        elif paired:
            # the layer ran the shared weight gradient inside the routed
            # (gathered) launch: the same tiles, each over all rows in order,
            # as the gathered product of one group through the identity map
            dsg = torch.empty(2 * F, d, dtype=torch.bfloat16, device="cuda")
            iota = torch.arange(T, dtype=torch.int32, device="cuda")
            M.moe_grouped_gemm_gather("TN", "none", 1, T, 2 * F, d, None, s_dgu, x, dsg, iota, T)
        else:
            dsg = torch.empty(2 * F, d, dtype=torch.bfloat16, device="cuda")
            nws = M.grouped_gemm_workspace_bytes("TN", "bf16", 1, T, 2 * F, d)
            M.moe_grouped_gemm("TN", "none", "bf16", 1, T, 2 * F, d, None, s_dgu, x, dsg,
                               ws=torch.empty(max(nws, 16), dtype=torch.uint8, device="cuda"))
        torch.cuda.synchronize()
        assert torch.equal(dsg.view(torch.int16), g["grads"]["d_s_gateup"].view(torch.int16))
    gdgu = host(dgu)
    gsdgu = host(s_dgu) if F else None
    print(f"[fp8 layer] {cfg.name}: oracle fp8 backward (stored pre-activations and dG | dU forced)", flush=True)
    fwb = dict(fw, preact=gpre, s_preact=gspre)
    bw = O.backward(oi["x"], oi["w_router"], oi["w_gateup"], oi["w_down"], oi["s_gateup"], oi["s_down"], fwb,
                    oi["dy"], score=cfg.score, renorm=cfg.renorm, fp8=True, forced_dgu=gdgu, forced_s_dgu=gsdgu,
                    fp8_grad_format=grad_format, fp8_wgrad=wgrad_fp8)
    assert_rounded(gdgu, bw["dgu"], "bf16", "dG | dU", extra=_dswiglu_noise(dh_rms[0], gpre, f))
    if F:
        assert_rounded(gsdgu, bw["s_dgu"], "bf16", "shared dG | dU", extra=_dswiglu_noise(dh_rms[1], gspre, F))
    assert_close(host(g["dx"]), bw["dx"], cfg.dtype, "dx")
    for name in ("d_w_gateup", "d_w_down", "d_s_gateup", "d_s_down"):
        if g["grads"][name] is not None:
            assert_close(host(g["grads"][name]), bw[name], cfg.dtype, name)
    assert_close(g["grads"]["d_w_router"].cpu().numpy(), bw["d_w_router"], cfg.dtype, "d_w_router")
    return g, fw, bw


@pytest.mark.parametrize("gather", [True, False], ids=["gather", "permuted-copy"])
def test_fp8_layer_small_against_oracle(gather):
    """A small fp8 layer (600 tokens: a ragged tail; 8 experts, top-2, one
    shared expert), forward and backward compared in full; with the permuted
    token copy the backward's weight gradient reads it instead of gathering."""
    _compare_fp8_layer(SMALL, gather)


def test_fp8_layer_e5m2_gradients_against_oracle():
    """The small fp8 layer with e5m2 gradient operands (dY~, dG | dU and the
    shared ones quantised to e5m2, weights e4m3), forward and backward
    compared in full."""
    _compare_fp8_layer(SMALL, True, "e5m2")


@pytest.mark.parametrize("cfg", [SMALL, FINE], ids=["small", "finegrained"])
def test_fp8_layer_fp8_weight_gradients_against_oracle(cfg):
    """The fp8 layer with e4m3 weight gradients (operands quantised along each
    expert's rows), forward and backward compared in full; every quantiser
    input is the GPU's after the checks above, so the weight gradients are
    compared against the oracle's fp8 products of the same codes."""
    _compare_fp8_layer(cfg, True, "e4m3", True)


# the routed down weight gradient has 64 x 4 x 4 = 1024 tiles, so the fp8
# backward's bf16 weight gradients run paired with the shared ones
PAIRED = synth.CONFIG_BY_NAME["finegrained_bf16"].replace(
    name="fp8_paired", T=2000, d=1024, E=64, k=4, f=1024, n_shared=1, f_shared=512, backward=True, seed=5)


def test_fp8_layer_paired_weight_gradients_against_oracle():
    """The fp8 layer whose shared weight gradients run inside the routed
    weight-gradient launches, forward and backward compared in full."""
    M.stage_timing(True)
    try:
        _compare_fp8_layer(PAIRED, True, paired=True)
        torch.cuda.synchronize()
        st = M.stage_times()
    finally:
        M.stage_timing(False)
    assert st["down_wgrad"][1] >= 1 and st["shared_down_wgrad"][1] == 0 and st["shared_gate_up_wgrad"][1] == 0


def test_fp8_layer_finegrained_against_oracle():
    """The fine-grained layer's shape (4096 tokens, 64 experts, top-8, one
    shared expert of 1024) through the fp8 calls, forward and backward,
    compared in full."""
    _compare_fp8_layer(FINE, True)


def test_fp8_layer_matches_its_products():
    """The fp8 forward's gate/up stage equals the gathered fp8 GEMM run on its
    own on the token rows quantised per token (same codes and scales): the
    saved H and pre-activations agree bit for bit."""
    cfg = SMALL
    inp = synth.make_inputs(cfg, with_dy=True)
    w = R.upload_layer(cfg, inp)
    x = dev(inp["x"])
    g = R.run_gpu(cfg, inp, backward=True, weights=w, x=x, keep_device=True, gather=True, fp8=True)
    sv, w8 = g["saved"], g["w8"]
    T, d, E, f, A = cfg.T, cfg.d, cfg.E, cfg.f, cfg.T * cfg.k
    xq = torch.empty(T, d, dtype=torch.uint8, device="cuda")
    xs = torch.empty(T, dtype=torch.float32, device="cuda")
    M.moe_quantize_fp8(x, xq, xs)
    h = torch.empty(A, f, dtype=torch.bfloat16, device="cuda")
    aux = torch.empty(A, 2 * f, dtype=torch.bfloat16, device="cuda")
    M.moe_grouped_gemm_fp8_gather("swiglu", E, A, 2 * f, d, sv["offsets"], xq, xs, w8["gateup_q"], w8["gateup_s"],
                                  h, sv["tok"], T, aux=aux)
    torch.cuda.synchronize()
    assert torch.equal(h.view(torch.int16), sv["h"].view(torch.int16))
    assert torch.equal(aux.view(torch.int16), sv["preact"].view(torch.int16))


def test_fp8_layer_full_size_experts():
    """The 7B-style layer (16384 tokens, 64 experts, top-6, two shared
    experts) through moe_forward_fp8 + moe_backward_fp8 in the benchmark's
    launch configuration (token rows gathered), checked on every row of four
    experts (the largest, the smallest non-empty one and two more): the
    pre-activations, H and the down outputs (on the GPU's H) against the
    oracle's fp8 products; dG | dU (formed through the public calls from the
    same kernels, and shown to be the layer's own by the gate/up weight
    gradient, bit for bit) against the oracle's on the GPU's dY~ rows and
    stored pre-activations; and those experts' weight gradients, bf16
    products of the GPU's bf16 operands, against their exact products."""
    cfg = synth.CONFIG_BY_NAME["moe7b_bf16"]
    print(f"[fp8 full] {cfg.name}: inputs", flush=True)
    inp = synth.make_inputs(cfg, with_dy=True)
    w = R.upload_layer(cfg, inp)
    x, dy = dev(inp["x"]), dev(inp["dy"])
    print(f"[fp8 full] {cfg.name}: GPU fp8 forward+backward", flush=True)
    g = R.run_gpu(cfg, inp, backward=True, weights=w, x=x, dy=dy, keep_device=True, gather=True, fp8=True)
    sv, w8 = g["saved"], g["w8"]
    T, d, E, k, f = cfg.T, cfg.d, cfg.E, cfg.k, cfg.f
    A = T * k
    dgu, _, dh_rms = _gpu_dgu(cfg, sv, w8, dy)
    dwg = torch.empty(E, 2 * f, d, dtype=torch.bfloat16, device="cuda")
    M.moe_grouped_gemm_gather("TN", "none", E, A, 2 * f, d, sv["offsets"], dgu, x, dwg, sv["tok"], T)
    torch.cuda.synchronize()
    assert torch.equal(dwg.view(torch.int16), g["grads"]["d_w_gateup"].view(torch.int16))
    off = sv["offsets"].cpu().numpy().astype(np.int64)
    tok = sv["tok"].cpu().numpy().astype(np.int64)
    src = sv["src"].cpu().numpy().astype(np.int64)
    gate = sv["gate"].cpu().numpy().reshape(-1)
    counts = np.diff(off)
    nz = np.where(counts > 0)[0]
    rng = np.random.default_rng(21)
    experts = [int(nz[np.argmax(counts[nz])]), int(nz[np.argmin(counts[nz])])]
    experts += [int(e) for e in rng.choice(np.setdiff1d(nz, experts), size=2, replace=False)]
    xf = synth.as_f64(inp["x"], "bf16")
    dyf = synth.as_f64(inp["dy"], "bf16")
    gu_all = synth.bf16_bits_to_f32(inp["w_gateup"])
    dn_all = synth.bf16_bits_to_f32(inp["w_down"])
    for e in experts:
        r0, r1 = int(off[e]), int(off[e + 1])
        print(f"[fp8 full] expert {e}: {r1 - r0} rows", flush=True)
        tk = tok[r0:r1]
        pre = host(sv["preact"][r0:r1])
        gh = host(sv["h"][r0:r1])
        ref = O.fp8_product(xf[tk], gu_all[e])
        assert_rounded(pre, ref, "bf16", f"preact, expert {e}")
        assert_rounded(gh, O.silu(ref[:, :f]) * ref[:, f:], "bf16", f"h, expert {e}", extra=_h_noise(ref, f))
        assert_rounded(host(sv["y_perm"][r0:r1]), O.fp8_product(gh, dn_all[e]), "bf16", f"y_perm, expert {e}",
                       extra=_fp8_sum_bound(gh, dn_all[e]))
        # the gate-weighted rows: one fp32 product of the GPU's gate and dy, rounded once
        dyp = O.round_bf16(gate[src[r0:r1]].astype(np.float64)[:, None] * dyf[tk])
        dH = O.fp8_product(dyp, dn_all[e].astype(np.float64).T)
        Gm, U = pre[:, :f], pre[:, f:]
        sg = 1.0 / (1.0 + np.exp(-Gm))
        dgu_ref = np.concatenate([dH * U * sg * (1.0 + Gm * (1.0 - sg)), dH * Gm * sg], axis=1)
        gdgu = host(dgu[r0:r1])
        assert_rounded(gdgu, dgu_ref, "bf16", f"dG | dU, expert {e}", extra=_dswiglu_noise(dh_rms[0], pre, f))
        # weight gradients: bf16 products of the GPU's bf16 operands
        rows = r1 - r0
        wg_ref = gdgu.T @ xf[tk]
        wg_acc = rows * 2.0 ** -24 * (np.abs(gdgu).T @ np.abs(xf[tk]))
        assert_rounded(host(g["grads"]["d_w_gateup"][e]), wg_ref, "bf16", f"dW_gateup, expert {e}", extra=wg_acc)
        wd_ref = dyp.T @ gh
        wd_acc = rows * 2.0 ** -24 * (np.abs(dyp).T @ np.abs(gh))
        assert_rounded(host(g["grads"]["d_w_down"][e]), wd_ref, "bf16", f"dW_down, expert {e}", extra=wd_acc)


def test_quantize_fp8_colwise_bit_exact():
    """Column-wise codes over each group's rows, stored transposed and padded:
    ragged groups, an empty one, a group of one row, rows read through a map;
    codes and scales bit-exact against the oracle's, zero codes in the
    padding, the padded offsets as defined."""
    g = np.random.default_rng(48)
    G, C = 6, 192
    m = np.array([70, 0, 1, 130, 64, 33])
    off = np.zeros(G + 1, np.int32)
    off[1:] = np.cumsum(m)
    Mrows = int(off[-1])
    S = 400
    xf = (g.standard_normal((S, C)) * np.exp(g.uniform(-3, 3, (1, C)))).astype(np.float32)
    xb = synth.f32_to_bf16_bits(xf)
    rows = g.integers(0, S, size=Mrows).astype(np.int32)
    pad = torch.empty(G + 1, dtype=torch.int32, device="cuda")
    q = torch.full((M.quantize_fp8_colwise_bytes(G, Mrows, C),), 0x55, dtype=torch.uint8, device="cuda")
    s = torch.empty(G, C, dtype=torch.float32, device="cuda")
    M.moe_quantize_fp8_colwise(dev(xb), G, dev(off), pad, q, s, rows=torch.from_numpy(rows).cuda(), M=Mrows)
    torch.cuda.synchronize()
    pm = (m + 63) // 64 * 64
    want_pad = np.concatenate([[0], np.cumsum(pm)])
    assert np.array_equal(pad.cpu().numpy(), want_pad)
    qh, sh = q.cpu().numpy(), s.cpu().numpy()
    xv = synth.bf16_bits_to_f32(xb)
    for e in range(G):
        blk = qh[C * want_pad[e]: C * want_pad[e + 1]].reshape(C, pm[e])
        if m[e] == 0:
            assert np.all(sh[e] == 1.0)
            continue
        qo, so = O.quantize_colwise(xv[rows[off[e]:off[e + 1]]])
        assert np.array_equal(sh[e], so), e
        assert np.array_equal(blk[:, :m[e]], qo.T), e
        assert not blk[:, m[e]:].any(), e


def test_grouped_gemm_fp8_wgrad_against_oracle():
    """The fp8 weight gradient C[g] = a_g^T b_g on ragged groups with an empty
    one (its gradient zero): one bf16 rounding of the oracle's product of the
    same column-wise codes, plus the fp32 summation bound."""
    g = np.random.default_rng(49)
    G, N, K = 5, 192, 320
    m = np.array([300, 0, 129, 64, 211])
    off = np.zeros(G + 1, np.int32)
    off[1:] = np.cumsum(m)
    Mrows = int(off[-1])
    ab = _bf16(g, (Mrows, N), 0.1)
    bb = _bf16(g, (Mrows, K))
    C = _fp8_wgrad_gpu(G, dev(off), dev(ab), dev(bb))
    torch.cuda.synchronize()
    out = host(C)
    av, bv = synth.bf16_bits_to_f32(ab).astype(np.float64), synth.bf16_bits_to_f32(bb).astype(np.float64)
    for e in range(G):
        if m[e] == 0:
            assert not out[e].any()
            continue
        a_e, b_e = av[off[e]:off[e + 1]], bv[off[e]:off[e + 1]]
        ref = O.wgrad_fp8(a_e, b_e)
        qa, sa = O.quantize_colwise(a_e)
        qb, sb = O.quantize_colwise(b_e)
        Ad = np.abs(O.e4m3_decode(qa)) * sa[None, :]
        Bd = np.abs(O.e4m3_decode(qb)) * sb[None, :]
        acc = m[e] * 2.0 ** -24 * (Ad.T @ Bd)
        assert_rounded(out[e], ref, "bf16", f"dW group {e}", extra=acc)
