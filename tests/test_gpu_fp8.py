"""fp8 (e4m3) expert path on the GPU against the oracle: row-wise quantisation
(bit-exact codes and scales) and the scaled fp8 grouped GEMM in the forward
layout, with and without the SwiGLU epilogue."""
import numpy as np
import pytest
import torch

import synth
from oracle import moe_oracle as O
from tests.gpu_util import assert_rounded, dev, host

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import mixture_experts_layer_18_amd as M


def _bf16(g, shape, scale=1.0):
    return synth.f32_to_bf16_bits((g.standard_normal(shape) * scale).astype(np.float32))


def _quant_gpu(xb):
    x = dev(xb)
    R = x.shape[0]
    C = x.numel() // R
    q = torch.empty(R, C, dtype=torch.uint8, device="cuda")
    s = torch.empty(R, dtype=torch.float32, device="cuda")
    M.moe_quantize_fp8(x.reshape(R, C), q, s)
    torch.cuda.synchronize()
    return q, s


def test_quantize_rowwise_bit_exact():
    g = np.random.default_rng(41)
    xb = _bf16(g, (300, 512), 3.0)
    xb[7] = 0                                     # an all-zero row
    xb[8, :5] = synth.f32_to_bf16_bits(np.array([1e-30, -2e-9, 6e4, -3.0, 0.5], np.float32))
    q, s = _quant_gpu(xb)
    qo, so = O.quantize_rowwise(synth.bf16_bits_to_f32(xb))
    assert np.array_equal(s.cpu().numpy(), so)
    assert np.array_equal(q.cpu().numpy(), qo)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_quantize_tensorwise_bit_exact(dtype):
    g = np.random.default_rng(43)
    xf = (g.standard_normal((257, 384)) * np.exp(g.uniform(-4, 4, (257, 1)))).astype(np.float32)
    xf[9] = 0
    if dtype == "bf16":
        xb = synth.f32_to_bf16_bits(xf)
        xv = synth.bf16_bits_to_f32(xb)
        x = dev(xb)
    else:
        xv = xf
        x = torch.from_numpy(xf).cuda()
    q = torch.empty(x.shape[0], x.shape[1], dtype=torch.uint8, device="cuda")
    s = torch.empty(x.shape[0], dtype=torch.float32, device="cuda")
    M.moe_quantize_fp8_tensorwise(x, q, s)
    torch.cuda.synchronize()
    qo, so = O.quantize_tensorwise(xv)
    assert np.all(s.cpu().numpy() == so)
    assert np.array_equal(q.cpu().numpy(), qo)
    # an all-zero tensor
    z = torch.zeros(5, 64, dtype=x.dtype, device="cuda")
    qz = torch.full((5, 64), 7, dtype=torch.uint8, device="cuda")
    sz = torch.empty(5, dtype=torch.float32, device="cuda")
    M.moe_quantize_fp8_tensorwise(z, qz, sz)
    torch.cuda.synchronize()
    assert np.all(sz.cpu().numpy() == 1.0) and not qz.cpu().numpy().any()


def test_grouped_gemm_fp8_tensorwise_activations():
    """Tensor-wise activations with row-wise weights through the same GEMM."""
    g = np.random.default_rng(44)
    G, N, K = 4, 256, 256
    off = np.array([0, 90, 90, 300, 333], np.int32)
    Mt = int(off[-1])
    ab = _bf16(g, (Mt, K))
    bb = _bf16(g, (G * N, K), 1 / np.sqrt(K))
    a = dev(ab)
    qa = torch.empty(Mt, K, dtype=torch.uint8, device="cuda")
    sa = torch.empty(Mt, dtype=torch.float32, device="cuda")
    M.moe_quantize_fp8_tensorwise(a, qa, sa)
    qb, sb = _quant_gpu(bb)
    qao, sao = O.quantize_tensorwise(synth.bf16_bits_to_f32(ab))
    qbo, sbo = O.quantize_rowwise(synth.bf16_bits_to_f32(bb))
    ref = O.grouped_gemm_fp8_nt(qao, np.full(Mt, sao, np.float32), qbo.reshape(G, N, K), sbo.reshape(G, N), off)
    C = torch.empty(Mt, N, dtype=torch.bfloat16, device="cuda")
    M.moe_grouped_gemm_fp8("none", G, Mt, N, K, dev(off), qa, sa, qb, sb, C)
    torch.cuda.synchronize()
    assert_rounded(host(C), ref, "bf16", "C")


@pytest.mark.parametrize("epi,N", [("none", 384), ("swiglu", 512)])
def test_grouped_gemm_fp8_against_oracle(epi, N):
    g = np.random.default_rng(42 + N)
    G, K = 6, 320
    m = g.integers(20, 300, size=G)
    m[1] = 0
    off = np.zeros(G + 1, np.int32)
    off[1:] = np.cumsum(m)
    Mt = int(off[-1])
    ab = _bf16(g, (Mt, K))
    bb = _bf16(g, (G * N, K), 1 / np.sqrt(K))
    qa, sa = _quant_gpu(ab)
    qb, sb = _quant_gpu(bb)
    qao, sao = O.quantize_rowwise(synth.bf16_bits_to_f32(ab))
    qbo, sbo = O.quantize_rowwise(synth.bf16_bits_to_f32(bb))
    ref = O.grouped_gemm_fp8_nt(qao, sao, qbo.reshape(G, N, K), sbo.reshape(G, N), off)
    print(f"[fp8] {epi} G={G} M={Mt} N={N} K={K}", flush=True)
    if epi == "none":
        C = torch.empty(Mt, N, dtype=torch.bfloat16, device="cuda")
        M.moe_grouped_gemm_fp8("none", G, Mt, N, K, dev(off), qa, sa, qb, sb, C)
        torch.cuda.synchronize()
        assert_rounded(host(C), ref, "bf16", "C")
    else:
        F = N // 2
        C = torch.empty(Mt, F, dtype=torch.bfloat16, device="cuda")
        aux = torch.empty(Mt, N, dtype=torch.bfloat16, device="cuda")
        M.moe_grouped_gemm_fp8("swiglu", G, Mt, N, K, dev(off), qa, sa, qb, sb, C, aux)
        torch.cuda.synchronize()
        assert_rounded(host(aux), ref, "bf16", "aux")
        # h = silu(G) * U comes from the fp32 G and U, which may each carry
        # the accumulation noise allowed above (1e-4 of their RMS); that
        # noise reaches h through the two partial derivatives before h is
        # rounded once
        Gm, U = ref[:, :F], ref[:, F:]
        e = 1e-4 * np.sqrt(np.mean(ref * ref))
        sg = 1.0 / (1.0 + np.exp(-Gm))
        dsilu = sg * (1.0 + Gm * (1.0 - sg))
        inherited = (np.abs(dsilu * U) + np.abs(O.silu(Gm))) * e
        assert_rounded(host(C), O.silu(Gm) * U, "bf16", "h", extra=inherited)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_quantize_transposed_bit_exact(dtype):
    """Quantisation along the first axis, stored transposed: codes and scales
    equal the oracle's bit for bit (an all-zero column, extreme values, 320
    columns: five 64-column tiles)."""
    g = np.random.default_rng(43)
    G, R, C = 3, 192, 320
    w = (g.standard_normal((G, R, C)) * np.exp(g.standard_normal(C))[None, None, :]).astype(np.float32)
    w[1, :, 7] = 0.0
    w[2, 5, :4] = np.array([1e-30, -2e-9, 6e4, -3.0], np.float32)
    if dtype == "bf16":
        wb = synth.f32_to_bf16_bits(w)
        src, ref_in = dev(wb), synth.bf16_bits_to_f32(wb)
    else:
        src, ref_in = torch.from_numpy(w).cuda(), w
    q = torch.empty(G, C, R, dtype=torch.uint8, device="cuda")
    s = torch.empty(G, C, dtype=torch.float32, device="cuda")
    M.moe_quantize_fp8_transposed(src, q, s)
    torch.cuda.synchronize()
    qo, so = O.quantize_rowwise_transposed(ref_in)
    assert np.array_equal(s.cpu().numpy(), so)
    assert np.array_equal(q.cpu().numpy(), qo)


def test_fp8_data_gradient_against_oracle():
    """The data gradient dX = dGU . W (W [G, N, K], reduction over N) in fp8:
    dGU quantised row-wise, W quantised along N and stored transposed, the
    product run by the forward-layout fp8 GEMM; ragged groups and an empty
    one."""
    g = np.random.default_rng(44)
    G, N, K = 5, 384, 256
    m = g.integers(30, 260, size=G)
    m[2] = 0
    off = np.zeros(G + 1, np.int32)
    off[1:] = np.cumsum(m)
    Mt = int(off[-1])
    db = _bf16(g, (Mt, N), 0.1)
    wb = _bf16(g, (G, N, K), 1 / np.sqrt(N))
    qa, sa = _quant_gpu(db)
    qw = torch.empty(G, K, N, dtype=torch.uint8, device="cuda")
    sw = torch.empty(G, K, dtype=torch.float32, device="cuda")
    M.moe_quantize_fp8_transposed(dev(wb), qw, sw)
    C = torch.empty(Mt, K, dtype=torch.bfloat16, device="cuda")
    print(f"[fp8] data gradient G={G} M={Mt} N={N} K={K}", flush=True)
    M.moe_grouped_gemm_fp8("none", G, Mt, K, N, dev(off), qa, sa, qw, sw, C)
    torch.cuda.synchronize()
    qao, sao = O.quantize_rowwise(synth.bf16_bits_to_f32(db))
    qwo, swo = O.quantize_rowwise_transposed(synth.bf16_bits_to_f32(wb))
    assert np.array_equal(qw.cpu().numpy(), qwo) and np.array_equal(sw.cpu().numpy(), swo)
    ref = O.grouped_gemm_fp8_nt(qao, sao, qwo, swo, off)
    assert_rounded(host(C), ref, "bf16", "dX")


def test_fp8_down_data_gradient_dswiglu_against_oracle():
    """The down projection's data gradient in fp8 with the dSwiGLU epilogue:
    dH = dY~ . W_d[e] (W_d [G, d, f], reduction over d) with dY~ quantised
    row-wise and W_d quantised along d and stored transposed, run in the
    forward layout; the epilogue turns dH and the pre-activations G | U into
    dG | dU.  Ragged groups and an empty one."""
    g = np.random.default_rng(45)
    G, d, f = 4, 256, 384
    m = g.integers(30, 260, size=G)
    m[1] = 0
    off = np.zeros(G + 1, np.int32)
    off[1:] = np.cumsum(m)
    Mt = int(off[-1])
    dyb = _bf16(g, (Mt, d))
    wdb = _bf16(g, (G, d, f), 1 / np.sqrt(d))
    preb = _bf16(g, (Mt, 2 * f))
    qa, sa = _quant_gpu(dyb)
    qw = torch.empty(G, f, d, dtype=torch.uint8, device="cuda")
    sw = torch.empty(G, f, dtype=torch.float32, device="cuda")
    M.moe_quantize_fp8_transposed(dev(wdb), qw, sw)
    C = torch.empty(Mt, 2 * f, dtype=torch.bfloat16, device="cuda")
    print(f"[fp8] down data gradient + dSwiGLU G={G} M={Mt} d={d} f={f}", flush=True)
    M.moe_grouped_gemm_fp8("dswiglu", G, Mt, f, d, dev(off), qa, sa, qw, sw, C, dev(preb))
    torch.cuda.synchronize()
    qao, sao = O.quantize_rowwise(synth.bf16_bits_to_f32(dyb))
    qwo, swo = O.quantize_rowwise_transposed(synth.bf16_bits_to_f32(wdb))
    dH = O.grouped_gemm_fp8_nt(qao, sao, qwo, swo, off)
    pre = synth.bf16_bits_to_f32(preb).astype(np.float64)
    Gm, U = pre[:, :f], pre[:, f:]
    z = np.zeros((Mt, 1))
    zw = np.zeros((f, 1))
    _, _, _, _, dG, dU = O.swiglu_ffn_backward(z, zw, zw, np.eye(f), Gm, U, O.silu(Gm) * U, dH)
    # dG and dU are one rounding of dH times a factor of the pre-activations;
    # dH may carry the accumulation noise allowed for a product (1e-4 of its
    # RMS), which reaches dG through |U silu'(G)| and dU through |silu(G)|
    e = 1e-4 * np.sqrt(np.mean(dH * dH))
    sg = 1.0 / (1.0 + np.exp(-Gm))
    inherited = np.concatenate([np.abs(U * sg * (1.0 + Gm * (1.0 - sg))), np.abs(O.silu(Gm))], axis=1) * e
    assert_rounded(host(C), np.concatenate([dG, dU], axis=1), "bf16", "dG | dU", extra=inherited)


def test_quantize_e5m2_bit_exact():
    """Row-wise e5m2 codes and scales equal the oracle's bit for bit (an
    all-zero row, extreme values, bf16 and fp32 inputs)."""
    g = np.random.default_rng(46)
    xf = (g.standard_normal((260, 384)) * np.exp(g.uniform(-6, 6, (260, 1)))).astype(np.float32)
    xf[3] = 0.0
    xf[4, :4] = np.array([1e-30, -6e4, 3.0, -2e-20], np.float32)
    xb = synth.f32_to_bf16_bits(xf)
    for x, ref_in in ((dev(xb), synth.bf16_bits_to_f32(xb)), (torch.from_numpy(xf).cuda(), xf)):
        q = torch.empty(x.shape[0], x.shape[1], dtype=torch.uint8, device="cuda")
        s = torch.empty(x.shape[0], dtype=torch.float32, device="cuda")
        M.moe_quantize_fp8(x, q, s, fmt="e5m2")
        torch.cuda.synchronize()
        qo, so = O.quantize_rowwise(ref_in, "e5m2")
        assert np.array_equal(s.cpu().numpy(), so)
        assert np.array_equal(q.cpu().numpy(), qo)


@pytest.mark.parametrize("K", [384, 128])
@pytest.mark.parametrize("epi", ["none", "dswiglu"])
def test_grouped_gemm_e5m2_gradient_operand(epi, K):
    """The fp8 product with e5m2 codes for A (a gradient) and e4m3 for B (a
    weight quantised along its reduction dimension, stored transposed): the
    gate/up data gradient (plain) and the down data gradient with the
    dSwiGLU epilogue, ragged groups and an empty one, against the oracle's
    product of the same codes.  K = 128: two 64-deep k-steps, fewer than the
    pipeline's stages."""
    g = np.random.default_rng(47)
    G, N = 4, 256
    m = g.integers(30, 260, size=G)
    m[2] = 0
    off = np.zeros(G + 1, np.int32)
    off[1:] = np.cumsum(m)
    Mt = int(off[-1])
    ab = _bf16(g, (Mt, K), 0.05)
    wb = _bf16(g, (G, K, N), 1 / np.sqrt(K))          # W [G, K(reduction), N], quantised along K
    qa = torch.empty(Mt, K, dtype=torch.uint8, device="cuda")
    sa = torch.empty(Mt, dtype=torch.float32, device="cuda")
    M.moe_quantize_fp8(dev(ab), qa, sa, fmt="e5m2")
    qw = torch.empty(G, N, K, dtype=torch.uint8, device="cuda")
    sw = torch.empty(G, N, dtype=torch.float32, device="cuda")
    M.moe_quantize_fp8_transposed(dev(wb), qw, sw)
    qao, sao = O.quantize_rowwise(synth.bf16_bits_to_f32(ab), "e5m2")
    qwo, swo = O.quantize_rowwise_transposed(synth.bf16_bits_to_f32(wb))
    ref = O.grouped_gemm_fp8_nt(qao, sao, qwo, swo, off, "e5m2")
    print(f"[fp8] e5m2 A, {epi}: G={G} M={Mt} N={N} K={K}", flush=True)
    if epi == "none":
        C = torch.empty(Mt, N, dtype=torch.bfloat16, device="cuda")
        M.moe_grouped_gemm_fp8("none", G, Mt, N, K, dev(off), qa, sa, qw, sw, C, a_fmt="e5m2")
        torch.cuda.synchronize()
        assert_rounded(host(C), ref, "bf16", "C")
    else:
        preb = _bf16(g, (Mt, 2 * N))
        C = torch.empty(Mt, 2 * N, dtype=torch.bfloat16, device="cuda")
        M.moe_grouped_gemm_fp8("dswiglu", G, Mt, N, K, dev(off), qa, sa, qw, sw, C, dev(preb), a_fmt="e5m2")
        torch.cuda.synchronize()
        pre = synth.bf16_bits_to_f32(preb).astype(np.float64)
        Gm, U = pre[:, :N], pre[:, N:]
        sg = 1.0 / (1.0 + np.exp(-Gm))
        dG = ref * U * sg * (1.0 + Gm * (1.0 - sg))
        dU = ref * Gm * sg
        e = 1e-4 * np.sqrt(np.mean(ref * ref))
        inherited = np.concatenate([np.abs(U * sg * (1.0 + Gm * (1.0 - sg))), np.abs(O.silu(Gm))], axis=1) * e
        assert_rounded(host(C), np.concatenate([dG, dU], axis=1), "bf16", "dG | dU", extra=inherited)
