"""Gather-on-load: the routed gate/up products read the token rows through the
row map instead of a permuted copy.

  * the gathered grouped GEMM (NT plain and SwiGLU, TN) against the oracle's
    product of the gathered rows (one rounding), and bit-identical to the
    same kernel run on an explicitly permuted copy where that copy takes the
    same kernel;
  * the whole layer without x_perm against the oracle, and bit-identical to
    the layer with x_perm in every output the two paths compute in the same
    order."""
import numpy as np
import pytest
import torch

import synth
from oracle import moe_oracle as O
from tests.gpu_util import assert_rounded, dev, host

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import mixture_experts_layer_18_amd as M
    from tests import layer_runner as R


def _bf16(g, shape, scale=1.0):
    return synth.f32_to_bf16_bits((g.standard_normal(shape) * scale).astype(np.float32))


def _offsets(g, G, mean):
    m = g.integers(mean // 2, mean * 3 // 2 + 1, size=G)
    m[1] = 0                 # an empty group
    m[-1] = mean * 2 + 37    # a ragged tail of several tiles
    off = np.zeros(G + 1, np.int32)
    off[1:] = np.cumsum(m)
    return off


@pytest.mark.parametrize("layout,epi,N,K", [("NT", "none", 384, 512), ("NT", "swiglu", 512, 256),
                                            ("TN", "none", 384, 256), ("TN", "none", 256, 512)])
def test_gathered_gemm(layout, epi, N, K):
    g = np.random.default_rng(7 + N + K)
    G, T_src = 6, 700
    off = _offsets(g, G, 230)
    Mt = int(off[-1])
    rows = g.integers(0, T_src, size=Mt).astype(np.int32)    # repeats, any order
    X = _bf16(g, (T_src, K))
    Xg = synth.bf16_bits_to_f32(X)[rows].astype(np.float64)
    print(f"[gather] {layout} {epi} G={G} M={Mt} N={N} K={K}", flush=True)
    if layout == "NT":
        B = _bf16(g, (G, N, K), 1 / np.sqrt(K))
        Bf = synth.bf16_bits_to_f32(B).astype(np.float64)
        ref = np.zeros((Mt, N))
        for e in range(G):
            ref[off[e]:off[e + 1]] = Xg[off[e]:off[e + 1]] @ Bf[e].T
        F = N // 2
        C = torch.empty(Mt, F if epi == "swiglu" else N, dtype=torch.bfloat16, device="cuda")
        aux = torch.empty(Mt, N, dtype=torch.bfloat16, device="cuda") if epi == "swiglu" else None
        M.moe_grouped_gemm_gather("NT", epi, G, Mt, N, K, dev(off), dev(X), dev(B), C, dev(rows), T_src, aux)
        # the same kernel on an explicitly permuted copy
        C2 = torch.empty_like(C)
        aux2 = torch.empty_like(aux) if aux is not None else None
        M.moe_grouped_gemm("NT", epi, "bf16", G, Mt, N, K, dev(off), dev(X)[dev(rows).long()].contiguous(),
                           dev(B), C2, aux2)
        torch.cuda.synchronize()
        assert torch.equal(C.view(torch.int16), C2.view(torch.int16))
        if epi == "swiglu":
            assert torch.equal(aux.view(torch.int16), aux2.view(torch.int16))
            assert_rounded(host(aux), ref, "bf16", "aux")
            H = np.zeros((Mt, F))
            for e in range(G):
                a0, a1 = off[e], off[e + 1]
                H[a0:a1] = O.swiglu_ffn(Xg[a0:a1], Bf[e, :F], Bf[e, F:], np.zeros((1, F)))[2]
            assert_rounded(host(C), H, "bf16", "h")
        else:
            assert_rounded(host(C), ref, "bf16", "C")
    else:
        A = _bf16(g, (Mt, N))
        Af = synth.bf16_bits_to_f32(A).astype(np.float64)
        ref = np.zeros((G, N, K))
        for e in range(G):
            ref[e] = Af[off[e]:off[e + 1]].T @ Xg[off[e]:off[e + 1]]
        C = torch.full((G, N, K), float("nan"), dtype=torch.bfloat16, device="cuda")
        M.moe_grouped_gemm_gather("TN", "none", G, Mt, N, K, dev(off), dev(A), dev(X), C, dev(rows), T_src)
        torch.cuda.synchronize()
        got = host(C)
        assert np.all(got[1] == 0)                          # the empty group
        assert_rounded(got, ref, "bf16", "dW")


GATHER_BF16 = synth.CONFIG_BY_NAME["moe7b_bf16"].replace(name="gather_bf16", T=1000, d=256, E=16, k=4, f=256,
                                                          n_shared=2, f_shared=128)


def test_layer_without_permuted_copy():
    cfg = GATHER_BF16
    inp = synth.make_inputs(cfg)
    print("[gather] layer fwd+bwd against the oracle", flush=True)
    R.compare_full(cfg, inp, backward=True, gather=True)
    print("[gather] layer with and without x_perm", flush=True)
    a = R.run_gpu(cfg, inp, backward=True, gather=True)
    b = R.run_gpu(cfg, inp, backward=True, gather=False)
    # the gathered weight gradient runs on the persistent kernel; with a
    # permuted copy this small problem goes to row slices (another order)
    for n in a:
        if n == "d_w_gateup":
            continue
        assert np.array_equal(a[n], b[n], equal_nan=True), n


def test_layer_without_permuted_copy_unsupported_shape():
    cfg = GATHER_BF16.replace(f=192)          # d_ff not a multiple of 128
    desc = M.desc_from_config(cfg)
    saved = M.alloc_saved(desc, gather=True)
    x = torch.zeros(cfg.T, cfg.d, dtype=torch.bfloat16, device="cuda")
    w = R.upload_layer(cfg, synth.make_inputs(cfg))
    with pytest.raises(M.MoeError):
        M.moe_forward(desc, w, x, torch.empty_like(x), saved, M.alloc_workspace(desc, "forward"))
