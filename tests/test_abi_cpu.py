"""The C ABI library loads, exports every function include/moe.h declares,
answers its size queries and rejects invalid arguments on the host, before
any GPU work (these calls never reach the HIP runtime)."""
import ctypes
import re

import pytest

from mixture_experts_layer_18_amd import _lib as L
from mixture_experts_layer_18_amd.api import make_desc


@pytest.fixture(scope="module")
def lib():
    return L.load()


def test_exports_every_declared_function(lib):
    names = L.header_functions()
    assert len(names) >= 11
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(L.SIGNATURES)
    assert lib.moe_abi_version() == 4


def test_status_strings(lib):
    for s in range(6):
        assert lib.moe_status_str(s).startswith(b"MOE_")
    assert lib.moe_status_str(99) == b"unknown status"


def test_struct_layout_matches_header():
    assert ctypes.sizeof(L.MoeDesc) == 7 * 8 + 4 * 4
    assert ctypes.sizeof(L.MoeWeights) == 6 * 8
    assert ctypes.sizeof(L.MoeSaved) == 14 * 8
    assert ctypes.sizeof(L.MoeGrads) == 5 * 8
    assert ctypes.sizeof(L.MoeFp8Weights) == 16 * 8
    text = open(L.HEADER).read()
    body = re.search(r"typedef struct moe_fp8_weights \{(.*?)\} moe_fp8_weights_t;", text, re.S).group(1)
    assert tuple(re.findall(r"\*(\w+);", body)) == L.FP8_WEIGHT_FIELDS


def test_queries(lib):
    d = make_desc(16384, 2048, 64, 6, 1408, 2, 1408, "sigmoid", True, "bf16")
    assert lib.moe_route_hist_elems(ctypes.byref(d)) == 64 * (16384 // 32)
    assert lib.moe_workspace_bytes(ctypes.byref(d), L.MOE_WS_PERMUTE) >= 64 * 512 * 4
    fw = lib.moe_workspace_bytes(ctypes.byref(d), L.MOE_WS_FORWARD)
    bw = lib.moe_workspace_bytes(ctypes.byref(d), L.MOE_WS_BACKWARD)
    A = 16384 * 6
    # backward holds dY~ (reused for dX~) and dG|dU in bf16 plus fp32 dlogits
    assert bw >= A * 2048 * 2 + A * 2 * 1408 * 2 + 16384 * 64 * 4
    assert 0 < fw < bw
    # ragged token count: histogram blocks round up
    d2 = make_desc(33, 128, 8, 2, 256, 0, 0, "softmax", False, "f32")
    assert lib.moe_route_hist_elems(ctypes.byref(d2)) == 8 * 2
    assert lib.moe_grouped_gemm_workspace_bytes(L.MOE_GEMM_NT, L.MOE_BF16, 8, 100, 128, 128) == 0


def test_weight_gradient_slice_counts(lib):
    """Row-slice counts of weight gradients with few output tiles, read back
    through the workspace size (slices x G x N x K fp32 partials).  One group
    on the persistent kernel: sliced until it has 128 output tiles, each slice
    at least 32 k-steps; so the 7B-style layer's shared gate/up weight gradient
    (176 tiles) takes none and its shared down weight gradient (88 tiles) two,
    and the large layer's need none.  Shapes that cannot reach 128 tiles go to
    the two-workgroup kernel, whose slices keep at least 512 rows."""
    ws = lambda G, M, N, K: lib.moe_grouped_gemm_workspace_bytes(L.MOE_GEMM_TN, L.MOE_BF16, G, M, N, K)  # noqa: E731
    assert ws(1, 16384, 5632, 2048) == 0
    assert ws(1, 16384, 2048, 2816) == 2 * 2048 * 2816 * 4
    assert ws(1, 65536, 4096, 4096) == 0
    # 20 tiles: 8 slices of 33 k-steps (the last one 26), 160 tiles
    assert ws(1, 8195, 1024, 1280) == 8 * 1024 * 1280 * 4
    assert ws(1, 4096, 256, 384) == 8 * 256 * 384 * 4
    assert ws(1, 4000, 256, 384) == 7 * 256 * 384 * 4
    assert ws(1, 600, 256, 384) == 0


def test_persistent_kernel_offset_limit(lib):
    """The persistent kernel's operand DMA uses 32-bit byte offsets from a
    group's first row.  A one-group weight gradient whose operand spans more
    than 2^32 bytes goes to the two-workgroup kernel (64-bit addresses, row
    slices with fp32 partials: a nonzero workspace); at exactly 2^32 bytes the
    last 16-byte load still starts below 2^32 and the persistent kernel (no
    workspace) takes it."""
    ws = lambda G, M, N, K: lib.moe_grouped_gemm_workspace_bytes(L.MOE_GEMM_TN, L.MOE_BF16, G, M, N, K)  # noqa: E731
    # 131072 tokens x (2 x 4096 shared experts): 131072 * 16384 * 2 = 2^32 bytes
    assert ws(1, 131072, 16384, 4096) == 0
    assert ws(1, 131072, 16448, 4096) > 0
    # the other operand (K columns) is bounded the same way
    assert ws(1, 131072, 4096, 16384) == 0
    assert ws(1, 131072, 4096, 16448) > 0


def test_no_workspace_forward_rejects_large_layers(lib):
    """moe_forward_no_workspace keeps its scratch in a fixed device array of
    MOE_STATIC_SCRATCH_BYTES (8 MiB): a layer whose forward scratch (two int32
    tables of E x ceil(T/32) entries) exceeds it is rejected on the host."""
    # E * ceil(T/32) = 2^20 fits exactly; one more block of 32 tokens does not
    d0 = make_desc(131072, 2048, 256, 8, 512, 0, 0, "sigmoid", True, "bf16")
    assert lib.moe_workspace_bytes(ctypes.byref(d0), L.MOE_WS_FORWARD) == 8 << 20
    d = make_desc(131072 + 32, 2048, 256, 8, 512, 0, 0, "sigmoid", True, "bf16")
    assert lib.moe_workspace_bytes(ctypes.byref(d), L.MOE_WS_FORWARD) > 8 << 20
    assert lib.moe_forward_no_workspace(ctypes.byref(d), None, None, None, None, None) == L.MOE_ERR_WORKSPACE
    bad = make_desc(64, 100, 8, 2, 256, 0, 0, "softmax", False, "f32")
    assert lib.moe_forward_no_workspace(ctypes.byref(bad), None, None, None, None, None) == L.MOE_ERR_INVALID


BAD = [
    dict(E=0), dict(E=257), dict(k=0), dict(k=17), dict(k=9, E=8), dict(d=100), dict(f=96),
    dict(T=-1), dict(score=2), dict(renorm=2), dict(dtype=3), dict(reserved=1), dict(n_shared=1, f_shared=0),
    dict(n_shared=1, f_shared=100),
]


@pytest.mark.parametrize("bad", BAD)
def test_invalid_descriptors_rejected(lib, bad):
    p = dict(T=64, d=128, E=8, k=2, f=256, n_shared=0, f_shared=0)
    p.update({k: v for k, v in bad.items() if k in p})
    d = make_desc(p["T"], p["d"], p["E"], p["k"], p["f"], p["n_shared"], p["f_shared"], "softmax", False, "f32")
    for field in ("score", "renorm", "dtype", "reserved"):
        if field in bad:
            setattr(d, field, bad[field])
    assert lib.moe_route_hist_elems(ctypes.byref(d)) == 0
    assert lib.moe_workspace_bytes(ctypes.byref(d), L.MOE_WS_FORWARD) == 0
    fake = ctypes.c_void_p(0x1000)
    st = lib.moe_route(ctypes.byref(d), fake, None, fake, fake, fake, None)
    assert st == L.MOE_ERR_INVALID


def test_null_and_misaligned_pointers_rejected(lib):
    d = make_desc(64, 128, 8, 2, 256, 0, 0, "softmax", False, "f32")
    a = ctypes.c_void_p(0x10000)
    mis = ctypes.c_void_p(0x10004)
    assert lib.moe_route(ctypes.byref(d), None, None, a, a, a, None) == L.MOE_ERR_INVALID
    assert lib.moe_route(ctypes.byref(d), mis, None, a, a, a, None) == L.MOE_ERR_ALIGN
    assert lib.moe_combine(ctypes.byref(d), a, a, a, None, None, None) == L.MOE_ERR_INVALID
    # workspace too small
    assert lib.moe_permute(ctypes.byref(d), a, a, a, a, a, a, a, a, a, a, 16, None) == L.MOE_ERR_WORKSPACE
    w = L.MoeWeights(a, None, a, a, None, None)
    s = L.MoeSaved(*([a] * 14))
    assert lib.moe_forward(ctypes.byref(d), ctypes.byref(w), a, a, ctypes.byref(s), a, 16, None) == \
        L.MOE_ERR_WORKSPACE
    assert lib.moe_forward(ctypes.byref(d), None, a, a, ctypes.byref(s), a, 1 << 30, None) == L.MOE_ERR_INVALID
    g = L.MoeGrads(a, a, a, None, None)
    s.preact = None
    assert lib.moe_backward(ctypes.byref(d), ctypes.byref(w), a, ctypes.byref(s), a, a, ctypes.byref(g), None,
                            None, a, 1 << 30, None) == L.MOE_ERR_INVALID
    # shared experts declared but no shared weights
    d2 = make_desc(64, 128, 8, 2, 256, 1, 128, "sigmoid", True, "bf16")
    s2 = L.MoeSaved(*([a] * 14))
    assert lib.moe_forward(ctypes.byref(d2), ctypes.byref(w), a, a, ctypes.byref(s2), a, 1 << 30, None) == \
        L.MOE_ERR_INVALID


def test_grouped_gemm_argument_checks(lib):
    a = ctypes.c_void_p(0x10000)
    ok = dict(layout=L.MOE_GEMM_NT, epi=L.MOE_EPI_NONE, dtype=L.MOE_BF16, G=4, M=100, N=128, K=128)

    def call(**kw):
        p = dict(ok)
        p.update(kw)
        return lib.moe_grouped_gemm(p["layout"], p["epi"], p["dtype"], p["G"], p["M"], p["N"], p["K"],
                                    a, a, a, a, a, None, 0, None)
    assert call(layout=5) == L.MOE_ERR_INVALID
    assert call(epi=L.MOE_EPI_DSWIGLU) == L.MOE_ERR_INVALID          # dswiglu needs NN
    assert call(layout=L.MOE_GEMM_TN, epi=L.MOE_EPI_SWIGLU) == L.MOE_ERR_INVALID
    assert call(G=0) == L.MOE_ERR_INVALID
    assert call(G=300) == L.MOE_ERR_INVALID
    assert call(N=100) == L.MOE_ERR_INVALID
    assert call(K=96) == L.MOE_ERR_INVALID
    assert call(epi=L.MOE_EPI_SWIGLU, N=192) == L.MOE_ERR_INVALID   # gate/up halves of 64
    assert call(dtype=7) == L.MOE_ERR_INVALID
    # no offset table: allowed for one group only (validation fails before any launch)
    assert lib.moe_grouped_gemm(L.MOE_GEMM_NT, L.MOE_EPI_NONE, L.MOE_BF16, 4, 100, 128, 128, None, a, a, a, a,
                                None, 0, None) == L.MOE_ERR_INVALID
    assert lib.moe_grouped_gemm(L.MOE_GEMM_NT, L.MOE_EPI_NONE, L.MOE_BF16, 1, 100, 128, 127, None, a, a, a, a,
                                None, 0, None) == L.MOE_ERR_INVALID


def test_stage_enum_matches_binding():
    text = open(L.HEADER).read()
    body = re.search(r"enum \{\s*(MOE_STAGE_ROUTER = 0,.*?MOE_NUM_STAGES)\s*\}", text, re.S).group(1)
    names = re.findall(r"MOE_STAGE_(\w+)", body)
    assert [n.lower() for n in names] == L.STAGES


def test_stage_timing_without_records(lib):
    # nothing recorded: no HIP call is made, every slot reads zero
    assert lib.moe_stage_timing(1) == L.MOE_OK
    ms = (ctypes.c_double * L.MOE_NUM_STAGES)(*([7.0] * L.MOE_NUM_STAGES))
    n = (ctypes.c_int64 * L.MOE_NUM_STAGES)(*([7] * L.MOE_NUM_STAGES))
    assert lib.moe_stage_times(ms, n) == L.MOE_OK
    assert list(ms) == [0.0] * L.MOE_NUM_STAGES and list(n) == [0] * L.MOE_NUM_STAGES
    assert lib.moe_stage_times(None, n) == L.MOE_ERR_INVALID
    assert lib.moe_stage_timing(0) == L.MOE_OK
    # a stage mask: still nothing recorded without launches
    assert lib.moe_stage_timing_mask(1 << L.STAGES.index("gate_up")) == L.MOE_OK
    assert lib.moe_stage_times(ms, n) == L.MOE_OK
    assert all(n[i] == 0 for i in range(L.MOE_NUM_STAGES))
    assert lib.moe_stage_timing_mask(0) == L.MOE_OK


def test_router_terms_and_bias_update_argument_checks(lib):
    """Host-side rejection of bad router-term arguments (no launch happens)."""
    d = make_desc(64, 128, 8, 2, 256, 0, 0, "sigmoid", True, "bf16")
    a = ctypes.c_void_p(1 << 20)
    w = L.MoeWeights(a, a, a, a, None, None)
    s = L.MoeSaved(*([a] * 11 + [None, None]))
    g = L.MoeGrads(a, a, a, None, None)
    big = 1 << 34

    def bwd(terms, losses=None):
        return lib.moe_backward(ctypes.byref(d), ctypes.byref(w), a, ctypes.byref(s), a, a, ctypes.byref(g),
                                None if terms is None else ctypes.byref(terms), losses, a, big, None)

    # losses without terms, a negative or NaN coefficient, a sequence length not dividing T
    assert bwd(None, a) == L.MOE_ERR_INVALID
    assert bwd(L.MoeRouterTerms(-1e-3, 0.0, 0.0, 0)) == L.MOE_ERR_INVALID
    assert bwd(L.MoeRouterTerms(float("nan"), 0.0, 0.0, 0)) == L.MOE_ERR_INVALID
    assert bwd(L.MoeRouterTerms(0.0, 1e-3, 0.0, 48)) == L.MOE_ERR_INVALID
    assert bwd(L.MoeRouterTerms(0.0, 1e-3, 0.0, -1)) == L.MOE_ERR_INVALID
    assert bwd(L.MoeRouterTerms(1e-3, 0.0, 0.0, 0), ctypes.c_void_p((1 << 20) + 4)) == L.MOE_ERR_ALIGN
    # bias update: NaN rate, null pointers, misaligned counts
    assert lib.moe_bias_update(ctypes.byref(d), a, float("nan"), a, None) == L.MOE_ERR_INVALID
    assert lib.moe_bias_update(ctypes.byref(d), None, 0.01, a, None) == L.MOE_ERR_INVALID
    assert lib.moe_bias_update(ctypes.byref(d), ctypes.c_void_p((1 << 20) + 4), 0.01, a, None) == L.MOE_ERR_ALIGN
    # zero tokens: nothing to do
    d0 = make_desc(0, 128, 8, 2, 256, 0, 0, "sigmoid", True, "bf16")
    assert lib.moe_bias_update(ctypes.byref(d0), None, 0.01, None, None) == L.MOE_OK


def test_fp8_argument_checks(lib):
    a = ctypes.c_void_p(1 << 20)
    # quantize: columns not a multiple of 64, bad dtype, misaligned, zero rows
    E4, E5 = L.MOE_E4M3, L.MOE_E5M2
    assert lib.moe_quantize_fp8(10, 100, L.MOE_BF16, E4, a, a, a, None) == L.MOE_ERR_INVALID
    assert lib.moe_quantize_fp8(10, 128, 7, E4, a, a, a, None) == L.MOE_ERR_INVALID
    assert lib.moe_quantize_fp8(10, 128, L.MOE_BF16, 2, a, a, a, None) == L.MOE_ERR_INVALID   # no such format
    assert lib.moe_quantize_fp8(10, 128, L.MOE_BF16, E5, ctypes.c_void_p((1 << 20) + 2), a, a, None) == \
        L.MOE_ERR_ALIGN
    assert lib.moe_quantize_fp8(0, 128, L.MOE_BF16, E5, None, None, None, None) == L.MOE_OK
    # tensor-wise: the same checks, and the scratch size (row maxima + scale)
    tw = lib.moe_quantize_fp8_tensorwise
    assert lib.moe_quantize_fp8_tensorwise_workspace_bytes(10) == 44
    assert tw(10, 100, L.MOE_BF16, a, a, a, a, 64, None) == L.MOE_ERR_INVALID
    assert tw(10, 128, L.MOE_BF16, a, a, a, None, 64, None) == L.MOE_ERR_INVALID
    assert tw(10, 128, L.MOE_BF16, a, a, a, ctypes.c_void_p((1 << 20) + 4), 64, None) == L.MOE_ERR_ALIGN
    assert tw(10, 128, L.MOE_BF16, a, a, a, a, 40, None) == L.MOE_ERR_WORKSPACE
    assert tw(0, 128, L.MOE_F32, None, None, None, None, 0, None) == L.MOE_OK
    # transposed (along the first axis): rows and columns multiples of 64, dtype, alignment, empty
    tq = lib.moe_quantize_fp8_transposed
    assert tq(2, 100, 128, L.MOE_BF16, a, a, a, None) == L.MOE_ERR_INVALID
    assert tq(2, 128, 96, L.MOE_BF16, a, a, a, None) == L.MOE_ERR_INVALID
    assert tq(-1, 128, 128, L.MOE_BF16, a, a, a, None) == L.MOE_ERR_INVALID
    assert tq(2, 128, 128, 5, a, a, a, None) == L.MOE_ERR_INVALID
    assert tq(2, 128, 128, L.MOE_BF16, a, None, a, None) == L.MOE_ERR_INVALID
    assert tq(2, 128, 128, L.MOE_F32, a, a, ctypes.c_void_p((1 << 20) + 8), None) == L.MOE_ERR_ALIGN
    assert tq(0, 128, 128, L.MOE_BF16, None, None, None, None) == L.MOE_OK
    assert tq(3, 0, 128, L.MOE_BF16, None, None, None, None) == L.MOE_OK
    # gemm: layout limits
    args = (a, a, a, a, a, a, None, None)
    gf = lib.moe_grouped_gemm_fp8
    assert gf(L.MOE_EPI_DSWIGLU, E4, 4, 100, 256, 128, *args) == L.MOE_ERR_INVALID  # no aux
    assert gf(3, E4, 4, 100, 256, 128, *args) == L.MOE_ERR_INVALID
    assert gf(L.MOE_EPI_NONE, E4, 0, 100, 256, 128, *args) == L.MOE_ERR_INVALID
    assert gf(L.MOE_EPI_NONE, E4, 4, 100, 256, 96, *args) == L.MOE_ERR_INVALID
    assert gf(L.MOE_EPI_SWIGLU, E4, 4, 100, 384, 128, *args) == L.MOE_ERR_INVALID
    assert gf(L.MOE_EPI_NONE, 2, 4, 100, 256, 128, *args) == L.MOE_ERR_INVALID       # no such format
    assert gf(L.MOE_EPI_SWIGLU, E5, 4, 100, 512, 128, *args) == L.MOE_ERR_UNSUPPORTED  # e5m2: data gradients
    assert gf(L.MOE_EPI_NONE, E4, 4, 100, 256, 128, a, a, a, a, a, ctypes.c_void_p((1 << 20) + 4), None,
              None) == L.MOE_ERR_ALIGN
    assert gf(L.MOE_EPI_NONE, E5, 4, 0, 256, 128, a, None, None, None, None, None, None, None) == L.MOE_OK


def test_gather_argument_checks(lib):
    """The gathered-row GEMM and the layer without a permuted token copy:
    unsupported layouts and shapes and missing maps are rejected on the host."""
    a = ctypes.c_void_p(0x10000)
    mis = ctypes.c_void_p(0x10004)
    NT, NN, TN = L.MOE_GEMM_NT, L.MOE_GEMM_NN, L.MOE_GEMM_TN
    NONE, SWIGLU = L.MOE_EPI_NONE, L.MOE_EPI_SWIGLU
    gg = lib.moe_grouped_gemm_gather
    assert gg(NN, NONE, 4, 64, 256, 256, a, a, a, a, None, a, 100, None) == L.MOE_ERR_UNSUPPORTED
    assert gg(TN, SWIGLU, 4, 64, 256, 256, a, a, a, a, a, a, 100, None) == L.MOE_ERR_INVALID
    assert gg(TN, NONE, 4, 64, 256, 192, a, a, a, a, None, a, 100, None) == L.MOE_ERR_UNSUPPORTED  # K % 256
    assert gg(NT, SWIGLU, 4, 64, 384, 256, a, a, a, a, a, a, 100, None) == L.MOE_ERR_UNSUPPORTED  # F % 128
    assert gg(NT, NONE, 4, 64, 256, 4096, a, a, a, a, None, a, 1 << 20, None) == L.MOE_ERR_UNSUPPORTED
    assert gg(NT, NONE, 4, 64, 256, 256, a, a, a, a, None, None, 100, None) == L.MOE_ERR_INVALID   # no map
    assert gg(NT, NONE, 4, 64, 256, 256, a, a, a, a, None, mis, 100, None) == L.MOE_ERR_ALIGN
    assert gg(NT, NONE, 4, 64, 256, 256, a, a, a, a, None, a, -1, None) == L.MOE_ERR_INVALID
    # layer without x_perm
    w = L.MoeWeights(a, None, a, a, None, None)
    s = L.MoeSaved(*([a] * 14))
    s.x_perm = None
    f32 = make_desc(64, 256, 8, 2, 256, 0, 0, "softmax", False, "f32")
    assert lib.moe_forward(ctypes.byref(f32), ctypes.byref(w), a, a, ctypes.byref(s), a, 1 << 30, None) == \
        L.MOE_ERR_UNSUPPORTED
    odd = make_desc(64, 192, 8, 2, 256, 0, 0, "softmax", False, "bf16")   # d % 256: no gathered weight gradient
    assert lib.moe_forward(ctypes.byref(odd), ctypes.byref(w), a, a, ctypes.byref(s), a, 1 << 30, None) == \
        L.MOE_ERR_UNSUPPORTED
    g = L.MoeGrads(a, a, a, None, None)
    assert lib.moe_backward(ctypes.byref(odd), ctypes.byref(w), a, ctypes.byref(s), a, a, ctypes.byref(g), None,
                            None, a, 1 << 30, None) == L.MOE_ERR_UNSUPPORTED
    s.tok = None
    ok = make_desc(64, 256, 8, 2, 256, 0, 0, "softmax", False, "bf16")
    assert lib.moe_forward(ctypes.byref(ok), ctypes.byref(w), a, a, ctypes.byref(s), a, 1 << 30, None) == \
        L.MOE_ERR_INVALID


def test_saved_layout_in_one_allocation(lib):
    """moe_saved_bytes / moe_saved_carve: every field the flags ask for is
    256-byte aligned, inside the allocation and disjoint from the others;
    the others are NULL.  Host arithmetic only."""
    d = make_desc(1000, 256, 16, 4, 192, 2, 128, "sigmoid", True, "bf16")
    T, D, E, k, f, F = 1000, 256, 16, 4, 192, 256
    A = T * k
    es = 2
    sizes = dict(logits=T * E * 4, idx=T * k * 4, gate=T * k * 4, counts=E * 4, offsets=(E + 1) * 4, pos=A * 4,
                 src=A * 4, tok=A * 4, x_perm=A * D * es, preact=A * 2 * f * es, h=A * f * es, y_perm=A * D * es,
                 s_preact=T * 2 * F * es, s_h=T * F * es)
    base = 1 << 30
    for flags in (0, L.MOE_SAVED_TRAINING, L.MOE_SAVED_PERMUTED_COPY,
                  L.MOE_SAVED_TRAINING | L.MOE_SAVED_PERMUTED_COPY):
        n = lib.moe_saved_bytes(ctypes.byref(d), flags)
        s = L.MoeSaved()
        assert lib.moe_saved_carve(ctypes.byref(d), flags, ctypes.c_void_p(base), n, ctypes.byref(s)) == L.MOE_OK
        spans = []
        for name, size in sizes.items():
            p = getattr(s, name)
            want = not ((name in ("preact", "s_preact") and not flags & L.MOE_SAVED_TRAINING) or
                        (name == "x_perm" and not flags & L.MOE_SAVED_PERMUTED_COPY))
            if not want:
                assert p is None, name
                continue
            assert p is not None and p % 256 == 0 and base <= p and p + size <= base + n, name
            spans.append((p, p + size))
        spans.sort()
        assert all(a[1] <= b[0] for a, b in zip(spans, spans[1:]))
        assert lib.moe_saved_carve(ctypes.byref(d), flags, ctypes.c_void_p(base), n - 1,
                                   ctypes.byref(s)) == L.MOE_ERR_WORKSPACE
    assert lib.moe_saved_bytes(ctypes.byref(d), 4) == 0
    s = L.MoeSaved()
    assert lib.moe_saved_carve(ctypes.byref(d), 0, ctypes.c_void_p(base + 16), 1 << 30, ctypes.byref(s)) == \
        L.MOE_ERR_ALIGN
    assert lib.moe_saved_carve(ctypes.byref(d), 8, ctypes.c_void_p(base), 1 << 30, ctypes.byref(s)) == \
        L.MOE_ERR_INVALID


def test_fp8_layer_workspace_sizes(lib):
    """The fp8 layer calls add their quantised operands to the bf16 calls'
    workspaces: the forward the token codes [T, d] with one scale per token and
    the larger of the routed [A, f] and shared [T, F] hidden codes with their
    scales; the backward the largest data-gradient operand (here dG | dU,
    [A, 2f]) with one scale per row, and dy's codes [T, d] with one scale per
    token (the shared down data gradient's operand, written by the combine
    backward)."""
    T, dm, E, k, f, F = 16384, 2048, 64, 6, 1408, 2 * 1408
    d = make_desc(T, dm, E, k, f, 2, 1408, "sigmoid", True, "bf16")
    A = T * k
    fw = lib.moe_workspace_bytes(ctypes.byref(d), L.MOE_WS_FORWARD)
    bw = lib.moe_workspace_bytes(ctypes.byref(d), L.MOE_WS_BACKWARD)
    fw8 = lib.moe_workspace_bytes(ctypes.byref(d), L.MOE_WS_FORWARD_FP8)
    bw8 = lib.moe_workspace_bytes(ctypes.byref(d), L.MOE_WS_BACKWARD_FP8)
    assert fw8 - fw >= T * dm + T * 4 + A * f + A * 4
    assert fw8 - fw < T * dm + T * 4 + A * f + A * 4 + 4 * 256
    assert bw8 - bw >= A * 2 * f + A * 4 + T * dm + T * 4
    assert bw8 - bw < A * 2 * f + A * 4 + T * dm + T * 4 + 4 * 256
    assert A * f > T * F


def test_fp8_layer_argument_checks(lib):
    """Host-side rejection for the fp8 layer calls: layers they do not take
    (fp32, a hidden width not a multiple of 128), a missing or misaligned fp8
    weight, a short workspace; and for the weight quantiser and the gathered
    fp8 GEMM.  No check reaches the GPU."""
    a = ctypes.c_void_p(0x10000)
    mis = ctypes.c_void_p(0x10004)
    d = make_desc(64, 256, 8, 2, 256, 1, 128, "sigmoid", True, "bf16")
    w = L.MoeWeights(a, a, a, a, a, a)
    s = L.MoeSaved(*([a] * 14))
    q = L.MoeFp8Weights(*([a] * 16))
    fwd = lambda dd, qq, nb: lib.moe_forward_fp8(ctypes.byref(dd), ctypes.byref(w), qq, a, a,  # noqa: E731
                                                 ctypes.byref(s), a, nb, None)
    assert fwd(d, ctypes.byref(q), 16) == L.MOE_ERR_WORKSPACE
    assert fwd(d, None, 1 << 30) == L.MOE_ERR_INVALID
    f32 = make_desc(64, 256, 8, 2, 256, 1, 128, "sigmoid", True, "f32")
    assert fwd(f32, ctypes.byref(q), 1 << 30) == L.MOE_ERR_UNSUPPORTED
    odd = make_desc(64, 256, 8, 2, 192, 0, 0, "sigmoid", True, "bf16")
    assert fwd(odd, ctypes.byref(q), 1 << 30) == L.MOE_ERR_UNSUPPORTED
    odd_shared = make_desc(64, 256, 8, 2, 256, 1, 64, "sigmoid", True, "bf16")
    assert fwd(odd_shared, ctypes.byref(q), 1 << 30) == L.MOE_ERR_UNSUPPORTED
    q2 = L.MoeFp8Weights(*([a] * 16))
    q2.down_s = None
    assert fwd(d, ctypes.byref(q2), 1 << 30) == L.MOE_ERR_INVALID
    q2.down_s = mis
    assert fwd(d, ctypes.byref(q2), 1 << 30) == L.MOE_ERR_ALIGN
    # the backward reads the data-gradient copies only
    g = L.MoeGrads(a, a, a, a, a)
    bwd = lambda qq, nb, fmt=L.MOE_E4M3, wg=0: lib.moe_backward_fp8(  # noqa: E731
        ctypes.byref(d), ctypes.byref(w), qq, fmt, wg, a, ctypes.byref(s), a, a, ctypes.byref(g), None, None, a, nb,
        None)
    assert bwd(ctypes.byref(q), 16) == L.MOE_ERR_WORKSPACE
    assert bwd(ctypes.byref(q), 16, L.MOE_E5M2) == L.MOE_ERR_WORKSPACE
    assert bwd(ctypes.byref(q), 1 << 30, 3) == L.MOE_ERR_INVALID
    assert bwd(ctypes.byref(q), 1 << 30, L.MOE_E4M3, 2) == L.MOE_ERR_INVALID
    need = lib.moe_workspace_bytes(ctypes.byref(d), L.MOE_WS_BACKWARD_FP8)
    assert bwd(ctypes.byref(q), need, L.MOE_E4M3, 1) == L.MOE_ERR_WORKSPACE    # fp8 weight gradients need more
    assert bwd(None, 1 << 30) == L.MOE_ERR_INVALID
    q3 = L.MoeFp8Weights(*([a] * 16))
    q3.s_down_tq = None
    assert bwd(ctypes.byref(q3), 1 << 30) == L.MOE_ERR_INVALID
    q3.s_down_tq = a
    q3.gateup_q = None                       # forward copy: not read by the backward
    assert bwd(ctypes.byref(q3), 16) == L.MOE_ERR_WORKSPACE
    # the weight quantiser
    assert lib.moe_fp8_weights_quantize(ctypes.byref(d), ctypes.byref(w), ctypes.byref(q), 0, None) == \
        L.MOE_ERR_INVALID
    assert lib.moe_fp8_weights_quantize(ctypes.byref(d), ctypes.byref(w), ctypes.byref(q), 4, None) == \
        L.MOE_ERR_INVALID
    assert lib.moe_fp8_weights_quantize(ctypes.byref(d), ctypes.byref(w), ctypes.byref(q3), 1, None) == \
        L.MOE_ERR_INVALID
    assert lib.moe_fp8_weights_quantize(ctypes.byref(f32), ctypes.byref(w), ctypes.byref(q), 3, None) == \
        L.MOE_ERR_UNSUPPORTED
    # the gathered fp8 GEMM
    gg = lambda epi, M, K, src, rows: lib.moe_grouped_gemm_fp8_gather(  # noqa: E731
        epi, 4, M, 256, K, a, a, a, a, a, a, None, rows, src, None)
    assert gg(L.MOE_EPI_DSWIGLU, 100, 256, 64, a) == L.MOE_ERR_INVALID
    assert gg(L.MOE_EPI_NONE, 100, 256, 64, None) == L.MOE_ERR_INVALID
    assert gg(L.MOE_EPI_NONE, 100, 65536, (1 << 16) + 1, a) == L.MOE_ERR_UNSUPPORTED
    assert gg(L.MOE_EPI_NONE, 100, 256, -1, a) == L.MOE_ERR_INVALID
    assert gg(L.MOE_EPI_NONE, 0, 256, 0, None) == L.MOE_OK


def test_mfma_ceiling_argument_checks(lib):
    """The matrix-core rate aid rejects unknown kinds, bad counts and null or
    misaligned outputs on the host; the HBM copy aid, sizes that are not whole
    16-byte vectors and null or misaligned pointers."""
    a = ctypes.c_void_p(0x10000)
    f = ctypes.c_double(0.0)
    # the HBM counterpart: sizes in 16-byte vectors, aligned pointers
    assert lib.moe_hbm_ceiling(a, a, 15, None) == L.MOE_ERR_INVALID
    assert lib.moe_hbm_ceiling(a, a, -16, None) == L.MOE_ERR_INVALID
    assert lib.moe_hbm_ceiling(None, a, 16, None) == L.MOE_ERR_INVALID
    assert lib.moe_hbm_ceiling(ctypes.c_void_p(a.value + 8), a, 16, None) == L.MOE_ERR_ALIGN
    assert lib.moe_hbm_ceiling(None, None, 0, None) == L.MOE_OK
    assert lib.moe_mfma_ceiling(4, 10, a, ctypes.byref(f), None) == L.MOE_ERR_INVALID
    assert lib.moe_mfma_ceiling(-1, 10, a, ctypes.byref(f), None) == L.MOE_ERR_INVALID
    assert lib.moe_mfma_ceiling(0, 0, a, ctypes.byref(f), None) == L.MOE_ERR_INVALID
    assert lib.moe_mfma_ceiling(0, 10, None, ctypes.byref(f), None) == L.MOE_ERR_INVALID
    assert lib.moe_mfma_ceiling(0, 10, ctypes.c_void_p(0x10004), ctypes.byref(f), None) == L.MOE_ERR_ALIGN
    assert len(L.MFMA_KINDS) == 4


def test_fp8_weight_gradient_calls(lib):
    """The column-wise quantiser's size query (an upper bound: every group's
    rows rounded up to 64) and the host checks of both weight-gradient calls;
    the fp8 weight-gradient workspace adds both operands' codes and scales."""
    assert lib.moe_quantize_fp8_colwise_bytes(64, 98304, 2048) == 2048 * (98304 + 63 * 64)
    assert lib.moe_quantize_fp8_colwise_bytes(0, 10, 64) == 0
    a = ctypes.c_void_p(0x10000)
    mis = ctypes.c_void_p(0x10004)
    qc = lib.moe_quantize_fp8_colwise
    assert qc(4, 100, 96, L.MOE_BF16, a, None, 0, a, a, a, a, None) == L.MOE_ERR_INVALID      # C % 64
    assert qc(4, 100, 128, L.MOE_BF16, None, None, 0, a, a, a, a, None) == L.MOE_ERR_INVALID  # offsets, G > 1
    assert qc(1, 100, 128, 9, None, None, 0, a, a, a, a, None) == L.MOE_ERR_INVALID
    assert qc(1, 100, 128, L.MOE_BF16, None, None, 0, a, None, a, a, None) == L.MOE_ERR_INVALID
    assert qc(1, 100, 128, L.MOE_BF16, None, mis, 10, a, a, a, a, None) == L.MOE_ERR_ALIGN
    wg = lib.moe_grouped_gemm_fp8_wgrad
    assert wg(0, 128, 128, a, a, a, a, a, a, None) == L.MOE_ERR_INVALID
    assert wg(4, 100, 128, a, a, a, a, a, a, None) == L.MOE_ERR_INVALID
    assert wg(4, 128, 128, a, a, a, a, None, a, None) == L.MOE_ERR_INVALID
    assert wg(4, 128, 128, a, mis, a, a, a, a, None) == L.MOE_ERR_ALIGN
    T, dm, E, k, f = 16384, 2048, 64, 6, 1408
    dd = make_desc(T, dm, E, k, f, 2, 1408, "sigmoid", True, "bf16")
    b8 = lib.moe_workspace_bytes(ctypes.byref(dd), L.MOE_WS_BACKWARD_FP8)
    bw8 = lib.moe_workspace_bytes(ctypes.byref(dd), L.MOE_WS_BACKWARD_FP8_WGRAD)
    A = T * k
    assert bw8 - b8 >= (2 * f + dm) * (A + 63 * E) + E * (2 * f + dm) * 4
