"""Python binding of the C ABI (include/moe.h), same call names.

Argument marshalling only: torch tensors are passed as device pointers and
the current torch stream as the HIP stream; every step of the layer runs in
the HIP library.  Buffer allocation helpers use torch for device memory.
"""
from __future__ import annotations

import ctypes

import numpy as np
from typing import Optional

import torch

from . import _lib as L

DTYPES = {"f32": L.MOE_F32, "bf16": L.MOE_BF16}
TORCH_DTYPE = {L.MOE_F32: torch.float32, L.MOE_BF16: torch.bfloat16}
SCORES = {"softmax": L.MOE_SOFTMAX, "sigmoid": L.MOE_SIGMOID}
LAYOUTS = {"NT": L.MOE_GEMM_NT, "NN": L.MOE_GEMM_NN, "TN": L.MOE_GEMM_TN}
EPILOGUES = {"none": L.MOE_EPI_NONE, "swiglu": L.MOE_EPI_SWIGLU, "dswiglu": L.MOE_EPI_DSWIGLU}


class MoeError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = L.load().moe_status_str(status).decode()
        super().__init__(f"{where}: {msg} (status {status})")


def _check(status: int, where: str):
    if status != L.MOE_OK:
        raise MoeError(status, where)


def _p(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensor must live in GPU memory")
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def make_desc(T, d, E, k, f, n_shared=0, f_shared=0, score="sigmoid", renorm=False, dtype="bf16"):
    return L.MoeDesc(num_tokens=T, d_model=d, num_experts=E, top_k=k, d_ff=f, num_shared=n_shared,
                     d_ff_shared=f_shared if n_shared else 0, score=SCORES[score], renorm=int(bool(renorm)),
                     dtype=DTYPES[dtype], reserved=0)


def desc_from_config(cfg, T=None):
    return make_desc(cfg.T if T is None else T, cfg.d, cfg.E, cfg.k, cfg.f, cfg.n_shared, cfg.f_shared,
                     cfg.score, cfg.renorm, cfg.dtype)


# ------------------------------------------------------------------ queries
def route_hist_elems(desc) -> int:
    return int(L.load().moe_route_hist_elems(ctypes.byref(desc)))


def workspace_bytes(desc, which: str) -> int:
    w = {"permute": L.MOE_WS_PERMUTE, "forward": L.MOE_WS_FORWARD, "backward": L.MOE_WS_BACKWARD,
         "forward_fp8": L.MOE_WS_FORWARD_FP8, "backward_fp8": L.MOE_WS_BACKWARD_FP8,
         "backward_fp8_wgrad": L.MOE_WS_BACKWARD_FP8_WGRAD}[which]
    return int(L.load().moe_workspace_bytes(ctypes.byref(desc), w))


def grouped_gemm_workspace_bytes(layout, dtype, G, M_total, N, K) -> int:
    return int(L.load().moe_grouped_gemm_workspace_bytes(LAYOUTS[layout], DTYPES[dtype], G, M_total, N, K))


# ------------------------------------------------------------------ calls
def moe_route(desc, logits, bias, idx, gate, block_hist, stream=None):
    _check(L.load().moe_route(ctypes.byref(desc), _p(logits), _p(bias), _p(idx), _p(gate), _p(block_hist),
                              _stream(stream)), "moe_route")


def moe_permute(desc, x, idx, block_hist, counts, offsets, pos, src, x_perm, ws, stream=None, tok=None):
    """x_perm may be None (no row copy); tok (int32 [T*k]) receives the token of each permuted row."""
    _check(L.load().moe_permute(ctypes.byref(desc), _p(x), _p(idx), _p(block_hist), _p(counts), _p(offsets),
                                _p(pos), _p(src), _p(tok), _p(x_perm), _p(ws), ws.numel() * ws.element_size(),
                                _stream(stream)), "moe_permute")


def moe_grouped_gemm(layout, epilogue, dtype, G, M_total, N, K, group_offsets, A, B, C, aux=None, ws=None,
                     stream=None):
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(L.load().moe_grouped_gemm(LAYOUTS[layout], EPILOGUES[epilogue], DTYPES[dtype], G, M_total, N, K,
                                     _p(group_offsets), _p(A), _p(B), _p(C), _p(aux), _p(ws), nbytes,
                                     _stream(stream)), "moe_grouped_gemm")


def moe_grouped_gemm_gather(layout, epilogue, G, M_total, N, K, group_offsets, A, B, C, rows, src_rows,
                            aux=None, stream=None):
    """bf16 grouped GEMM reading the routed rows of the token matrix through `rows` (NT: A, TN: B)."""
    _check(L.load().moe_grouped_gemm_gather(LAYOUTS[layout], EPILOGUES[epilogue], G, M_total, N, K,
                                            _p(group_offsets), _p(A), _p(B), _p(C), _p(aux), _p(rows),
                                            src_rows, _stream(stream)), "moe_grouped_gemm_gather")


def moe_combine(desc, y_perm, gate, pos, shared_y, y, stream=None):
    _check(L.load().moe_combine(ctypes.byref(desc), _p(y_perm), _p(gate), _p(pos), _p(shared_y), _p(y),
                                _stream(stream)), "moe_combine")


def _weights(w: dict) -> L.MoeWeights:
    return L.MoeWeights(*(_p(w.get(n)) for n in ("w_router", "bias", "w_gateup", "w_down", "s_gateup",
                                                  "s_down")))


SAVED_FIELDS = ("logits", "idx", "gate", "counts", "offsets", "pos", "src", "tok", "x_perm", "preact", "h",
                "y_perm",
                "s_preact", "s_h")
GRAD_FIELDS = ("d_w_router", "d_w_gateup", "d_w_down", "d_s_gateup", "d_s_down")


def moe_forward(desc, weights: dict, x, y, saved: dict, ws, stream=None):
    w = _weights(weights)
    s = L.MoeSaved(*(_p(saved.get(n)) for n in SAVED_FIELDS))
    _check(L.load().moe_forward(ctypes.byref(desc), ctypes.byref(w), _p(x), _p(y), ctypes.byref(s), _p(ws),
                                ws.numel() * ws.element_size(), _stream(stream)), "moe_forward")


def moe_forward_no_workspace(desc, weights: dict, x, y, saved: dict, stream=None):
    """moe_forward with the library's own device scratch instead of a workspace."""
    w = _weights(weights)
    s = L.MoeSaved(*(_p(saved.get(n)) for n in SAVED_FIELDS))
    _check(L.load().moe_forward_no_workspace(ctypes.byref(desc), ctypes.byref(w), _p(x), _p(y), ctypes.byref(s),
                                             _stream(stream)), "moe_forward_no_workspace")


def _terms(terms):
    if terms is None:
        return None
    return ctypes.byref(L.MoeRouterTerms(aux_coeff=float(terms.get("aux_coeff", 0.0)),
                                         seq_aux_coeff=float(terms.get("seq_aux_coeff", 0.0)),
                                         z_coeff=float(terms.get("z_coeff", 0.0)),
                                         seq_len=int(terms.get("seq_len", 0))))


def moe_backward(desc, weights: dict, x, saved: dict, dy, dx, grads: dict, ws, stream=None, terms=None,
                 losses=None):
    """terms: None or dict(aux_coeff=, seq_aux_coeff=, z_coeff=, seq_len=); losses: None or a float32
    device tensor of 3 elements receiving the aux, seq_aux and z values."""
    w = _weights(weights)
    s = L.MoeSaved(*(_p(saved.get(n)) for n in SAVED_FIELDS))
    g = L.MoeGrads(*(_p(grads.get(n)) for n in GRAD_FIELDS))
    _check(L.load().moe_backward(ctypes.byref(desc), ctypes.byref(w), _p(x), ctypes.byref(s), _p(dy), _p(dx),
                                 ctypes.byref(g), _terms(terms), _p(losses), _p(ws), ws.numel() * ws.element_size(),
                                 _stream(stream)), "moe_backward")


def _fp8_weights(w8: dict) -> L.MoeFp8Weights:
    return L.MoeFp8Weights(*(_p(w8.get(n)) for n in L.FP8_WEIGHT_FIELDS))


def moe_fp8_weights_quantize(desc, weights: dict, w8: dict, forward=True, backward=True, stream=None):
    """Writes the e4m3 copies of the expert weights into the buffers of w8 (alloc_fp8_weights)."""
    parts = (L.MOE_FP8_FORWARD_LAYOUT if forward else 0) | (L.MOE_FP8_BACKWARD_LAYOUT if backward else 0)
    w = _weights(weights)
    q = _fp8_weights(w8)
    _check(L.load().moe_fp8_weights_quantize(ctypes.byref(desc), ctypes.byref(w), ctypes.byref(q), parts,
                                             _stream(stream)), "moe_fp8_weights_quantize")


def moe_forward_fp8(desc, weights: dict, w8: dict, x, y, saved: dict, ws, stream=None):
    w = _weights(weights)
    q = _fp8_weights(w8)
    s = L.MoeSaved(*(_p(saved.get(n)) for n in SAVED_FIELDS))
    _check(L.load().moe_forward_fp8(ctypes.byref(desc), ctypes.byref(w), ctypes.byref(q), _p(x), _p(y),
                                    ctypes.byref(s), _p(ws), ws.numel() * ws.element_size(), _stream(stream)),
           "moe_forward_fp8")


def moe_backward_fp8(desc, weights: dict, w8: dict, x, saved: dict, dy, dx, grads: dict, ws, stream=None,
                     terms=None, losses=None, grad_format="e4m3", wgrad_fp8=False):
    """grad_format: "e4m3" or "e5m2" for the gradient operands of the fp8 data gradients; wgrad_fp8: the
    weight gradients in e4m3 too (workspace "backward_fp8_wgrad")."""
    w = _weights(weights)
    q = _fp8_weights(w8)
    s = L.MoeSaved(*(_p(saved.get(n)) for n in SAVED_FIELDS))
    g = L.MoeGrads(*(_p(grads.get(n)) for n in GRAD_FIELDS))
    _check(L.load().moe_backward_fp8(ctypes.byref(desc), ctypes.byref(w), ctypes.byref(q), L.FP8_FORMATS[grad_format],
                                     int(bool(wgrad_fp8)), _p(x), ctypes.byref(s),
                                     _p(dy), _p(dx), ctypes.byref(g), _terms(terms), _p(losses), _p(ws),
                                     ws.numel() * ws.element_size(), _stream(stream)), "moe_backward_fp8")


def moe_bias_update(desc, counts, rate, bias, stream=None):
    """bias [E] fp32 (in place) += rate * (mean load - counts) / mean load."""
    _check(L.load().moe_bias_update(ctypes.byref(desc), _p(counts), float(rate), _p(bias), _stream(stream)),
           "moe_bias_update")


def moe_quantize_fp8(x, q, scale, stream=None, fmt="e4m3"):
    """Row-wise fp8 quantisation ("e4m3" or "e5m2") of x [rows, cols] (bf16 or fp32) into q (uint8) and
    scale (fp32)."""
    dt = L.MOE_BF16 if x.dtype == torch.bfloat16 else L.MOE_F32
    rows, cols = x.shape[0], x.numel() // max(x.shape[0], 1)
    _check(L.load().moe_quantize_fp8(rows, cols, dt, L.FP8_FORMATS[fmt], _p(x), _p(q), _p(scale), _stream(stream)),
           "moe_quantize_fp8")


def moe_quantize_fp8_transposed(w, q, scale, stream=None):
    """w [G, R, C] -> codes q [G, C, R] and scales [G, C], quantised along R."""
    dt = L.MOE_BF16 if w.dtype == torch.bfloat16 else L.MOE_F32
    G, R, C = w.shape
    _check(L.load().moe_quantize_fp8_transposed(G, R, C, dt, _p(w), _p(q), _p(scale), _stream(stream)),
           "moe_quantize_fp8_transposed")


def moe_quantize_fp8_tensorwise(x, q, scale, ws=None, stream=None):
    """Tensor-wise e4m3 quantisation of x [rows, cols]: one scale, written to every entry of scale [rows]."""
    dt = L.MOE_BF16 if x.dtype == torch.bfloat16 else L.MOE_F32
    rows, cols = x.shape[0], x.numel() // max(x.shape[0], 1)
    need = L.load().moe_quantize_fp8_tensorwise_workspace_bytes(rows)
    if ws is None:
        ws = torch.empty(max(need, 16), dtype=torch.uint8, device=x.device)
    _check(L.load().moe_quantize_fp8_tensorwise(rows, cols, dt, _p(x), _p(q), _p(scale), _p(ws),
                                                ws.numel() * ws.element_size(), _stream(stream)),
           "moe_quantize_fp8_tensorwise")


def moe_grouped_gemm_fp8(epilogue, G, M_total, N, K, group_offsets, A, a_scale, B, b_scale, C, aux=None,
                         stream=None, a_fmt="e4m3"):
    """a_fmt: the format of A's codes ("e4m3", or "e5m2" with the "none" / "dswiglu" epilogues)."""
    _check(L.load().moe_grouped_gemm_fp8(EPILOGUES[epilogue], L.FP8_FORMATS[a_fmt], G, M_total, N, K,
                                         _p(group_offsets), _p(A),
                                         _p(a_scale), _p(B), _p(b_scale), _p(C), _p(aux), _stream(stream)),
           "moe_grouped_gemm_fp8")


def moe_quantize_fp8_colwise(x, G, offsets, pad_offsets, q, scale, rows=None, M=None, stream=None):
    """e4m3 codes of each column of x over each group's rows, stored transposed and padded (the
    operands of an fp8 weight gradient); x [src_rows, C] (read through rows when given, M rows)."""
    dt = L.MOE_BF16 if x.dtype == torch.bfloat16 else L.MOE_F32
    src_rows, C = x.shape
    M = src_rows if M is None else M
    _check(L.load().moe_quantize_fp8_colwise(G, M, C, dt, _p(offsets), _p(rows), src_rows, _p(x), _p(pad_offsets),
                                             _p(q), _p(scale), _stream(stream)), "moe_quantize_fp8_colwise")


def quantize_fp8_colwise_bytes(G, M, C) -> int:
    return int(L.load().moe_quantize_fp8_colwise_bytes(G, M, C))


def moe_grouped_gemm_fp8_wgrad(G, N, K, pad_offsets, A, a_scale, B, b_scale, C, stream=None):
    _check(L.load().moe_grouped_gemm_fp8_wgrad(G, N, K, _p(pad_offsets), _p(A), _p(a_scale), _p(B), _p(b_scale),
                                               _p(C), _stream(stream)), "moe_grouped_gemm_fp8_wgrad")


def moe_grouped_gemm_fp8_gather(epilogue, G, M_total, N, K, group_offsets, A, a_scale, B, b_scale, C, rows,
                                src_rows, aux=None, stream=None):
    """fp8 grouped GEMM reading routed row m's codes and scale at rows[m] of A [src_rows, K] / a_scale."""
    _check(L.load().moe_grouped_gemm_fp8_gather(EPILOGUES[epilogue], G, M_total, N, K, _p(group_offsets), _p(A),
                                                _p(a_scale), _p(B), _p(b_scale), _p(C), _p(aux), _p(rows),
                                                src_rows, _stream(stream)), "moe_grouped_gemm_fp8_gather")


# ------------------------------------------------------------------ buffers (torch device memory)
def alloc_saved(desc, device="cuda", training=True, gather=False) -> dict:
    """gather=True: no permuted token copy (x_perm None); the gate/up products read x through tok."""
    T, d, E, k, f = desc.num_tokens, desc.d_model, desc.num_experts, desc.top_k, desc.d_ff
    F = desc.num_shared * desc.d_ff_shared
    A = T * k
    dt = TORCH_DTYPE[desc.dtype]
    e = lambda *s, dtype=dt: torch.empty(*s, dtype=dtype, device=device)  # noqa: E731
    out = dict(logits=e(T, E, dtype=torch.float32), idx=e(T, k, dtype=torch.int32),
               gate=e(T, k, dtype=torch.float32), counts=e(E, dtype=torch.int32),
               offsets=e(E + 1, dtype=torch.int32), pos=e(A, dtype=torch.int32), src=e(A, dtype=torch.int32),
               tok=e(A, dtype=torch.int32), x_perm=None if gather else e(A, d), preact=e(A, 2 * f) if training else None, h=e(A, f), y_perm=e(A, d),
               s_preact=e(T, 2 * F) if (F and training) else None, s_h=e(T, F) if F else None)
    return out


def alloc_saved_one_buffer(desc, device="cuda", training=True, gather=False) -> dict:
    """The saved buffers as views into one allocation laid out by moe_saved_carve
    (the "_buffer" entry keeps it alive)."""
    T, d, E, k, f = desc.num_tokens, desc.d_model, desc.num_experts, desc.top_k, desc.d_ff
    F = desc.num_shared * desc.d_ff_shared
    A = T * k
    dt = TORCH_DTYPE[desc.dtype]
    flags = (L.MOE_SAVED_TRAINING if training else 0) | (0 if gather else L.MOE_SAVED_PERMUTED_COPY)
    lib = L.load()
    n = lib.moe_saved_bytes(ctypes.byref(desc), flags)
    buf = torch.empty(max(n, 256), dtype=torch.uint8, device=device)
    s = L.MoeSaved()
    _check(lib.moe_saved_carve(ctypes.byref(desc), flags, _p(buf), buf.numel(), ctypes.byref(s)), "moe_saved_carve")
    shapes = dict(logits=((T, E), torch.float32), idx=((T, k), torch.int32), gate=((T, k), torch.float32),
                  counts=((E,), torch.int32), offsets=((E + 1,), torch.int32), pos=((A,), torch.int32),
                  src=((A,), torch.int32), tok=((A,), torch.int32), x_perm=((A, d), dt), preact=((A, 2 * f), dt),
                  h=((A, f), dt), y_perm=((A, d), dt), s_preact=((T, 2 * F), dt), s_h=((T, F), dt))
    out = {"_buffer": buf}
    for name, (shape, t) in shapes.items():
        ptr = getattr(s, name)
        if ptr is None:
            out[name] = None
            continue
        off = ptr - buf.data_ptr()
        nbytes = int(np.prod(shape)) * torch.empty((), dtype=t).element_size()
        out[name] = buf[off:off + nbytes].view(t).view(*shape)
    return out


def alloc_grads(desc, device="cuda") -> dict:
    d, E, f = desc.d_model, desc.num_experts, desc.d_ff
    F = desc.num_shared * desc.d_ff_shared
    dt = TORCH_DTYPE[desc.dtype]
    return dict(d_w_router=torch.empty(E, d, dtype=torch.float32, device=device),
                d_w_gateup=torch.empty(E, 2 * f, d, dtype=dt, device=device),
                d_w_down=torch.empty(E, d, f, dtype=dt, device=device),
                d_s_gateup=torch.empty(2 * F, d, dtype=dt, device=device) if F else None,
                d_s_down=torch.empty(d, F, dtype=dt, device=device) if F else None)


def alloc_fp8_weights(desc, device="cuda", forward=True, backward=True) -> dict:
    """Buffers for the e4m3 copies of the expert weights (layouts of moe_fp8_weights_t)."""
    d, E, f = desc.d_model, desc.num_experts, desc.d_ff
    F = desc.num_shared * desc.d_ff_shared
    u8, f32 = torch.uint8, torch.float32
    shapes = {}
    if forward:
        shapes.update(gateup_q=((E, 2 * f, d), u8), gateup_s=((E, 2 * f), f32), down_q=((E, d, f), u8),
                      down_s=((E, d), f32))
        if F:
            shapes.update(s_gateup_q=((2 * F, d), u8), s_gateup_s=((2 * F,), f32), s_down_q=((d, F), u8),
                          s_down_s=((d,), f32))
    if backward:
        shapes.update(gateup_tq=((E, d, 2 * f), u8), gateup_ts=((E, d), f32), down_tq=((E, f, d), u8),
                      down_ts=((E, f), f32))
        if F:
            shapes.update(s_gateup_tq=((d, 2 * F), u8), s_gateup_ts=((d,), f32), s_down_tq=((F, d), u8),
                          s_down_ts=((F,), f32))
    return {n: torch.empty(sh, dtype=dt, device=device) for n, (sh, dt) in shapes.items()}


def alloc_workspace(desc, which: str, device="cuda") -> torch.Tensor:
    n = max(workspace_bytes(desc, which), 256)
    return torch.empty(n, dtype=torch.uint8, device=device)


def mfma_ceiling(kind: str, iters: int, out, stream=None) -> float:
    """Launch the matrix-core rate kernel of one instruction kind (L.MFMA_KINDS); returns its flops."""
    flop = ctypes.c_double(0.0)
    _check(L.load().moe_mfma_ceiling(L.MFMA_KINDS.index(kind), int(iters), _p(out), ctypes.byref(flop),
                                     _stream(stream)), "moe_mfma_ceiling")
    return flop.value


def hbm_ceiling(src, dst, stream=None):
    """Copy src to dst (same byte size, a multiple of 16) with the streaming
    kernels' access pattern; the caller times it."""
    nbytes = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() != nbytes:
        raise ValueError("hbm_ceiling: src and dst sizes differ")
    _check(L.load().moe_hbm_ceiling(_p(src), _p(dst), nbytes, _stream(stream)), "moe_hbm_ceiling")


def stage_timing(enable: bool, stages=None):
    """Start (clearing earlier records) or stop per-stage event timing of
    moe_forward / moe_backward; `stages` (names from STAGES) limits it to
    those stages."""
    if stages is None or not enable:
        _check(L.load().moe_stage_timing(int(bool(enable))), "moe_stage_timing")
        return
    mask = 0
    for name in stages:
        mask |= 1 << L.STAGES.index(name)
    _check(L.load().moe_stage_timing_mask(mask), "moe_stage_timing_mask")


def stage_times() -> dict:
    """{stage: (total ms, launches)} of everything recorded since timing was
    enabled or last read; waits for the recorded events."""
    ms = (ctypes.c_double * L.MOE_NUM_STAGES)()
    n = (ctypes.c_int64 * L.MOE_NUM_STAGES)()
    _check(L.load().moe_stage_times(ms, n), "moe_stage_times")
    return {name: (ms[i], n[i]) for i, name in enumerate(L.STAGES)}
