"""ctypes view of the C ABI in include/moe.h (structs, enums, signatures).

Loading fails loudly if the built library is missing: there is no fallback."""
from __future__ import annotations

import ctypes
import os
import re

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libmoe_mi355x.so")
HEADER = os.path.join(os.path.dirname(PKG), "include", "moe.h")

c_i32, c_i64, c_sz, c_vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.c_void_p

MOE_OK, MOE_ERR_INVALID, MOE_ERR_ALIGN, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_HIP = range(6)
MOE_F32, MOE_BF16 = 0, 1
MOE_SOFTMAX, MOE_SIGMOID = 0, 1
MOE_GEMM_NT, MOE_GEMM_NN, MOE_GEMM_TN = 0, 1, 2
MOE_EPI_NONE, MOE_EPI_SWIGLU, MOE_EPI_DSWIGLU = 0, 1, 2
MOE_WS_PERMUTE, MOE_WS_FORWARD, MOE_WS_BACKWARD, MOE_WS_FORWARD_FP8, MOE_WS_BACKWARD_FP8 = 0, 1, 2, 3, 4
MOE_WS_BACKWARD_FP8_WGRAD = 5
MOE_FP8_FORWARD_LAYOUT, MOE_FP8_BACKWARD_LAYOUT = 1, 2
MOE_E4M3, MOE_E5M2 = 0, 1
FP8_FORMATS = {"e4m3": MOE_E4M3, "e5m2": MOE_E5M2}
MOE_SAVED_TRAINING, MOE_SAVED_PERMUTED_COPY = 1, 2
MOE_ROUTE_BLOCK = 32
MFMA_KINDS = ["bf16_32x32x16", "bf16_16x16x32", "e4m3_32x32x64", "e4m3_16x16x128"]
STAGES = ["router", "route", "permute", "gate_up", "down", "shared_gate_up", "shared_down", "combine",
          "combine_bwd", "down_dgrad", "down_wgrad", "gate_up_wgrad", "gate_up_dgrad", "shared_down_dgrad",
          "shared_down_wgrad", "shared_gate_up_wgrad", "shared_gate_up_dgrad", "router_wgrad",
          "unpermute_sum", "router_terms", "fp8_quantize"]
MOE_NUM_STAGES = len(STAGES)


class MoeDesc(ctypes.Structure):
    _fields_ = [("num_tokens", c_i64), ("d_model", c_i64), ("num_experts", c_i64), ("top_k", c_i64),
                ("d_ff", c_i64), ("num_shared", c_i64), ("d_ff_shared", c_i64), ("score", c_i32),
                ("renorm", c_i32), ("dtype", c_i32), ("reserved", c_i32)]


class MoeWeights(ctypes.Structure):
    _fields_ = [("w_router", c_vp), ("bias", c_vp), ("w_gateup", c_vp), ("w_down", c_vp),
                ("s_gateup", c_vp), ("s_down", c_vp)]


class MoeSaved(ctypes.Structure):
    _fields_ = [("logits", c_vp), ("idx", c_vp), ("gate", c_vp), ("counts", c_vp), ("offsets", c_vp),
                ("pos", c_vp), ("src", c_vp), ("tok", c_vp), ("x_perm", c_vp), ("preact", c_vp), ("h", c_vp),
                ("y_perm", c_vp), ("s_preact", c_vp), ("s_h", c_vp)]


FP8_WEIGHT_FIELDS = ("gateup_q", "gateup_s", "down_q", "down_s", "gateup_tq", "gateup_ts", "down_tq", "down_ts",
                     "s_gateup_q", "s_gateup_s", "s_down_q", "s_down_s", "s_gateup_tq", "s_gateup_ts",
                     "s_down_tq", "s_down_ts")


class MoeFp8Weights(ctypes.Structure):
    _fields_ = [(n, c_vp) for n in FP8_WEIGHT_FIELDS]


class MoeRouterTerms(ctypes.Structure):
    _fields_ = [("aux_coeff", ctypes.c_float), ("seq_aux_coeff", ctypes.c_float), ("z_coeff", ctypes.c_float),
                ("seq_len", c_i32)]


class MoeGrads(ctypes.Structure):
    _fields_ = [("d_w_router", c_vp), ("d_w_gateup", c_vp), ("d_w_down", c_vp), ("d_s_gateup", c_vp),
                ("d_s_down", c_vp)]


_P = ctypes.POINTER
SIGNATURES = {
    "moe_status_str": (ctypes.c_char_p, [c_i32]),
    "moe_abi_version": (c_i32, []),
    "moe_route_hist_elems": (c_sz, [_P(MoeDesc)]),
    "moe_workspace_bytes": (c_sz, [_P(MoeDesc), c_i32]),
    "moe_grouped_gemm_workspace_bytes": (c_sz, [c_i32, c_i32, c_i64, c_i64, c_i64, c_i64]),
    "moe_route": (c_i32, [_P(MoeDesc), c_vp, c_vp, c_vp, c_vp, c_vp, c_vp]),
    "moe_permute": (c_i32, [_P(MoeDesc), c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_sz,
                            c_vp]),
    "moe_saved_bytes": (c_sz, [_P(MoeDesc), c_i32]),
    "moe_saved_carve": (c_i32, [_P(MoeDesc), c_i32, c_vp, c_sz, _P(MoeSaved)]),
    "moe_grouped_gemm_gather": (c_i32, [c_i32, c_i32, c_i64, c_i64, c_i64, c_i64, c_vp, c_vp, c_vp, c_vp,
                                        c_vp, c_vp, c_i64, c_vp]),
    "moe_grouped_gemm": (c_i32, [c_i32, c_i32, c_i32, c_i64, c_i64, c_i64, c_i64, c_vp, c_vp, c_vp, c_vp,
                                 c_vp, c_vp, c_sz, c_vp]),
    "moe_combine": (c_i32, [_P(MoeDesc), c_vp, c_vp, c_vp, c_vp, c_vp, c_vp]),
    "moe_forward": (c_i32, [_P(MoeDesc), _P(MoeWeights), c_vp, c_vp, _P(MoeSaved), c_vp, c_sz, c_vp]),
    "moe_forward_no_workspace": (c_i32, [_P(MoeDesc), _P(MoeWeights), c_vp, c_vp, _P(MoeSaved), c_vp]),
    "moe_backward": (c_i32, [_P(MoeDesc), _P(MoeWeights), c_vp, _P(MoeSaved), c_vp, c_vp, _P(MoeGrads),
                             _P(MoeRouterTerms), c_vp, c_vp, c_sz, c_vp]),
    "moe_forward_fp8": (c_i32, [_P(MoeDesc), _P(MoeWeights), _P(MoeFp8Weights), c_vp, c_vp, _P(MoeSaved), c_vp,
                                c_sz, c_vp]),
    "moe_backward_fp8": (c_i32, [_P(MoeDesc), _P(MoeWeights), _P(MoeFp8Weights), c_i32, c_i32, c_vp, _P(MoeSaved),
                                 c_vp, c_vp, _P(MoeGrads), _P(MoeRouterTerms), c_vp, c_vp, c_sz, c_vp]),
    "moe_quantize_fp8_colwise_bytes": (c_sz, [c_i64, c_i64, c_i64]),
    "moe_quantize_fp8_colwise": (c_i32, [c_i64, c_i64, c_i64, c_i32, c_vp, c_vp, c_i64, c_vp, c_vp, c_vp, c_vp,
                                         c_vp]),
    "moe_grouped_gemm_fp8_wgrad": (c_i32, [c_i64, c_i64, c_i64, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp]),
    "moe_fp8_weights_quantize": (c_i32, [_P(MoeDesc), _P(MoeWeights), _P(MoeFp8Weights), c_i32, c_vp]),
    "moe_grouped_gemm_fp8_gather": (c_i32, [c_i32, c_i64, c_i64, c_i64, c_i64, c_vp, c_vp, c_vp, c_vp, c_vp,
                                            c_vp, c_vp, c_vp, c_i64, c_vp]),
    "moe_bias_update": (c_i32, [_P(MoeDesc), c_vp, ctypes.c_float, c_vp, c_vp]),
    "moe_quantize_fp8": (c_i32, [c_i64, c_i64, c_i32, c_i32, c_vp, c_vp, c_vp, c_vp]),
    "moe_quantize_fp8_transposed": (c_i32, [c_i64, c_i64, c_i64, c_i32, c_vp, c_vp, c_vp, c_vp]),
    "moe_quantize_fp8_tensorwise_workspace_bytes": (c_sz, [c_i64]),
    "moe_quantize_fp8_tensorwise": (c_i32, [c_i64, c_i64, c_i32, c_vp, c_vp, c_vp, c_vp, c_sz, c_vp]),
    "moe_grouped_gemm_fp8": (c_i32, [c_i32, c_i32, c_i64, c_i64, c_i64, c_i64, c_vp, c_vp, c_vp, c_vp, c_vp,
                                     c_vp, c_vp, c_vp]),
    "moe_mfma_ceiling": (c_i32, [c_i32, c_i64, c_vp, _P(ctypes.c_double), c_vp]),
    "moe_hbm_ceiling": (c_i32, [c_vp, c_vp, c_i64, c_vp]),
    "moe_stage_timing_mask": (c_i32, [ctypes.c_uint32]),
    "moe_stage_timing": (c_i32, [c_i32]),
    "moe_stage_times": (c_i32, [_P(ctypes.c_double), _P(c_i64)]),
}

_lib = None


def header_functions():
    """Names of the functions declared in include/moe.h."""
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(moe_\w+)\s*\(", text, re.M)))


def load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"HIP library not built: {LIB_PATH} is missing "
                           "(run python -m mixture_experts_layer_18_amd.build)")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib
