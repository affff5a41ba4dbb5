"""Seeded synthetic inputs for the MoE layer (shared by tests, bench and smoke).

This module only draws random numbers and casts them; it holds none of the
layer's arithmetic (no routing, no GEMM, no activation).  The HIP path and the
oracle both consume exactly the arrays produced here.

Recipe (stands in for the workloads the pages describe; no dataset is used):
  * every normal tensor is filled in row-major chunks of 2^20 elements,
    chunk c from ``np.random.default_rng([seed, tensor_id, c])``, seed 0,
    with the tensor ids listed in ``TENSOR_ID`` (the bias and the skew
    permutation use ``default_rng([seed, tensor_id])``);
  * x ~ N(0, 1) (the normalised hidden state entering the MoE block);
  * expert / shared weights ~ N(0, 1/fan_in) (variance 1/fan_in);
  * router weight ~ N(0, 0.02^2) (standard deviation 0.02), fp32 always;
  * router bias ~ U(-0.1, 0.1), or the skewed recipe of ``skew_bias``;
  * upstream gradient dY ~ N(0, 1);
  * values are drawn in fp32 and, for bf16 layers, rounded to bf16 with
    round-to-nearest-even.  Both sides see the identical bf16 values.

Shapes follow the pages' models: hidden 2048 and 64 experts as in the Ultimate
MoE Training Handbook (section 2.5, "First training of MoE"), sequences of 4096
tokens (section 2.4, dense baseline), and 128 experts / top-8 as in the
GPTConfig of the "Train Large Model from Scratch" README.
"""
from __future__ import annotations

import dataclasses
import json
import os
from typing import Optional

import numpy as np

TENSOR_ID = {
    "x": 0, "w_router": 1, "bias": 2, "w_gate": 3, "w_up": 4, "w_down": 5,
    "s_gate": 6, "s_up": 7, "s_down": 8, "dy": 9, "skew_perm": 10,
}


@dataclasses.dataclass(frozen=True)
class LayerConfig:
    name: str
    T: int                 # tokens
    d: int                 # d_model
    E: int                 # routed experts
    k: int                 # experts per token
    f: int                 # routed expert d_ff
    n_shared: int          # shared experts
    f_shared: int          # d_ff of each shared expert
    score: str             # "softmax" | "sigmoid"
    renorm: bool           # softmax only: renormalise the top-k probabilities
    bias: Optional[str]    # None | "uniform" | "zipf"
    dtype: str             # "f32" | "bf16"
    backward: bool         # whether the workload runs the backward pass
    seed: int = 0

    @property
    def F_shared(self) -> int:
        return self.n_shared * self.f_shared

    @property
    def A(self) -> int:
        return self.T * self.k

    def replace(self, **kw) -> "LayerConfig":
        return dataclasses.replace(self, **kw)


CONFIGS = [
    LayerConfig("tiny_fp32", T=256, d=128, E=8, k=2, f=256, n_shared=0, f_shared=0,
                score="softmax", renorm=False, bias=None, dtype="f32", backward=False),
    LayerConfig("finegrained_bf16", T=4096, d=1024, E=64, k=8, f=512, n_shared=1, f_shared=1024,
                score="sigmoid", renorm=True, bias="uniform", dtype="bf16", backward=False),
    LayerConfig("moe7b_bf16", T=16384, d=2048, E=64, k=6, f=1408, n_shared=2, f_shared=1408,
                score="sigmoid", renorm=True, bias="uniform", dtype="bf16", backward=True),
    LayerConfig("skew_bf16", T=16384, d=2048, E=64, k=6, f=1408, n_shared=2, f_shared=1408,
                score="sigmoid", renorm=True, bias="zipf", dtype="bf16", backward=True),
    LayerConfig("large_bf16", T=65536, d=4096, E=128, k=8, f=1536, n_shared=1, f_shared=4096,
                score="sigmoid", renorm=True, bias="uniform", dtype="bf16", backward=True),
]
CONFIG_BY_NAME = {c.name: c for c in CONFIGS}


def rng(cfg: LayerConfig, tensor: str) -> np.random.Generator:
    return np.random.default_rng([cfg.seed, TENSOR_ID[tensor]])


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (round-to-nearest-even) and return the raw uint16 bits."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    nan = np.isnan(a)
    if nan.any():
        r = np.where(nan, np.uint32(0x7FC0), r)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


CHUNK = 1 << 20   # elements per independently seeded chunk


def _fill_chunk(args):
    seed, tid, c, std, flat, bf16 = args
    g = np.random.default_rng([seed, tid, c])
    v = g.standard_normal(flat.size, dtype=np.float32)
    if std != 1.0:
        v *= np.float32(std)
    if bf16:
        u = v.view(np.uint32)
        r = (u >> np.uint32(16)) & np.uint32(1)
        r += np.uint32(0x7FFF)
        r += u
        r >>= np.uint32(16)
        flat[...] = r
    else:
        flat[...] = v


_POOL = None


def _pool():
    global _POOL
    if _POOL is None:
        from concurrent.futures import ThreadPoolExecutor
        n = min(16, len(os.sched_getaffinity(0)))
        _POOL = ThreadPoolExecutor(max(1, n))
    return _POOL


def _normal(cfg, tensor, shape, std):
    """N(0, std^2) values, stored in the layer's dtype.

    The tensor is filled in row-major order, in chunks of CHUNK elements;
    chunk c is drawn as standard normal fp32 from
    default_rng([seed, tensor_id, c]), multiplied by std in fp32 and, for bf16
    layers, rounded to bf16 (nearest even).  Returned as fp32, or as raw bf16
    bits in uint16."""
    shape = tuple(int(s) for s in shape)
    n = int(np.prod(shape))
    bf16 = cfg.dtype != "f32"
    out = np.empty(n, dtype=np.uint16 if bf16 else np.float32)
    jobs = [(cfg.seed, TENSOR_ID[tensor], c, float(std), out[c * CHUNK:(c + 1) * CHUNK], bf16)
            for c in range((n + CHUNK - 1) // CHUNK)]
    list(_pool().map(_fill_chunk, jobs))
    return out.reshape(shape)


def _skew_alpha_path():
    return os.path.join(os.path.dirname(os.path.abspath(__file__)), "skew_alpha.json")


def skew_bias(cfg: LayerConfig, alpha: Optional[float] = None) -> np.ndarray:
    """Zipf-shaped router bias for the skewed-load layer.

    A seeded permutation gives every expert a rank r = 1..E.  The E-4 best
    ranks get b = -1.2 * alpha * ln(r) (a Zipf(s=1.2) profile in log space);
    the 4 worst ranks get b = -2.0, below every reachable sigmoid score, so
    those experts receive no tokens.  alpha is calibrated once (by a script
    that runs the oracle's router) so that the busiest expert receives about
    4x the mean load; the calibrated value is stored in skew_alpha.json."""
    if alpha is None:
        with open(_skew_alpha_path()) as fh:
            alpha = float(json.load(fh)[cfg.name]["alpha"])
    perm = rng(cfg, "skew_perm").permutation(cfg.E)
    ranks = np.empty(cfg.E, dtype=np.int64)
    ranks[perm] = np.arange(1, cfg.E + 1)
    b = (-1.2 * alpha * np.log(ranks.astype(np.float64))).astype(np.float32)
    b[ranks > cfg.E - 4] = np.float32(-2.0)
    return b


ALL_PARTS = ("x", "router", "experts", "shared", "dy")


def make_inputs(cfg: LayerConfig, with_dy: Optional[bool] = None, skew_alpha: Optional[float] = None,
                parts=None):
    """Return a dict of host arrays for one layer.

    Keys: x [T,d]; w_router [E,d] f32; bias [E] f32 or None; w_gateup [E,2f,d]
    (gate rows first, then up rows); w_down [E,d,f]; s_gateup [2F_s,d] and
    s_down [d,F_s] (None without shared experts); dy [T,d] when requested.
    bf16 tensors are uint16 bit patterns.  ``parts`` limits what is drawn
    (any of "x", "router", "experts", "shared", "dy"); every tensor has its
    own stream, so a subset is identical to the same keys of the full set."""
    if with_dy is None:
        with_dy = cfg.backward
    parts = set(ALL_PARTS if parts is None else parts)
    if not with_dy:
        parts.discard("dy")
    T, d, E, f, Fs = cfg.T, cfg.d, cfg.E, cfg.f, cfg.F_shared
    out = {}
    if "x" in parts:
        out["x"] = _normal(cfg, "x", (T, d), 1.0)
    if "router" in parts:
        out["w_router"] = _normal(cfg.replace(dtype="f32"), "w_router", (E, d), 0.02)
        if cfg.bias is None:
            out["bias"] = None
        elif cfg.bias == "uniform":
            out["bias"] = rng(cfg, "bias").uniform(-0.1, 0.1, size=E).astype(np.float32)
        elif cfg.bias == "zipf":
            out["bias"] = skew_bias(cfg, skew_alpha)
        else:
            raise ValueError(cfg.bias)
    if "experts" in parts:
        _experts(cfg, out)
    if "shared" in parts:
        _shared(cfg, out)
    if "dy" in parts:
        out["dy"] = _normal(cfg, "dy", (T, d), 1.0)
    return out


def _experts(cfg, out):
    T, d, E, f = cfg.T, cfg.d, cfg.E, cfg.f
    wg = _normal(cfg, "w_gate", (E * f, d), 1.0 / np.sqrt(d)).reshape(E, f, d)
    wu = _normal(cfg, "w_up", (E * f, d), 1.0 / np.sqrt(d)).reshape(E, f, d)
    out["w_gateup"] = np.concatenate([wg, wu], axis=1)
    del wg, wu
    out["w_down"] = _normal(cfg, "w_down", (E * d, f), 1.0 / np.sqrt(f)).reshape(E, d, f)


def _shared(cfg, out):
    d, Fs = cfg.d, cfg.F_shared
    if Fs > 0:
        sg = _normal(cfg, "s_gate", (Fs, d), 1.0 / np.sqrt(d))
        su = _normal(cfg, "s_up", (Fs, d), 1.0 / np.sqrt(d))
        out["s_gateup"] = np.concatenate([sg, su], axis=0)
        out["s_down"] = _normal(cfg, "s_down", (d, Fs), 1.0 / np.sqrt(cfg.f_shared))
    else:
        out["s_gateup"] = None
        out["s_down"] = None


def as_f64(a: Optional[np.ndarray], dtype: str) -> Optional[np.ndarray]:
    """Exact conversion of a stored tensor (fp32 or bf16 bits) to float64."""
    if a is None:
        return None
    if a.dtype == np.uint16:
        return bf16_bits_to_f32(a).astype(np.float64)
    return a.astype(np.float64)
