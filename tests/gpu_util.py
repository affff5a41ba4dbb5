"""Helpers for GPU parity tests: host <-> device transfer of synth arrays and
the comparison metrics the tolerances are stated in."""
import numpy as np
import torch

import synth


def dev(a, dtype=None):
    """Host array -> CUDA tensor.  uint16 arrays are bf16 bit patterns."""
    if a is None:
        return None
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    t = torch.from_numpy(a)
    if dtype is not None:
        t = t.to(dtype)
    return t.cuda()


def host(t):
    """CUDA tensor -> numpy (bf16 -> float64 exactly; others keep their dtype)."""
    if t.dtype == torch.bfloat16:
        bits = t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
        return synth.bf16_bits_to_f32(bits).astype(np.float64)
    return t.cpu().numpy()


def rel_l2(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def max_abs_over_rms(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    rms = np.sqrt(np.mean(b * b))
    return float(np.max(np.abs(a - b)) / max(rms, 1e-300))


# tolerances: fp32 layer rel-L2 <= 1e-5; bf16 layers rel-L2 <= 1e-2 and
# max-abs <= 5e-2 * RMS(reference)
def assert_close(gpu, ref, dtype, what=""):
    r = rel_l2(gpu, ref)
    if dtype == "f32":
        assert r <= 1e-5, f"{what}: rel-L2 {r:.3e} > 1e-5"
    else:
        m = max_abs_over_rms(gpu, ref)
        assert r <= 1e-2, f"{what}: rel-L2 {r:.3e} > 1e-2"
        assert m <= 5e-2, f"{what}: max-abs/RMS {m:.3e} > 5e-2"
    return r


def assert_close_per_expert(gpu, ref, what=""):
    """Routed weight gradients of degenerate routings (one token, every token
    on one expert, a few rows per expert): each expert's matrix (a slice
    along the first axis) is compared on its own.  A slice with an all-zero
    reference must be exactly zero;
    otherwise rel-L2 <= 1e-2 over the tensor and per expert, and every
    element at least as large as its expert's RMS within 5 % of its value.
    (The max-abs <= 5e-2 * RMS bar assumes each element sums many rows; for
    a rank-one gradient the largest elements are 10+ times the RMS and one
    bf16 rounding of them exceeds that bar.)"""
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    r = rel_l2(gpu, ref)
    assert r <= 1e-2, f"{what}: rel-L2 {r:.3e} > 1e-2"
    for e in range(ref.shape[0]):
        g, x = gpu[e], ref[e]
        rms = np.sqrt(np.mean(x * x))
        if rms == 0.0:
            assert np.all(g == 0.0), f"{what}: slice {e} with a zero reference is not zero"
            continue
        re = rel_l2(g, x)
        assert re <= 1e-2, f"{what}: slice {e} rel-L2 {re:.3e} > 1e-2"
        big = np.abs(x) >= rms
        worst = np.max(np.abs(g[big] - x[big]) / np.abs(x[big]))
        assert worst <= 5e-2, f"{what}: slice {e} relative error {worst:.3e} > 5e-2 on |ref| >= RMS"
    return r


def assert_close_large(gpu, ref, what=""):
    """A rank-one weight gradient (one token) of a single matrix: rel-L2 <=
    1e-2 over the tensor and every element at least as large as the tensor's
    RMS within 5 % of its value.  Small elements are rows or columns scaled
    by a near-zero factor, whose relative error says nothing about the
    arithmetic."""
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    r = rel_l2(gpu, ref)
    assert r <= 1e-2, f"{what}: rel-L2 {r:.3e} > 1e-2"
    rms = np.sqrt(np.mean(ref * ref))
    if rms == 0.0:
        assert np.all(gpu == 0.0), f"{what}: zero reference, nonzero result"
        return r
    big = np.abs(ref) >= rms
    worst = np.max(np.abs(gpu[big] - ref[big]) / np.abs(ref[big]))
    assert worst <= 5e-2, f"{what}: relative error {worst:.3e} > 5e-2 on |ref| >= RMS"
    return r


def assert_rounded(gpu, ref, dtype, what="", extra=0.0):
    """Outputs stored once in `dtype` after fp32 accumulation: each element
    may differ from the exact value by one rounding (half an ulp: 2^-8
    relative for bf16, 2^-24 for fp32) plus fp32 accumulation noise.
    `extra` (scalar or per element) widens the bound by an error the value
    inherits from its inputs before that rounding."""
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    rms = np.sqrt(np.mean(ref * ref))
    r = rel_l2(gpu, ref)
    if dtype == "f32":
        assert r <= 1e-5, f"{what}: rel-L2 {r:.3e} > 1e-5"
        return r
    assert r <= 1e-2, f"{what}: rel-L2 {r:.3e} > 1e-2"
    bound = 2.0 ** -8 * np.abs(ref) * (1 + 1e-3) + 1e-4 * rms + extra
    bad = np.abs(gpu - ref) > bound
    if bad.any():
        w = np.argsort(-(np.abs(gpu - ref) / bound).ravel())[:5]
        print(f"{what}: worst gpu / ref / bound:",
              [(float(gpu.ravel()[i]), float(ref.ravel()[i]), float(bound.ravel()[i])) for i in w], flush=True)
    assert not bad.any(), f"{what}: {bad.sum()} elements beyond one bf16 rounding"
    return r


def ulp_f32(x):
    x = np.abs(np.asarray(x, np.float32))
    return np.spacing(x).astype(np.float64)
