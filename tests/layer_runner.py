"""Run the whole layer on the GPU through the C ABI and compare with the oracle.

Comparison protocol (same for every layer size):
  * router logits: rel-L2 <= 1e-5 (fp32 accumulation on both sides);
  * routing indices: bit-exact on every token whose oracle selection margin
    (k-th minus (k+1)-th key) is >= 1e-3; on the other tokens the GPU's
    choice must be valid: each picked key >= the oracle's k-th key - 1e-3;
  * outputs, input gradients and weight gradients: compared on every token,
    with the oracle re-run on the GPU's routing (its expert indices forced,
    its gates recomputed from the oracle's own scores) wherever a near-tie
    made the two choose differently; the number of such tokens is reported;
  * tolerance: fp32 rel-L2 <= 1e-5; bf16 rel-L2 <= 1e-2 and
    max-abs <= 5e-2 * RMS(reference)."""
import numpy as np
import torch

import synth
from oracle import moe_oracle as O
from tests.gpu_util import assert_close, assert_close_large, assert_close_per_expert, dev, host, rel_l2

import mixture_experts_layer_18_amd as M

MARGIN = 1e-3


def upload_layer(cfg, inp):
    w = dict(w_router=dev(inp["w_router"]), bias=dev(inp["bias"]), w_gateup=dev(inp["w_gateup"]),
             w_down=dev(inp["w_down"]), s_gateup=dev(inp.get("s_gateup")), s_down=dev(inp.get("s_down")))
    return w


def run_gpu(cfg, inp, backward, weights=None, x=None, dy=None, keep_device=False, terms=None, gather=False,
            fp8=False, grad_format="e4m3", wgrad_fp8=False):
    """gather: no permuted token copy; the gate/up products read x through the token map.
    fp8: the fp8 layer calls (moe_forward_fp8 / moe_backward_fp8) on e4m3 copies of the
    expert weights written by moe_fp8_weights_quantize."""
    desc = M.desc_from_config(cfg)
    w = upload_layer(cfg, inp) if weights is None else weights
    x = dev(inp["x"]) if x is None else x
    saved = M.alloc_saved(desc, training=backward, gather=gather)
    y = torch.empty_like(x)
    w8 = None
    if fp8:
        w8 = M.alloc_fp8_weights(desc, backward=backward)
        M.moe_fp8_weights_quantize(desc, w, w8, forward=True, backward=backward)
        M.moe_forward_fp8(desc, w, w8, x, y, saved, M.alloc_workspace(desc, "forward_fp8"))
    else:
        ws = M.alloc_workspace(desc, "forward")
        M.moe_forward(desc, w, x, y, saved, ws)
    out = dict(y=y, saved=saved, w8=w8)
    if backward:
        dy = dev(inp["dy"]) if dy is None else dy
        grads = M.alloc_grads(desc)
        dx = torch.empty_like(x)
        losses = torch.zeros(4, dtype=torch.float32, device="cuda") if terms is not None else None
        if fp8:
            wsb = M.alloc_workspace(desc, "backward_fp8_wgrad" if wgrad_fp8 else "backward_fp8")
            M.moe_backward_fp8(desc, w, w8, x, saved, dy, dx, grads, wsb, terms=terms, losses=losses,
                               grad_format=grad_format, wgrad_fp8=wgrad_fp8)
        else:
            wsb = M.alloc_workspace(desc, "backward")
            M.moe_backward(desc, w, x, saved, dy, dx, grads, wsb, terms=terms, losses=losses)
        out.update(dx=dx, grads=grads, losses=losses)
    torch.cuda.synchronize()
    if keep_device:
        return out
    res = dict(y=host(y), logits=saved["logits"].cpu().numpy(), idx=saved["idx"].cpu().numpy(),
               gate=saved["gate"].cpu().numpy(), counts=saved["counts"].cpu().numpy(),
               offsets=saved["offsets"].cpu().numpy())
    if backward:
        res["dx"] = host(out["dx"])
        if out["losses"] is not None:
            res["losses"] = out["losses"][:3].cpu().numpy()
        for n, t in out["grads"].items():
            if t is not None:
                res[n] = host(t)
    return res


def oracle_inputs(cfg, inp):
    """Exact values of the stored inputs.  Expert weights stay fp32 (exact for
    bf16 values); the oracle widens each expert to fp64 when it uses it."""
    f = lambda a: synth.as_f64(a, cfg.dtype)  # noqa: E731
    w32 = lambda a: synth.bf16_bits_to_f32(a) if a.dtype == np.uint16 else a  # noqa: E731
    return dict(x=f(inp["x"]), w_router=inp["w_router"], bias=inp["bias"], w_gateup=w32(inp["w_gateup"]),
                w_down=w32(inp["w_down"]), s_gateup=f(inp.get("s_gateup")), s_down=f(inp.get("s_down")),
                dy=f(inp.get("dy")) if inp.get("dy") is not None else None)


def oracle_run(cfg, oi, backward, tokens=None, terms=None):
    x = oi["x"] if tokens is None else oi["x"][tokens]
    fw = O.forward(x, oi["w_router"], oi["bias"], oi["w_gateup"], oi["w_down"], oi["s_gateup"], oi["s_down"],
                   top_k=cfg.k, score=cfg.score, renorm=cfg.renorm)
    bw = None
    if backward:
        dy = oi["dy"] if tokens is None else oi["dy"][tokens]
        bw = O.backward(x, oi["w_router"], oi["w_gateup"], oi["w_down"], oi["s_gateup"], oi["s_down"], fw, dy,
                        score=cfg.score, renorm=cfg.renorm, terms=terms)
    return fw, bw


def oracle_routing(cfg, oi):
    """The oracle's router on every token (logits, keys, its own top-k and
    margins), without the experts: enough for check_routing."""
    logits = O.router_logits(oi["x"], oi["w_router"])
    scores = O.router_scores(logits, cfg.score)
    keys = O.selection_keys(logits, scores, oi["bias"], cfg.score)
    idx, margin = O.select_topk(keys, cfg.k)
    return dict(logits=logits, scores=scores, keys=keys, idx=idx, margin=margin)


def check_routing(cfg, g_logits, g_idx, fw, tokens=None):
    """Check the GPU routing against the oracle's; returns the mask of tokens
    whose GPU expert set equals the oracle's (their outputs are comparable).

    Tokens whose boundary margin (k-th minus (k+1)-th key) is >= 1e-3 must
    pick the same expert set; if in addition every gap between consecutive
    keys inside the top k is >= 1e-3, the slots must match in order too.
    Every other token must make a valid choice: k distinct experts, each
    with key >= the oracle's k-th key - 1e-3, listed in non-increasing key
    order up to 1e-3."""
    ol = fw["logits"]
    gl = g_logits if tokens is None else g_logits[tokens]
    gi = g_idx if tokens is None else g_idx[tokens]
    r = rel_l2(gl, ol)
    assert r <= 1e-5, f"logits rel-L2 {r:.3e}"
    keys = fw["keys"].astype(np.float64)
    srt = -np.sort(-keys, axis=1)
    k = cfg.k
    inner_gap = (srt[:, :k - 1] - srt[:, 1:k]).min(axis=1) if k > 1 else np.full(len(srt), np.inf)
    clear_set = fw["margin"] >= MARGIN
    clear_order = clear_set & (inner_gap >= MARGIN)
    same_set = np.all(np.sort(gi, axis=1) == np.sort(fw["idx"], axis=1), axis=1)
    same_order = np.all(gi == fw["idx"], axis=1)
    for name, bad in (("expert set", clear_set & ~same_set), ("slot order", clear_order & ~same_order)):
        if bad.any():
            for t in np.where(bad)[0][:5]:
                d = np.abs(gl[t].astype(np.float64) - ol[t])
                print(f"token {t}: margin {fw['margin'][t]:.3e} inner gap {inner_gap[t]:.3e} oracle "
                      f"{fw['idx'][t].tolist()} gpu {gi[t].tolist()} max|dlogit| {d.max():.3e}", flush=True)
        assert not bad.any(), f"{bad.sum()} clear tokens differ in {name}"
    # near-tie tokens: the GPU's picks must be a valid top-k
    kth = srt[:, k - 1]
    picked = np.take_along_axis(keys, gi.astype(np.int64), axis=1)
    assert np.all(picked >= kth[:, None] - MARGIN)
    assert np.all(picked[:, :-1] >= picked[:, 1:] - MARGIN)
    assert np.all(np.diff(np.sort(gi, axis=1), axis=1) > 0), "repeated expert"
    return same_set


def oracle_on_gpu_routing(cfg, oi, g_idx, backward, fw, bw, tokens=None, terms=None):
    """The oracle's forward (and backward) with the GPU's expert choice forced,
    when any token's choice (set or slot order) differs from the oracle's own;
    otherwise the given results.  Returns (fw, bw, flipped token count)."""
    gi = g_idx if tokens is None else g_idx[tokens]
    flips = int(np.sum(np.any(gi != fw["idx"], axis=1)))
    if flips == 0:
        return fw, bw, 0
    x = oi["x"] if tokens is None else oi["x"][tokens]
    fw = O.forward(x, oi["w_router"], oi["bias"], oi["w_gateup"], oi["w_down"], oi["s_gateup"], oi["s_down"],
                   top_k=cfg.k, score=cfg.score, renorm=cfg.renorm, forced_idx=gi)
    if backward:
        dy = oi["dy"] if tokens is None else oi["dy"][tokens]
        bw = O.backward(x, oi["w_router"], oi["w_gateup"], oi["w_down"], oi["s_gateup"], oi["s_down"], fw, dy,
                        score=cfg.score, renorm=cfg.renorm, terms=terms)
    return fw, bw, flips


def compare_full(cfg, inp, backward, gather=False, degenerate=False):
    """Full comparison on a layer small enough for the oracle to run whole.
    degenerate: the routed weight gradients are compared expert by expert
    (assert_close_per_expert), for routings that leave few rows per expert."""
    g = run_gpu(cfg, inp, backward, gather=gather)
    oi = oracle_inputs(cfg, inp)
    fw, bw = oracle_run(cfg, oi, backward)
    same = check_routing(cfg, g["logits"], g["idx"], fw)
    fw, bw, flips = oracle_on_gpu_routing(cfg, oi, g["idx"], backward, fw, bw)
    print(f"[compare] {cfg.name}: tokens on a near-tie choice other than the oracle's: {flips} of {cfg.T}",
          flush=True)
    assert_close(g["y"], fw["y"], cfg.dtype, "y")
    assert np.array_equal(g["counts"].sum(), cfg.T * cfg.k)
    if backward:
        assert_close(g["dx"], bw["dx"], cfg.dtype, "dx")
        if degenerate and cfg.dtype != "f32":
            assert_close_per_expert(g["d_w_gateup"], bw["d_w_gateup"], "dW_gateup")
            assert_close_per_expert(g["d_w_down"], bw["d_w_down"], "dW_down")
        else:
            assert_close(g["d_w_gateup"], bw["d_w_gateup"], cfg.dtype, "dW_gateup")
            assert_close(g["d_w_down"], bw["d_w_down"], cfg.dtype, "dW_down")
        if degenerate and cfg.dtype != "f32":
            # a single token makes the router and shared gradients rank one
            assert_close_large(g["d_w_router"], bw["d_w_router"], "dW_router")
            if cfg.F_shared:
                assert_close_large(g["d_s_gateup"], bw["d_s_gateup"], "dS_gateup")
                assert_close_large(g["d_s_down"], bw["d_s_down"], "dS_down")
        else:
            # the router weight gradient is fp32 in every layer
            assert_close(g["d_w_router"], bw["d_w_router"], "f32" if cfg.dtype == "f32" else "bf16", "dW_router")
            if cfg.F_shared:
                assert_close(g["d_s_gateup"], bw["d_s_gateup"], cfg.dtype, "dS_gateup")
                assert_close(g["d_s_down"], bw["d_s_down"], cfg.dtype, "dS_down")
    return g, fw, bw, same
