"""Whole-layer GPU parity (moe_forward / moe_backward) against the oracle."""
import numpy as np
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from tests import layer_runner as R


def test_forward_tiny_fp32():
    cfg = synth.CONFIG_BY_NAME["tiny_fp32"]
    print(f"[layer] {cfg.name} fwd", flush=True)
    R.compare_full(cfg, synth.make_inputs(cfg), backward=False)


def test_backward_tiny_fp32():
    cfg = synth.CONFIG_BY_NAME["tiny_fp32"].replace(backward=True)
    print(f"[layer] {cfg.name} fwd+bwd", flush=True)
    R.compare_full(cfg, synth.make_inputs(cfg), backward=True)


@pytest.mark.parametrize("score,renorm", [("softmax", True), ("sigmoid", True)])
def test_backward_fp32_other_routers(score, renorm):
    cfg = synth.CONFIG_BY_NAME["tiny_fp32"].replace(score=score, renorm=renorm, backward=True, n_shared=1,
                                                   f_shared=128, T=200, bias="uniform" if score == "sigmoid"
                                                   else None)
    print(f"[layer] fp32 {score} renorm={renorm} shared", flush=True)
    R.compare_full(cfg, synth.make_inputs(cfg), backward=True)


def test_forward_finegrained_bf16():
    cfg = synth.CONFIG_BY_NAME["finegrained_bf16"]
    print(f"[layer] {cfg.name} fwd", flush=True)
    R.compare_full(cfg, synth.make_inputs(cfg), backward=False)


SMALL_BF16 = synth.CONFIG_BY_NAME["moe7b_bf16"].replace(name="small_bf16", T=1000, d=256, E=16, k=4, f=192,
                                                         n_shared=2, f_shared=128)


def test_backward_small_bf16():
    print("[layer] small_bf16 fwd+bwd", flush=True)
    R.compare_full(SMALL_BF16, synth.make_inputs(SMALL_BF16), backward=True)


# 64 experts x 4 x 4 weight-gradient tiles = 1024: the routed down weight
# gradient runs on the persistent kernel, so each shared weight gradient
# (16 and 8 output tiles, one round's last partial) runs in the launch of its
# routed counterpart; 2000 tokens (a ragged last k-step of the shared
# products) over groups of about 125 rows
PAIRED_BF16 = synth.CONFIG_BY_NAME["moe7b_bf16"].replace(name="paired_bf16", T=2000, d=1024, E=64, k=4, f=1024,
                                                          n_shared=1, f_shared=512)
# widths that leave partial 256-column tiles in the down products and their
# weight gradients (f = 3.5 tiles, the shared width 2.5); 4000 tokens, so that
# every expert's weight gradient sums enough rows for the bf16 bar (at 2000
# tokens the smallest experts had 18 rows, and one bf16 step of their largest
# elements reached 5.02e-2 of the RMS)
PAIRED_RAGGED = PAIRED_BF16.replace(name="paired_ragged", T=4000, f=896, f_shared=640)


@pytest.mark.parametrize("cfg", [PAIRED_BF16, PAIRED_RAGGED], ids=["tile-multiples", "ragged-widths"])
@pytest.mark.parametrize("gather", [False, True], ids=["permuted-copy", "gathered"])
def test_backward_paired_shared_weight_gradients(gather, cfg):
    import mixture_experts_layer_18_amd as M
    print(f"[layer] paired shared weight gradients {cfg.name} gather={gather}", flush=True)
    M.stage_timing(True)
    try:
        R.compare_full(cfg, synth.make_inputs(cfg), backward=True, gather=gather)
        torch.cuda.synchronize()
        st = M.stage_times()
    finally:
        M.stage_timing(False)
    # the shared weight gradients ran inside the routed launches
    assert st["down_wgrad"][1] >= 1 and st["gate_up_wgrad"][1] >= 1
    assert st["shared_down_wgrad"][1] == 0 and st["shared_gate_up_wgrad"][1] == 0


def test_backward_small_bf16_skewed():
    cfg = SMALL_BF16.replace(name="small_skew", bias="zipf")
    print("[layer] small skew fwd+bwd", flush=True)
    inp = synth.make_inputs(cfg, skew_alpha=0.3)
    g, fw, bw, same = R.compare_full(cfg, inp, backward=True)
    assert (g["counts"] == 0).sum() >= 4          # the pinned-down experts stay empty
    empty = np.where(g["counts"] == 0)[0]
    assert np.all(g["d_w_gateup"][empty] == 0) and np.all(g["d_w_down"][empty] == 0)


def test_forward_backward_deterministic():
    cfg = SMALL_BF16
    inp = synth.make_inputs(cfg)
    a = R.run_gpu(cfg, inp, backward=True)
    b = R.run_gpu(cfg, inp, backward=True)
    for n in a:
        assert np.array_equal(a[n], b[n], equal_nan=True), n


def test_zero_tokens_is_a_noop():
    cfg = SMALL_BF16.replace(T=0)
    inp = synth.make_inputs(cfg)
    g = R.run_gpu(cfg, inp, backward=True)
    assert np.all(g["counts"] == 0) and np.all(g["offsets"] == 0)
    assert np.all(g["d_w_gateup"] == 0) and np.all(g["d_w_router"] == 0)


# ----------------------------------------------------------------------------- limits and degenerate routings
@pytest.mark.parametrize("gather", [False, True], ids=["permuted-copy", "gathered"])
def test_maximum_experts_and_top_k(gather):
    """E = 256 experts (the most the router and the grouped GEMMs take) with
    top-16: 256 small groups, some of them empty."""
    cfg = SMALL_BF16.replace(name="max_ek", T=700, d=256, E=256, k=16, f=128, n_shared=1, f_shared=128)
    print(f"[layer] E=256 k=16 gather={gather}", flush=True)
    g, fw, bw, same = R.compare_full(cfg, synth.make_inputs(cfg), backward=True, gather=gather, degenerate=True)
    assert g["counts"].sum() == cfg.T * cfg.k


def test_single_token():
    cfg = SMALL_BF16.replace(name="one_token", T=1)
    print("[layer] one token", flush=True)
    R.compare_full(cfg, synth.make_inputs(cfg), backward=True, degenerate=True)


@pytest.mark.parametrize("gather", [False, True], ids=["permuted-copy", "gathered"])
def test_every_token_to_one_expert(gather):
    """A selection bias far above every score sends all tokens to expert 2
    (top-1): one group holds every row, the others are empty, and the gates
    renormalise to exactly 1."""
    cfg = SMALL_BF16.replace(name="one_expert", T=900, d=256, E=8, k=1, f=256, n_shared=0, f_shared=0)
    inp = synth.make_inputs(cfg)
    inp["bias"] = np.zeros(cfg.E, np.float32)
    inp["bias"][2] = 10.0
    print(f"[layer] every token to one expert gather={gather}", flush=True)
    g, fw, bw, same = R.compare_full(cfg, inp, backward=True, gather=gather, degenerate=True)
    assert g["counts"][2] == cfg.T and g["counts"].sum() == cfg.T
    assert np.all(g["gate"] == 1.0)
    empty = [e for e in range(cfg.E) if e != 2]
    assert np.all(g["d_w_gateup"][empty] == 0) and np.all(g["d_w_down"][empty] == 0)


def test_forward_bf16_width_not_multiple_of_128():
    """d = 192: the bf16 router product falls back to the fp32 matrix cores
    (the split-weight kernel steps 128 columns at a time)."""
    cfg = SMALL_BF16.replace(name="d192", T=300, d=192)
    print("[layer] bf16 d=192 fwd", flush=True)
    R.compare_full(cfg, synth.make_inputs(cfg), backward=False)


def test_backward_bf16_odd_expert_count():
    """E = 7: the bf16 router weight gradient falls back to the fp32 matrix
    cores (the split kernel loads expert pairs)."""
    cfg = SMALL_BF16.replace(name="e7", T=300, E=7, k=2, f=128, n_shared=0, f_shared=0)
    print("[layer] bf16 E=7 fwd+bwd", flush=True)
    R.compare_full(cfg, synth.make_inputs(cfg), backward=True)


@pytest.mark.parametrize("gather", [False, True], ids=["permuted-copy", "gathered"])
def test_saved_buffers_in_one_allocation(gather):
    """The saved buffers carved from one allocation (moe_saved_carve) give the
    same bits as separate allocations."""
    import mixture_experts_layer_18_amd as M
    cfg = SMALL_BF16.replace(name="carved", d=256, f=256)
    inp = synth.make_inputs(cfg)
    desc = M.desc_from_config(cfg)
    w = R.upload_layer(cfg, inp)
    x = R.dev(inp["x"])
    dy = R.dev(inp["dy"])
    outs = []
    for saved in (M.alloc_saved(desc, gather=gather), M.alloc_saved_one_buffer(desc, gather=gather)):
        y = torch.empty_like(x)
        M.moe_forward(desc, w, x, y, saved, M.alloc_workspace(desc, "forward"))
        grads = M.alloc_grads(desc)
        dx = torch.empty_like(x)
        M.moe_backward(desc, w, x, saved, dy, dx, grads, M.alloc_workspace(desc, "backward"))
        torch.cuda.synchronize()
        outs.append([y, dx] + [g for g in grads.values() if g is not None])
    for a, b in zip(*outs):
        assert torch.equal(a.view(torch.uint8), b.view(torch.uint8))
