"""Router training terms on the GPU against the oracle: the balance losses and
the z-loss inside moe_backward, and the proportional bias update."""
import numpy as np
import pytest
import torch

import synth
from oracle import moe_oracle as O
from tests.gpu_util import assert_close, dev, rel_l2

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import mixture_experts_layer_18_amd as M
    from tests import layer_runner as R

TERMS = dict(aux_coeff=0.5, seq_aux_coeff=0.3, z_coeff=0.1)


def _check_losses(g, bw):
    want = np.array([bw["router_terms"]["aux"], bw["router_terms"]["seq_aux"], bw["router_terms"]["z"]])
    got = g["losses"].astype(np.float64)
    assert np.all(np.abs(got - want) <= 1e-6 * np.abs(want) + 1e-12), (got, want)


@pytest.mark.parametrize("score", ["softmax", "sigmoid"])
def test_router_terms_fp32(score):
    """fp32 layer: the terms' gradients reach d_w_router and dx at the fp32 bar."""
    cfg = synth.CONFIG_BY_NAME["tiny_fp32"].replace(score=score, backward=True,
                                                   bias="uniform" if score == "sigmoid" else None,
                                                   renorm=score == "sigmoid")
    terms = dict(TERMS, seq_len=64)
    print(f"[terms] fp32 {score}", flush=True)
    inp = synth.make_inputs(cfg)
    g = R.run_gpu(cfg, inp, backward=True, terms=terms)
    fw, bw = R.oracle_run(cfg, R.oracle_inputs(cfg, inp), True, terms=terms)
    same = R.check_routing(cfg, g["logits"], g["idx"], fw)
    assert same.all()
    _check_losses(g, bw)
    assert_close(g["d_w_router"], bw["d_w_router"], "f32", "dW_router")
    assert_close(g["dx"], bw["dx"], "f32", "dx")
    assert_close(g["d_w_gateup"], bw["d_w_gateup"], "f32", "dW_gateup")


def test_router_terms_bf16_small():
    cfg = synth.CONFIG_BY_NAME["moe7b_bf16"].replace(name="small_terms", T=1000, d=256, E=16, k=4, f=192,
                                                     n_shared=1, f_shared=128)
    terms = dict(aux_coeff=1e-2, seq_aux_coeff=1e-2, z_coeff=1e-3, seq_len=125)
    print("[terms] bf16 small", flush=True)
    inp = synth.make_inputs(cfg)
    g = R.run_gpu(cfg, inp, backward=True, terms=terms)
    fw, bw = R.oracle_run(cfg, R.oracle_inputs(cfg, inp), True, terms=terms)
    same = R.check_routing(cfg, g["logits"], g["idx"], fw)
    assert same.all()
    _check_losses(g, bw)
    assert_close(g["d_w_router"], bw["d_w_router"], "bf16", "dW_router")
    assert_close(g["dx"], bw["dx"], "bf16", "dx")


def test_router_terms_off_changes_nothing():
    """Terms with every coefficient 0 (and no loss output) leave every gradient
    bit-identical; enabled terms change only the router gradient and dx."""
    cfg = synth.CONFIG_BY_NAME["moe7b_bf16"].replace(name="small_terms", T=512, d=256, E=16, k=4, f=128,
                                                     n_shared=0, f_shared=0)
    inp = synth.make_inputs(cfg)
    base = R.run_gpu(cfg, inp, backward=True)
    off = R.run_gpu(cfg, inp, backward=True, terms=dict(seq_len=128))
    on = R.run_gpu(cfg, inp, backward=True, terms=dict(TERMS, seq_len=128))
    for n in ("d_w_router", "dx", "d_w_gateup", "d_w_down", "y"):
        assert np.array_equal(base[n], off[n]), n
    for n in ("d_w_gateup", "d_w_down", "y"):
        assert np.array_equal(base[n], on[n]), n
    assert not np.array_equal(base["d_w_router"], on["d_w_router"])


@pytest.mark.parametrize("rate", [1e-3, 0.01])
def test_bias_update_matches_oracle(rate):
    T, E, k = 4096, 64, 6
    g = np.random.default_rng(int(rate * 1e4))
    bias = g.uniform(-0.1, 0.1, E).astype(np.float32)
    counts = g.multinomial(T * k, np.full(E, 1.0 / E)).astype(np.int32)
    counts[5] = 0
    desc = M.make_desc(T, 256, E, k, 128, 0, 0, "sigmoid", True, "bf16")
    b = dev(bias)
    M.moe_bias_update(desc, dev(counts), rate, b)
    torch.cuda.synchronize()
    want = O.bias_update(bias, counts, T, k, rate)
    assert np.array_equal(b.cpu().numpy(), want)


def test_router_terms_full_size_values():
    """The 16k-token layer with the training settings of the Apex-3 command
    (per-sequence balance loss 1e-3 over 4096-token sequences) plus the
    Handbook's balance loss 1e-3 and a z-loss: the loss values on every token."""
    cfg = synth.CONFIG_BY_NAME["moe7b_bf16"]
    terms = dict(aux_coeff=1e-3, seq_aux_coeff=1e-3, z_coeff=1e-3, seq_len=4096)
    print("[terms] full size", flush=True)
    inp = synth.make_inputs(cfg, with_dy=True)
    g = R.run_gpu(cfg, inp, backward=True, terms=terms)
    xf = synth.as_f64(inp["x"], cfg.dtype)
    logits = O.router_logits(xf, inp["w_router"])
    scores = O.router_scores(logits, cfg.score)
    keys = O.selection_keys(logits, scores, inp["bias"], cfg.score)
    idx, margin = O.select_topk(keys, cfg.k)
    counts = np.bincount(idx.reshape(-1), minlength=cfg.E)
    vals, _ = O.router_terms(logits, idx, counts, cfg.k, cfg.score, terms)
    want = np.array([vals["aux"], vals["seq_aux"], vals["z"]])
    got = g["losses"].astype(np.float64)
    # a near-tie may flip one token's expert between the two sides: the load
    # shares move by 1/(T k) per flip, far below this bound
    assert np.all(np.abs(got - want) <= 1e-5 * np.abs(want)), (got, want)
    assert rel_l2(g["logits"], logits) <= 1e-5
