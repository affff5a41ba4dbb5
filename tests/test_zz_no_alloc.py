"""moe_forward_no_workspace (the forward whose scratch lives in the library's
own device array) against moe_forward with a caller workspace: the same
kernels, so every output and saved buffer must match bit for bit.  Two calls
in a row on one GPU, the second on a smaller layer, so the second call runs
on the scratch the first one left behind."""
import numpy as np
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import mixture_experts_layer_18_amd as M
    from tests import layer_runner as R
    from tests.gpu_util import dev

FIELDS = ("logits", "idx", "gate", "counts", "offsets", "pos", "src", "tok", "preact", "h", "y_perm",
          "s_preact", "s_h")


def _bits(t):
    return t.contiguous().view(torch.uint8).cpu().numpy() if t is not None else None


def _run(cfg, inp, no_workspace, training, gather):
    desc = M.desc_from_config(cfg)
    w = R.upload_layer(cfg, inp)
    x = dev(inp["x"])
    y = torch.full_like(x, float("nan"))
    saved = M.alloc_saved(desc, training=training, gather=gather)
    for t in saved.values():
        if t is not None and t.is_floating_point():
            t.fill_(float("nan"))
        elif t is not None:
            t.fill_(-7)
    if no_workspace:
        M.moe_forward_no_workspace(desc, w, x, y, saved)
    else:
        M.moe_forward(desc, w, x, y, saved, M.alloc_workspace(desc, "forward"))
    torch.cuda.synchronize()
    return y, saved


def _compare(cfg, training, gather):
    inp = synth.make_inputs(cfg)
    y0, s0 = _run(cfg, inp, False, training, gather)
    y1, s1 = _run(cfg, inp, True, training, gather)
    assert np.array_equal(_bits(y0), _bits(y1)), f"{cfg.name}: y differs"
    for n in FIELDS:
        a, b = s0.get(n), s1.get(n)
        assert (a is None) == (b is None), n
        if a is not None:
            assert np.array_equal(_bits(a), _bits(b)), f"{cfg.name}: saved {n} differs"
    counts = s1["counts"].cpu().numpy()
    assert counts.sum() == cfg.T * cfg.k


@pytest.mark.parametrize("training", [True, False], ids=["training", "inference"])
def test_no_workspace_forward_two_calls(training):
    big = synth.CONFIG_BY_NAME["finegrained_bf16"]
    small = big.replace(name="finegrained_small", T=1000)
    print(f"[no-ws] {big.name} then {small.name}, training={training}", flush=True)
    _compare(big, training, gather=True)
    _compare(small, training, gather=True)


def test_no_workspace_forward_fp32_and_permuted_copy():
    tiny = synth.CONFIG_BY_NAME["tiny_fp32"]
    small = synth.CONFIG_BY_NAME["moe7b_bf16"].replace(name="small_bf16", T=600, d=256, E=16, k=4, f=256,
                                                        n_shared=2, f_shared=128)
    print("[no-ws] tiny fp32, then a small bf16 layer with a permuted token copy", flush=True)
    _compare(tiny, True, gather=False)
    _compare(small, True, gather=False)
