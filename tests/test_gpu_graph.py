"""The layer captured in a HIP graph: moe_forward + moe_backward recorded
once on a capture stream and replayed with new token rows and upstream
gradients copied into the graph's input buffers.  Every kernel of the path
is deterministic, so each replay must equal an eager run on the same inputs
bit for bit (outputs, saved routing, input and weight gradients).  The
replays are separated by eager work and synchronisations, and each is checked
against its own eager result."""
import numpy as np
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import mixture_experts_layer_18_amd as M
    from tests import layer_runner as R
    from tests.gpu_util import dev

# gathered token rows, two shared experts, a ragged token count
CFG = synth.CONFIG_BY_NAME["moe7b_bf16"].replace(name="graph_bf16", T=1000, d=256, E=16, k=4, f=256,
                                                 n_shared=2, f_shared=128)
OUTS = ("y", "dx")


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


@pytest.mark.parametrize("fp8", [False, True], ids=["bf16", "fp8"])
def test_layer_graph_replays_equal_eager(fp8):
    print(f"[graph] capture and replay fp8={fp8}", flush=True)
    inp = synth.make_inputs(CFG, with_dy=True)
    desc = M.desc_from_config(CFG)
    w = R.upload_layer(CFG, inp)
    x = dev(inp["x"])
    dy = dev(inp["dy"])
    w8 = None
    if fp8:
        w8 = M.alloc_fp8_weights(desc, backward=True)
        M.moe_fp8_weights_quantize(desc, w, w8, True, True)
    saved = M.alloc_saved(desc, gather=True, training=True)
    grads = M.alloc_grads(desc)
    y, dx = torch.empty_like(x), torch.empty_like(x)
    wsf = M.alloc_workspace(desc, "forward_fp8" if fp8 else "forward")
    wsb = M.alloc_workspace(desc, "backward_fp8" if fp8 else "backward")

    def step(stream):
        if fp8:
            M.moe_forward_fp8(desc, w, w8, x, y, saved, wsf, stream)
            M.moe_backward_fp8(desc, w, w8, x, saved, dy, dx, grads, wsb, stream)
        else:
            M.moe_forward(desc, w, x, y, saved, wsf, stream)
            M.moe_backward(desc, w, x, saved, dy, dx, grads, wsb, stream)

    def snapshot():
        torch.cuda.synchronize()
        out = {"y": y.clone(), "dx": dx.clone()}
        for n in ("idx", "gate", "counts", "offsets", "pos", "tok", "preact", "h"):
            out[n] = saved[n].clone()
        for n, t in grads.items():
            if t is not None:
                out[n] = t.clone()
        return out

    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        step(cap)  # warm-up on the capture stream (library set-up happens outside the graph)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=cap):
        step(cap)
    torch.cuda.synchronize()

    gen = np.random.default_rng(7)
    for rep in range(3):
        # new inputs, copied into the graph's buffers
        xn = torch.from_numpy(gen.standard_normal(x.shape).astype(np.float32)).to(torch.bfloat16).cuda()
        dyn = torch.from_numpy(gen.standard_normal(dy.shape).astype(np.float32)).to(torch.bfloat16).cuda()
        x.copy_(xn)
        dy.copy_(dyn)
        torch.cuda.synchronize()
        step(torch.cuda.current_stream())          # eager on the same inputs
        want = snapshot()
        y.zero_()
        dx.zero_()
        for t in grads.values():
            if t is not None:
                t.zero_()
        torch.cuda.synchronize()
        g.replay()
        got = snapshot()
        for n, t in want.items():
            assert torch.equal(_bits(got[n]) if got[n].is_floating_point() else got[n],
                               _bits(t) if t.is_floating_point() else t), f"replay {rep}: {n} differs from eager"
        print(f"[graph] replay {rep} equals eager", flush=True)
