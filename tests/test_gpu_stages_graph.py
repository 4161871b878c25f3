"""The two-stage entry points (stage 1 owns w1, stage 2 owns w2; the backward
runs stage 2 first) give bit-identical results to moe_forward / moe_backward,
and a HIP graph that captures the whole forward + backward replays to the
eager results, replay after replay, with eager work of the program in between.
(Page "MegaMoE", "Design: two stages + weight modules" and "Example 2": the
layer is split into two weight-owning stages and is captured into a graph.)"""
import pytest
import torch

from grouped_gemm_expert_amd import inputs, ops
from tests import harness as hz

pytestmark = pytest.mark.gpu

NAMES = ["tiny", "mid_sigmoid", "mid_skewed", "mid_split"]
OUTS = ["y", "aux", "dx", "dlogits", "dWr", "dW1", "dW2"]


def _alloc(w, d, cfg, dev):
    saved = ops.alloc_saved(cfg, dev)
    if d["logits"] is not None:
        saved["logits"].copy_(d["logits"])
    t = dict(
        saved=saved,
        y=torch.empty((w.T, w.H), dtype=torch.float32, device=dev),
        aux=torch.empty((1,), dtype=torch.float32, device=dev),
        dx=torch.empty((w.T, w.H), dtype=torch.float32, device=dev),
        dlogits=torch.empty((w.T, w.E), dtype=torch.float32, device=dev),
        dWr=torch.empty((w.E, w.H), dtype=torch.float32, device=dev) if d["Wr"] is not None else None,
        dW1=torch.empty((w.E, 2 * w.I, w.H), dtype=torch.float32, device=dev),
        dW2=torch.empty((w.E, w.H, w.I), dtype=torch.float32, device=dev),
        d_aux=torch.ones((1,), dtype=torch.float32, device=dev),
        wsf=ops.workspace(cfg, "fwd", dev),
        wsb=ops.workspace(cfg, "bwd", dev),
    )
    return t


def _one_call(cfg, d, t):
    ops.moe_forward(cfg, d["x"], d["Wr"], d["bias"], d["w1"], d["w2"], t["y"], t["aux"],
                    t["saved"], t["wsf"])
    ops.moe_backward(cfg, t["saved"], d["x"], d["Wr"], d["w1"], d["w2"], d["dy"], t["d_aux"],
                     t["dx"], t["dlogits"], t["dWr"], t["dW1"], t["dW2"], t["wsb"])


def _staged(cfg, d, t):
    ops.moe_stage1_forward(cfg, d["x"], d["Wr"], d["bias"], d["w1"], t["aux"], t["saved"], t["wsf"])
    ops.moe_stage2_forward(cfg, d["w2"], t["saved"], t["y"], t["wsf"])
    ops.moe_stage2_backward(cfg, t["saved"], d["w2"], d["dy"], t["dW2"], t["wsb"])
    ops.moe_stage1_backward(cfg, t["saved"], d["x"], d["Wr"], d["w1"], t["d_aux"], t["dx"],
                            t["dlogits"], t["dWr"], t["dW1"], t["wsb"])


def _same(name, a, b):
    if a is None:
        assert b is None
        return
    assert torch.equal(a, b), f"{name} differs"


@pytest.mark.parametrize("name", NAMES)
def test_two_stages_equal_one_call(name):
    w = inputs.WORKLOADS[name]
    hz.say(f"stages {inputs.describe(w)}")
    d = hz.to_device(inputs.make_inputs(w))
    cfg = ops.config_from_workload(w)
    a = _alloc(w, d, cfg, "cuda")
    b = _alloc(w, d, cfg, "cuda")
    _one_call(cfg, d, a)
    _staged(cfg, d, b)
    torch.cuda.synchronize()
    for k in OUTS:
        _same(k, a[k], b[k])
    for k in ("topk_idx", "topk_w", "counts", "offsets", "row_map", "pos", "h", "a"):
        _same(k, a["saved"][k], b["saved"][k])


def test_graph_capture_replays_to_eager():
    w = inputs.WORKLOADS["mid_sigmoid"]
    hz.say(f"graph {inputs.describe(w)}")
    d = hz.to_device(inputs.make_inputs(w))
    cfg = ops.config_from_workload(w)
    ref = _alloc(w, d, cfg, "cuda")
    _one_call(cfg, d, ref)
    torch.cuda.synchronize()

    t = _alloc(w, d, cfg, "cuda")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):          # warm-up off the default stream before capture
        _staged(cfg, d, t)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        _staged(cfg, d, t)
    torch.cuda.synchronize()

    other = _alloc(w, d, cfg, "cuda")
    for rep in range(3):
        for k in OUTS:                       # poison every output before the replay
            if t[k] is not None:
                t[k].fill_(float("nan"))
        g.replay()
        _one_call(cfg, d, other)             # eager work of the program between replays
        torch.cuda.synchronize()
        hz.say(f"graph replay {rep}")
        for k in OUTS:
            _same(f"replay {rep} {k}", t[k], ref[k])
            _same(f"eager {rep} {k}", other[k], ref[k])
