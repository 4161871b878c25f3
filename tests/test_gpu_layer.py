"""The autograd binding (grouped_gemm_expert_amd.layer.MoEFunction): y and aux
of its forward and the .grad of x, Wr, w1 and w2 that torch.autograd leaves
after loss = <y, dy> + aux, against the oracle's forward and backward on the
same seeded inputs.  The grads arrive in each input's dtype (bf16 for x, w1,
w2), so the bounds hold after that rounding too."""
import numpy as np
import pytest
import torch

import oracle
from grouped_gemm_expert_amd import inputs
from tests import harness as hz

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name", ["tiny", "mid_sigmoid", "mid_softmax"])
def test_moe_function_grads_against_oracle(name):
    from grouped_gemm_expert_amd import ops
    from grouped_gemm_expert_amd.layer import MoEFunction
    w = inputs.WORKLOADS[name]
    hz.say(f"layer {inputs.describe(w)}")
    dc = inputs.make_inputs(w, seed=0)
    assert dc["Wr"] is not None
    d = hz.to_device(dc)
    x = d["x"].clone().requires_grad_()
    Wr = d["Wr"].clone().requires_grad_()
    w1 = d["w1"].clone().requires_grad_()
    w2 = d["w2"].clone().requires_grad_()
    cfg = ops.config_from_workload(w)
    y, aux = MoEFunction.apply(x, Wr, d["bias"], w1, w2, cfg)
    loss = (y * d["dy"].float()).sum() + aux.sum()
    loss.backward()
    torch.cuda.synchronize()

    l64, r = hz.oracle_route(w, dc)
    ref = hz.oracle_forward_backward(w, dc, r, l64, d_aux=1.0)
    hz.assert_close(f"layer {name} y", y.detach().cpu().numpy(), ref["y"], hz.FWD_TOL)
    assert abs(float(aux.detach().cpu()) - r["aux"]) <= 1e-4 * abs(r["aux"]) + 1e-9
    for got, key in ((x.grad, "dx"), (Wr.grad, "dWr"), (w1.grad, "dW1"), (w2.grad, "dW2")):
        assert got is not None and got.dtype == {"dx": x, "dWr": Wr, "dW1": w1, "dW2": w2}[key].dtype
        hz.assert_close(f"layer {name} {key}", got.float().cpu().numpy(), ref[key], hz.GRAD_TOL)
