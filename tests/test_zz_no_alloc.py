"""moe_forward_noalloc: moe_forward on a scratch array the library holds on
each GPU (no workspace argument; the call allocates nothing).  Through the C
ABI, against moe_forward on a caller workspace: every output and saved tensor
bit for bit, on consecutive calls, the second with fewer tokens (the array
keeps the first call's contents), and the outputs within the oracle's bounds."""
import dataclasses

import numpy as np
import pytest
import torch

from grouped_gemm_expert_amd import inputs
from tests import harness as hz

pytestmark = pytest.mark.gpu

SAVED = ["logits", "topk_idx", "topk_w", "counts", "offsets", "row_map", "pos", "h", "a"]


def _one(w, seed, oracle_check):
    from grouped_gemm_expert_amd import ops
    hz.say(f"noalloc {inputs.describe(w)}")
    cfg = ops.config_from_workload(w)
    need = ops.moe_forward_noalloc_bytes(cfg)
    assert need <= ops.NOALLOC_SCRATCH_BYTES, need
    if oracle_check:
        dc = inputs.make_inputs(w, seed=seed, with_dy=False)
        d = hz.to_device(dc)
    else:                       # large weights: drawn on the GPU
        d = inputs.make_inputs(w, seed=seed, with_dy=False, device="cuda")
    outs = []
    for use_scratch in (False, True):
        saved = ops.alloc_saved(cfg)
        if d["logits"] is not None:
            saved["logits"].copy_(d["logits"])
        y = torch.full((w.T, w.H), float("nan"), device="cuda")
        aux = torch.full((1,), float("nan"), device="cuda")
        if use_scratch:
            ops.moe_forward_noalloc(cfg, d["x"], d["Wr"], d["bias"], d["w1"], d["w2"], y, aux,
                                    saved)
        else:
            ops.moe_forward(cfg, d["x"], d["Wr"], d["bias"], d["w1"], d["w2"], y, aux, saved,
                            ops.workspace(cfg, "fwd"))
        outs.append((y, aux, saved))
    torch.cuda.synchronize()
    (y0, a0, s0), (y1, a1, s1) = outs
    assert torch.equal(y0, y1) and torch.equal(a0, a1)
    for k in SAVED + (["h_lo", "a_lo"] if w.precision == "split" else []):
        assert torch.equal(s0[k], s1[k]), k
    if oracle_check:
        l64, r = hz.oracle_route(w, dc)
        assert np.array_equal(s1["topk_idx"].cpu().numpy(), r["idx"])
        ref = hz.oracle_forward_backward(w, dc, r, l64, backward=False)
        hz.assert_close(f"noalloc {w.name} y", y1.cpu().numpy(), ref["y"], hz.FWD_TOL)


@pytest.mark.parametrize("base,Ts", [("mid_sigmoid", (500, 200)), ("mid_split", (600, 150))])
def test_noalloc_matches_moe_forward_on_two_calls(base, Ts):
    for i, T in enumerate(Ts):
        _one(dataclasses.replace(inputs.WORKLOADS[base], T=T), seed=10 + i, oracle_check=True)


def test_noalloc_decode_sized_batches_at_deepseek_shapes():
    """The DeepSeek-V3 layer shapes (H=7168, I=2048, sigmoid + bias, groups)
    with 32 experts, at decode-sized batches: 160 tokens, then 48."""
    base = dataclasses.replace(inputs.WORKLOADS["deepseek_v3"], E=32, n_groups=8, topk_groups=4)
    for i, T in enumerate((160, 48)):
        _one(dataclasses.replace(base, T=T), seed=20 + i, oracle_check=False)


def test_noalloc_rejects_configs_past_its_scratch():
    from grouped_gemm_expert_amd import ops
    w = dataclasses.replace(inputs.WORKLOADS["deepseek_v3"], T=4096)
    cfg = ops.config_from_workload(w)
    assert ops.moe_forward_noalloc_bytes(cfg) > ops.NOALLOC_SCRATCH_BYTES
    saved = ops.alloc_saved(ops.config_from_workload(dataclasses.replace(w, T=1)))
    t = torch.empty((16,), device="cuda")
    with pytest.raises(ops.MoeError, match="workspace too small"):
        # rejected on the host from the config alone: no pointer is read
        ops.moe_forward_noalloc(cfg, t, None, None, t, t, t, t, saved)
