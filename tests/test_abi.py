"""The C ABI library loads without a GPU, exports every entry point that
include/moe.h declares, and validates configurations on the host."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^[ \t]*(?:const\s+)?[A-Za-z_][\w]*\s*\**\s*(moe_\w+)\s*\(", src, flags=re.M)
    return sorted(set(names))


def test_header_declares_the_entry_points():
    names = _declared()
    for n in ("moe_router", "moe_permute", "moe_grouped_gemm", "moe_swiglu", "moe_combine",
              "moe_forward", "moe_backward"):
        assert n in names


def test_library_exports_every_declared_symbol():
    from grouped_gemm_expert_amd import ops
    lib = ctypes.CDLL(ops.lib_path())
    missing = [n for n in _declared() if not hasattr(lib, n)]
    assert not missing, missing
    assert set(ops.SYMBOLS) == set(_declared())


def test_version_string():
    from grouped_gemm_expert_amd import ops
    assert "gfx950" in ops.moe_version()


BAD = [
    (dict(k=9, E=8), 2),                      # k > E
    (dict(H=100), 2),                         # H not a multiple of 64
    (dict(I=96), 2),                          # I not a multiple of 64
    (dict(E=2048, k=2), 2),                   # too many experts
    (dict(k=40, E=64), 2),                    # k above 32
    (dict(E=16, n_groups=3), 2),              # groups do not divide E
    (dict(E=16, n_groups=4, topk_groups=5), 2),
    (dict(E=16, n_groups=4, topk_groups=1, k=5), 2),  # k above the experts of kept groups
    (dict(score=7), 1),
    (dict(T=-1), 1),
    (dict(H=0), 1),
    (dict(route=7), 1),                       # unknown route mode
]


@pytest.mark.parametrize("override,status", BAD)
def test_config_validation(override, status):
    from grouped_gemm_expert_amd import ops
    kw = dict(T=16, H=128, I=64, E=8, k=2, n_groups=1, topk_groups=1, score=0)
    kw.update(override)
    cfg = ops.config(**kw)
    assert ops.moe_check_config(cfg) == status


def test_valid_configs_and_workspace_sizes():
    from grouped_gemm_expert_amd import inputs, ops
    for name, w in inputs.WORKLOADS.items():
        cfg = ops.config_from_workload(w)
        assert ops.moe_check_config(cfg) == 0, name
        f, b = ops.moe_workspace_size(cfg)
        # the forward workspace holds at least the fp32 expert outputs [M, H]
        assert f >= w.M * w.H * 4 and b >= w.M * w.H * 4
    cfg = ops.config(T=0, H=128, I=64, E=8, k=2)
    assert ops.moe_check_config(cfg) == 0
