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


def test_saved_sizes():
    from grouped_gemm_expert_amd import ops
    cfg = ops.config(T=100, H=128, I=64, E=8, k=3)
    s = ops.moe_saved_sizes(cfg)
    M = 300
    assert s == {"logits": 100 * 8 * 4, "topk_idx": M * 4, "topk_w": M * 4, "counts": 8 * 4,
                 "offsets": 9 * 4, "row_map": M * 4, "pos": M * 4, "h": M * 128 * 2,
                 "a": M * 64 * 2, "h_lo": 0, "a_lo": 0}
    assert ops.moe_check_config(ops.config(T=100, H=128, I=64, E=8, k=9)) == 2


def test_size_limits_stated_in_the_header():
    """The header's Supported line: at H = 7168 and I = 2048 (W = max(H, 2I) =
    7168), T*k <= 299593 and T <= 299465; one past either is unsupported."""
    from grouped_gemm_expert_amd import ops
    kw = dict(H=7168, I=2048, E=256, k=1)
    assert ops.moe_check_config(ops.config(T=299465, **kw)) == 0
    assert ops.moe_check_config(ops.config(T=299466, **kw)) == 2     # W * (T + 128)
    assert ops.moe_check_config(ops.config(T=149796, **dict(kw, k=2))) == 0   # T*k = 299592
    assert ops.moe_check_config(ops.config(T=149797, **dict(kw, k=2))) == 2   # T*k = 299594
    # 2 * I * H < 2^31: one expert's w1
    assert ops.moe_check_config(ops.config(T=16, H=65536, I=16384, E=8, k=2)) == 2


def _fake(n=1):
    """Distinct 256-byte-aligned stand-ins for device pointers: the host layer
    checks them for null and alignment and returns before anything is
    launched, so they are never dereferenced."""
    return [ctypes.c_void_p(0x100000 + 0x1000 * i) for i in range(n)]


def test_error_paths_return_before_any_launch():
    """Workspace, pointer and enum errors are reported from the host, with no
    GPU present (also run under the sanitizers)."""
    from grouped_gemm_expert_amd import ops
    lib = ops._lib
    cfg = ops.config(T=64, H=128, I=64, E=8, k=2)
    f, b = ops.moe_workspace_size(cfg)
    saved = ops.MoeSaved(*[p.value for p in _fake(11)])
    x, Wr, bias, w1, w2, y, aux, ws = _fake(8)
    stream = None
    by = ctypes.byref
    # forward: a workspace far too small, and a misaligned output
    assert lib.moe_forward(by(cfg), x, Wr, None, w1, w2, y, aux, by(saved), ws, 256, stream) == 3
    y_bad = ctypes.c_void_p(y.value + 4)
    assert lib.moe_forward(by(cfg), x, Wr, None, w1, w2, y_bad, aux, by(saved), ws, f, stream) == 1
    # backward: a workspace one byte short; a bad weight-gradient dtype
    dy, d_aux, dx, dl, dWr, dW1, dW2 = _fake(7)
    assert lib.moe_backward(by(cfg), by(saved), x, Wr, w1, w2, dy, d_aux, dx, dl, dWr, dW1, dW2,
                            0, 0, ws, b - 1, stream) == 3
    assert lib.moe_backward(by(cfg), by(saved), x, Wr, w1, w2, dy, d_aux, dx, dl, dWr, dW1, dW2,
                            7, 0, ws, b, stream) == 1
    # permute_checked needs its status word
    c, o, rm, ps = _fake(4)
    assert lib.moe_permute_checked(by(cfg), x, c, o, rm, ps, None, ws, f, stream) == 1
    # saved sizes need an output array; MX sizes need K % 32 == 0
    assert lib.moe_saved_sizes(by(cfg), None) == 1
    n = ctypes.c_size_t(0)
    assert lib.moe_mx_size(10, 48, by(n)) == 1
    assert lib.moe_mx_size(10, 64, by(n)) == 0 and n.value > 0
    # split intermediates: the MXFP8 and per-op GEMM entry points refuse them,
    # and the forward needs h_lo / a_lo in the saved set
    cfg_s = ops.config(T=64, H=128, I=64, E=8, k=2, precision="split")
    fs, bs = ops.moe_workspace_size(cfg_s)
    assert fs >= f and bs > b
    assert lib.moe_forward_mx(by(cfg_s), x, Wr, None, w1, w2, y, aux, by(saved), ws, fs,
                              stream) == 2
    saved_nolo = ops.MoeSaved(*([p.value for p in _fake(9)] + [None, None]))
    assert lib.moe_forward(by(cfg_s), x, Wr, None, w1, w2, y, aux, by(saved_nolo), ws, fs,
                           stream) == 1
    assert ops.moe_check_config(ops.config(T=64, H=128, I=64, E=8, k=2, precision=5)) == 1
    sz = ops.moe_saved_sizes(cfg_s)
    assert sz["h_lo"] == sz["h"] and sz["a_lo"] == sz["a"]
    assert ops.moe_saved_sizes(cfg)["h_lo"] == 0
    # an unknown grouped-GEMM op
    args = ops.MoeGemmArgs()
    args.counts, args.offsets = c.value, o.value
    assert lib.moe_grouped_gemm(17, by(cfg), by(args), ws, f, stream) == 1
