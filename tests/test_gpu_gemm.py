"""Per-op parity of the grouped GEMMs (moe_grouped_gemm) and the stand-alone
SwiGLU / combine entry points.  Operands are seeded synthetic tensors; the
routing maps come from the oracle's permutation; each expert segment is
checked against an fp64 matmul of the op's definition on the CPU."""
import numpy as np
import pytest
import torch

import oracle
from tests import harness as hz

pytestmark = pytest.mark.gpu

SHAPES = [
    # T, H, I, E, k  -- ragged M segments, an empty expert, N and K tails
    (300, 384, 320, 8, 3),
    (97, 128, 64, 4, 2),
    (513, 256, 192, 16, 4),
]


def _setup(T, H, I, E, k, seed=0, idx=None):
    g = torch.Generator().manual_seed(seed)
    rng = np.random.default_rng(seed)
    if idx is None:
        p = 1.0 / np.arange(1, E + 1) ** 1.1
        p[E // 2] = 0.0                              # one empty expert
        idx = np.stack([rng.choice(E, size=k, replace=False, p=p / p.sum()) for _ in range(T)])
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    counts, offsets, row_map, pos = oracle.permute(idx, E)
    M = T * k
    bf = lambda *s, std=1.0: (torch.randn(*s, generator=g) * std).to(torch.bfloat16)
    t = dict(
        x=bf(T, H), dy=bf(T, H), w1=bf(E, 2 * I, H, std=0.05), w2=bf(E, H, I, std=0.05),
        h=bf(M, 2 * I), a=bf(M, I, std=0.5), dh=bf(M, 2 * I, std=0.5),
        topk_w=torch.rand(T, k, generator=g),
    )
    maps = dict(counts=counts, offsets=offsets, row_map=row_map, pos=pos, idx=idx)
    return t, maps


def _dev(t, maps):
    d = {k: v.cuda() for k, v in t.items()}
    for k in ("counts", "offsets", "row_map", "pos"):
        d[k] = torch.from_numpy(maps[k]).cuda()
    return d


def _segments(maps, E):
    return [(e, int(maps["offsets"][e]), int(maps["offsets"][e + 1])) for e in range(E)]


@pytest.mark.parametrize("shape", SHAPES)
def test_up_swiglu_and_down(shape):
    T, H, I, E, k = shape
    hz.say(f"gemm up_swiglu/down T={T} H={H} I={I} E={E} k={k}")
    t, maps = _setup(T, H, I, E, k)
    _check_forward(T, H, I, E, k, t, maps)


def _check_forward(T, H, I, E, k, t, maps):
    """GEMM1 (with the SwiGLU epilogue) and GEMM2 of the given routing against
    an fp64 evaluation of their definitions, per expert segment."""
    from grouped_gemm_expert_amd import ops
    d = _dev(t, maps)
    cfg = ops.config(T=T, H=H, I=I, E=E, k=k)
    M = T * k
    ws = ops.workspace(cfg, "fwd")
    h = torch.empty((M, 2 * I), dtype=torch.bfloat16, device="cuda")
    a = torch.empty((M, I), dtype=torch.bfloat16, device="cuda")
    o = torch.empty((M, H), dtype=torch.float32, device="cuda")
    ops.moe_grouped_gemm(ops.MOE_GEMM_UP_SWIGLU, cfg, ws, x=d["x"], w1=d["w1"],
                         counts=d["counts"], offsets=d["offsets"], row_map=d["row_map"], h=h, a=a)
    ops.moe_grouped_gemm(ops.MOE_GEMM_DOWN, cfg, ws, a=d["a"], w2=d["w2"], counts=d["counts"],
                         offsets=d["offsets"], row_map=d["row_map"], o=o)
    torch.cuda.synchronize()
    x, w1, w2, a_in = (t[n].double() for n in ("x", "w1", "w2", "a"))
    rm = torch.from_numpy(maps["row_map"]).long()
    hg, ag, og = h.double().cpu(), a.double().cpu(), o.double().cpu()
    for e, s0, s1 in _segments(maps, E):
        if s1 == s0:
            continue
        xs = x[rm[s0:s1] // k]
        hr = xs @ w1[e].T                                   # [rows, 2I]
        gr, ur = hr[:, :I], hr[:, I:]
        ar = gr * torch.sigmoid(gr) * ur
        tol = 2.0 ** -8 * hr.abs() + 1e-4
        assert ((hg[s0:s1] - hr).abs() <= tol).all(), e
        assert ((ag[s0:s1] - ar).abs() <= 2.0 ** -8 * ar.abs() + 1e-4).all(), e
        orf = a_in[s0:s1] @ w2[e].T
        mx, fro = hz.errors(og[s0:s1].numpy(), orf.numpy())
        assert fro <= 1e-5 and mx <= 1e-4 * float(orf.abs().max()) + 1e-6, (e, mx, fro)


@pytest.mark.parametrize("shape", SHAPES)
def test_dgrad_ops(shape):
    T, H, I, E, k = shape
    hz.say(f"gemm dgrad T={T} H={H} I={I} E={E} k={k}")
    t, maps = _setup(T, H, I, E, k, seed=1)
    _check_dgrad(T, H, I, E, k, t, maps)


# Rows per expert around the points where a segment's last 256-row m-tile
# changes shape in the dgrad kernels' partial main loop: a wave copies 32
# rows of A and multiplies 32-row fragments, so 1, 31..33, 63..65, 127..129,
# 224, 225, 255..257 and 511 rows, and an empty expert.
BOUNDARY_ROWS = [1, 15, 16, 17, 31, 32, 33, 63, 64, 65, 127, 128, 129, 224, 225, 255, 256, 257,
                 0, 511]


def test_dgrad_partial_tiles_at_wave_boundaries():
    E, H, I = len(BOUNDARY_ROWS), 128, 64
    idx = np.repeat(np.arange(E, dtype=np.int32), BOUNDARY_ROWS)
    np.random.default_rng(4).shuffle(idx)            # tokens of an expert scattered
    T = len(idx)
    hz.say(f"gemm dgrad, segment ends at wave boundaries: T={T} E={E} k=1")
    t, maps = _setup(T, H, I, E, 1, seed=4, idx=idx[:, None])
    assert maps["counts"].tolist() == BOUNDARY_ROWS
    _check_dgrad(T, H, I, E, 1, t, maps)


# Rows per expert around the mixed m-tiling's shapes (forward and dgrad
# GEMMs): 257..320 rows are one 320-row tile, 321 two 256-row tiles, 513 and
# 576 a 256-row tile and a 320-row one, 577 three 256-row tiles, 832 two
# 256-row tiles and a 320-row one.
MIXED_ROWS = [257, 258, 288, 289, 300, 319, 320, 321, 512, 513, 576, 577, 832, 256, 255, 65, 0,
              1]


def test_mixed_m_tiles():
    E, H, I = len(MIXED_ROWS), 384, 320
    idx = np.repeat(np.arange(E, dtype=np.int32), MIXED_ROWS)
    np.random.default_rng(6).shuffle(idx)
    T = len(idx)
    hz.say(f"gemm up_swiglu/down/dgrad, mixed m-tiles: T={T} E={E} k=1")
    t, maps = _setup(T, H, I, E, 1, seed=6, idx=idx[:, None])
    assert maps["counts"].tolist() == MIXED_ROWS
    _check_forward(T, H, I, E, 1, t, maps)
    _check_dgrad(T, H, I, E, 1, t, maps)


def _check_dgrad(T, H, I, E, k, t, maps):
    """dgrad2 (with the SwiGLU backward and row-dot epilogue) and dgrad1 of the
    given routing against an fp64 evaluation of their definitions, per
    expert segment."""
    from grouped_gemm_expert_amd import ops
    d = _dev(t, maps)
    cfg = ops.config(T=T, H=H, I=I, E=E, k=k)
    M = T * k
    ncols = ops.moe_dw_part_cols(cfg)
    ws = ops.workspace(cfg, "fwd")
    dh = torch.empty((M, 2 * I), dtype=torch.bfloat16, device="cuda")
    dwp = torch.empty((M, ncols), dtype=torch.float32, device="cuda")
    dxp = torch.empty((M, H), dtype=torch.float32, device="cuda")
    ops.moe_grouped_gemm(ops.MOE_GEMM_DOWN_DGRAD, cfg, ws, dy=d["dy"], w2=d["w2"],
                         counts=d["counts"], offsets=d["offsets"], row_map=d["row_map"],
                         topk_w=d["topk_w"], h=d["h"], a=d["a"], dh=dh, dw_part=dwp)
    ops.moe_grouped_gemm(ops.MOE_GEMM_UP_DGRAD, cfg, ws, dh=d["dh"], w1=d["w1"],
                         counts=d["counts"], offsets=d["offsets"], row_map=d["row_map"], dxp=dxp)
    torch.cuda.synchronize()
    dy, w1, w2, h, a, dh_in = (t[n].double() for n in ("dy", "w1", "w2", "h", "a", "dh"))
    tw = t["topk_w"].double().reshape(-1)
    rm = torch.from_numpy(maps["row_map"]).long()
    dhg, dwg, dxg = dh.double().cpu(), dwp.double().cpu().sum(1), dxp.double().cpu()
    for e, s0, s1 in _segments(maps, E):
        if s1 == s0:
            continue
        rows = rm[s0:s1]
        dap = dy[rows // k] @ w2[e]                         # [rows, I]
        dw_ref = (dap * a[s0:s1]).sum(1)
        assert ((dwg[s0:s1] - dw_ref).abs() <= 1e-4 * (dap.abs() * a[s0:s1].abs()).sum(1)
                + 1e-6).all(), e
        da = tw[rows][:, None] * dap
        gg, uu = h[s0:s1, :I], h[s0:s1, I:]
        sg = torch.sigmoid(gg)
        dg = da * uu * sg * (1 + gg * (1 - sg))
        du = da * gg * sg
        ref = torch.cat([dg, du], 1)
        assert ((dhg[s0:s1] - ref).abs() <= 2.0 ** -8 * ref.abs() + 1e-4 * (1 + ref.abs().max())).all(), e
        dx_ref = dh_in[s0:s1] @ w1[e]
        mx, fro = hz.errors(dxg[s0:s1].numpy(), dx_ref.numpy())
        assert fro <= 1e-5, (e, mx, fro)


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("accumulate", [False, True])
def test_wgrad_ops(shape, accumulate):
    from grouped_gemm_expert_amd import ops
    T, H, I, E, k = shape
    hz.say(f"gemm wgrad T={T} H={H} I={I} E={E} k={k} acc={accumulate}")
    t, maps = _setup(T, H, I, E, k, seed=2)
    d = _dev(t, maps)
    cfg = ops.config(T=T, H=H, I=I, E=E, k=k)
    ws = ops.workspace(cfg, "fwd")
    g = torch.Generator().manual_seed(5)
    init1 = torch.randn(E, 2 * I, H, generator=g)
    init2 = torch.randn(E, H, I, generator=g)
    dW1 = init1.cuda() if accumulate else torch.full((E, 2 * I, H), 7.0, device="cuda")
    dW2 = init2.cuda() if accumulate else torch.full((E, H, I), 7.0, device="cuda")
    kw = dict(counts=d["counts"], offsets=d["offsets"], row_map=d["row_map"],
              dw_accumulate=accumulate)
    ops.moe_grouped_gemm(ops.MOE_GEMM_DOWN_WGRAD, cfg, ws, dy=d["dy"], a=d["a"],
                         topk_w=d["topk_w"], dW2=dW2, **kw)
    ops.moe_grouped_gemm(ops.MOE_GEMM_UP_WGRAD, cfg, ws, dh=d["dh"], x=d["x"], dW1=dW1, **kw)
    torch.cuda.synchronize()
    x, dy, a, dh_in = (t[n].double() for n in ("x", "dy", "a", "dh"))
    tw = t["topk_w"].double().reshape(-1)
    rm = torch.from_numpy(maps["row_map"]).long()
    g1, g2 = dW1.double().cpu(), dW2.double().cpu()
    if accumulate:
        g1 -= init1.double()
        g2 -= init2.double()
    for e, s0, s1 in _segments(maps, E):
        rows = rm[s0:s1]
        if s1 == s0:
            if accumulate:
                assert torch.equal(dW1[e].cpu(), init1[e]) and torch.equal(dW2[e].cpu(), init2[e])
            else:
                assert not dW1[e].any() and not dW2[e].any()
            continue
        ref2 = (tw[rows][:, None] * dy[rows // k]).T @ a[s0:s1]      # [H, I]
        mx, fro = hz.errors(g2[e].numpy(), ref2.numpy())
        assert fro <= 4e-3, (e, mx, fro)
        ref1 = dh_in[s0:s1].T @ x[rows // k]                         # [2I, H]
        mx, fro = hz.errors(g1[e].numpy(), ref1.numpy())
        assert fro <= 1e-5, (e, mx, fro)


def test_swiglu_and_combine_entry_points():
    from grouped_gemm_expert_amd import ops
    hz.say("swiglu + combine")
    T, H, I, E, k = 200, 256, 192, 8, 3
    t, maps = _setup(T, H, I, E, k, seed=3)
    M = T * k
    h = t["h"].cuda()
    a = torch.empty((M, I), dtype=torch.bfloat16, device="cuda")
    ops.moe_swiglu(False, h, a)
    g = torch.Generator().manual_seed(9)
    da = torch.randn(M, I, generator=g)
    dh = torch.empty((M, 2 * I), dtype=torch.bfloat16, device="cuda")
    ops.moe_swiglu(True, h, dh, da=da.cuda())
    o = torch.randn(M, H, generator=g)
    y = torch.empty((T, H), device="cuda")
    cfg = ops.config(T=T, H=H, I=I, E=E, k=k)
    ops.moe_combine(cfg, o.cuda(), t["topk_w"].cuda(), torch.from_numpy(maps["pos"]).cuda(), y)
    y1 = torch.empty((T, H), device="cuda")
    ops.moe_combine(cfg, o.cuda(), None, torch.from_numpy(maps["pos"]).cuda(), y1)
    torch.cuda.synchronize()
    hd = t["h"].double()
    gg, uu = hd[:, :I], hd[:, I:]
    sg = torch.sigmoid(gg)
    ar = gg * sg * uu
    assert ((a.double().cpu() - ar).abs() <= 2.0 ** -8 * ar.abs() + 1e-6).all()
    dd = da.double()
    ref = torch.cat([dd * uu * sg * (1 + gg * (1 - sg)), dd * gg * sg], 1)
    assert ((dh.double().cpu() - ref).abs() <= 2.0 ** -8 * ref.abs() + 1e-6).all()
    pos = torch.from_numpy(maps["pos"]).long().view(T, k)
    od = o.double()
    yr = (t["topk_w"].double()[:, :, None] * od[pos]).sum(1)
    assert (y.double().cpu() - yr).abs().max() <= 1e-5 * float(yr.abs().max())
    assert (y1.double().cpu() - od[pos].sum(1)).abs().max() <= 1e-5 * float(od.abs().max() * k)
