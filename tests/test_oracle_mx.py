"""Pins for the oracle's MXFP8 half (page "MegaMoE", "Expert precision": the
mxfp8 mode runs both expert stages in MXFP8).  MXFP8 is read as the OCP
Microscaling format: E4M3 elements, blocks of 32 along the contraction
dimension, one E8M0 scale 2^X per block with X = floor(log2 amax) - 8.  CPU
only."""
import math
import os

import numpy as np
import pytest
import scipy.special

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "mx_blocks.txt")


def _bf16(a):
    """float array -> bf16 bit patterns (the inputs here are exactly representable)."""
    f = np.ascontiguousarray(a, np.float32)
    u = f.view(np.uint32)
    assert np.all(u & 0xFFFF == 0), "input not exactly representable in bf16"
    return (u >> 16).astype(np.uint16)


def _bf16_value(b):
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


# ----------------------------------------------------------- E4M3 points ----

def test_e4m3_fixed_points():
    v = oracle.e4m3_values()
    # the points the E4M3 definition fixes: zero, the smallest subnormal and
    # the largest one, the smallest normal, one, the largest finite value
    assert v[0x00] == 0.0 and not math.copysign(1, v[0x00]) < 0
    assert v[0x80] == 0.0 and math.copysign(1, v[0x80]) < 0
    assert v[0x01] == 2.0 ** -9
    assert v[0x07] == 7 * 2.0 ** -9
    assert v[0x08] == 2.0 ** -6
    assert v[0x38] == 1.0
    assert v[0x7E] == 448.0
    assert math.isnan(v[0x7F]) and math.isnan(v[0xFF])
    assert v[0xFE] == -448.0


def test_e4m3_monotone_and_symmetric():
    v = oracle.e4m3_values()
    pos = v[0x00:0x7F]
    assert np.all(np.diff(pos) > 0)
    assert np.array_equal(v[0x80:0xFF], -pos)
    # every finite positive value has at most 4 significant bits
    for x in pos[1:]:
        m, _ = math.frexp(x)
        assert (m * 16) == int(m * 16)


# --------------------------------------------------------------- golden ----

def _golden_blocks():
    blocks = []
    with open(GOLDEN) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            parts = line.split()
            if parts[0] == "block":
                blocks.append((parts[1], int(parts[2]), []))
            else:
                blocks[-1][2].append((int(parts[0]), int(parts[1], 16), int(parts[2], 16)))
    return blocks


@pytest.mark.parametrize("block", _golden_blocks(), ids=lambda b: b[0])
def test_golden_blocks(block):
    name, scale, items = block
    src = np.zeros((1, 32), np.uint16)
    want = np.zeros(32, np.uint8)
    for pos, bits, code in items:
        src[0, pos] = bits
        want[pos] = code
    codes, scales = oracle.mx_quantize(src)
    assert scales[0, 0] == scale, name
    assert np.array_equal(codes[0], want), (name, codes[0], want)


# --------------------------------------------------------- round trips ----

def test_every_finite_code_round_trips():
    """Blocks holding 448 * 2^j fix X = j, so every E4M3 value times 2^j is
    exactly representable and must come back as its own code."""
    v = oracle.e4m3_values()
    finite = [c for c in range(256) if not math.isnan(v[c])]
    for j in (-20, 0, 7, 60):
        vals = [v[c] * 2.0 ** j for c in finite]
        codes_in = list(finite)
        while len(vals) % 31:
            vals.append(0.0)
            codes_in.append(0x00)
        rows = []
        want = []
        for b in range(0, len(vals), 31):
            rows.append([448.0 * 2.0 ** j] + vals[b:b + 31])
            want.append([0x7E] + codes_in[b:b + 31])
        src = _bf16(np.array(rows))
        codes, scales = oracle.mx_quantize(src)
        assert np.all(scales == j + 127)
        assert np.array_equal(codes, np.array(want, np.uint8))
        assert np.array_equal(oracle.mx_dequantize(codes, scales), _bf16_value(src))


# ------------------------------------------------------------ error bound ----

@pytest.mark.parametrize("sigma", [1e-3, 0.02, 1.0, 300.0])
def test_scale_range_and_half_spacing_bound(sigma):
    rng = np.random.default_rng(11)
    x = rng.normal(0.0, sigma, (64, 256)).astype(np.float32)
    x[3, 32:64] = 0.0                                   # an all-zero block
    x[5, :32] *= 1e-3                                   # a block far below the rest of its row
    src = (x.view(np.uint32) >> 16).astype(np.uint16)   # truncated to bf16
    v = _bf16_value(src)
    codes, scales = oracle.mx_quantize(src)
    d = oracle.mx_dequantize(codes, scales)
    X = scales.astype(np.int64) - 127
    blocks = np.abs(v).reshape(64, 8, 32)
    amax = blocks.max(axis=2)
    nz = amax > 0
    # 2^8 <= amax / 2^X < 2^9 for every non-zero block
    r = amax[nz] / np.ldexp(1.0, X[nz])
    assert np.all((r >= 256) & (r < 512))
    assert np.all(X[~nz] == -127)
    # each element is within half a grid spacing of its value; the grid
    # spacing at |q| = |v| / 2^X is 2^(max(floor(log2 |q|), -6) - 3); values
    # above 448 * 2^X saturate to it
    sx = np.repeat(np.ldexp(1.0, X), 32, axis=1)
    q = np.abs(v) / sx
    sat = q > 448
    assert np.all(np.abs(d[sat]) == 448 * sx[sat])
    assert np.all(np.sign(d[sat]) == np.sign(v[sat]))
    e = np.floor(np.log2(np.where(q > 0, q, 1.0)))
    spacing = np.ldexp(1.0, (np.maximum(e, -6) - 3).astype(np.int64)) * sx
    err = np.abs(d - v)
    assert np.all(err[~sat] <= spacing[~sat] / 2)
    # exact ties (bf16 keeps 8 significant bits, E4M3 4, so about one value
    # in 16 is halfway) go to the even grid point
    tie = (~sat) & (err == spacing / 2) & (err > 0)
    assert tie.any()
    assert np.all((np.abs(d[tie]) / spacing[tie]) % 2 == 0)


# ------------------------------------------------------- the MX GEMMs ----

def _representable(rng, shape, kaxis_len):
    """Integers in [-7, 7] with |v| in 4..7 somewhere in every 32-block, each
    block times its own 2^j: then X = j + 2 - 8 and every value is exact in
    E4M3 (7 * 2^6 = 448), with a different scale from block to block."""
    a = rng.integers(-7, 8, size=shape).astype(np.float64)
    flat = a.reshape(-1, kaxis_len // 32, 32)
    flat[:, :, 0] = rng.choice([-7, -6, -5, -4, 4, 5, 6, 7], size=flat.shape[:2])
    flat *= np.ldexp(1.0, rng.integers(-3, 4, size=flat.shape[:2]))[:, :, None]
    return flat.reshape(shape)


def test_mx_gemms_exact_on_representable_inputs():
    rng = np.random.default_rng(3)
    T, H, I, E, k = 12, 64, 64, 3, 2
    x = _representable(rng, (T, H), H)
    w1 = _representable(rng, (E, 2 * I, H), H)
    w2 = _representable(rng, (E, H, I), I)
    ops = oracle.MxOperands(_bf16(x), _bf16(w1), _bf16(w2))
    assert np.array_equal(oracle.mx_dequantize(ops.xq, ops.xs), x)
    idx = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    slots = np.arange(T * k)
    g, u, a, aq, as_, o = oracle.mx_expert_rows(ops, idx, slots)
    for f in slots:
        t, e = f // k, idx.flat[f]
        h = x[t] @ w1[e].T   # exact: dyadic values, sums far below 2^53
        assert np.array_equal(g[f], h[:I]) and np.array_equal(u[f], h[I:])
        ref_a = g[f] * scipy.special.expit(g[f]) * u[f]
        assert np.allclose(a[f], ref_a, rtol=1e-12, atol=0)
        # the second GEMM takes the MX values of a: bf16(fp32(a)) quantised
        ab = _bf16_value(_round_bf16(a[f].astype(np.float32)))
        ac, asc = oracle.mx_quantize(_round_bf16(a[f].astype(np.float32))[None, :])
        assert np.array_equal(aq[f], ac[0]) and np.array_equal(as_[f], asc[0])
        ad = oracle.mx_dequantize(ac, asc)[0]
        sx = np.repeat(np.ldexp(1.0, asc[0].astype(np.int64) - 127), 32)
        sat = np.abs(ab) > 448 * sx       # the floor-based scale saturates (448, 512) * 2^X
        assert np.all(np.abs(ad[sat]) == 448 * sx[sat])
        assert np.all(np.abs(ad - ab)[~sat] <= (np.abs(ab) * 2.0 ** -4 + 2.0 ** -10 * sx)[~sat])
        assert np.allclose(o[f], w2[e] @ ad, rtol=1e-12, atol=1e-9)


def _round_bf16(f32):
    u = np.ascontiguousarray(f32, np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def test_mx_forward_combines_expert_rows_and_is_permutation_invariant():
    rng = np.random.default_rng(5)
    T, H, I, E, k = 10, 64, 96, 4, 2
    x = _round_bf16(rng.normal(0, 1, (T, H)).astype(np.float32))
    w1 = _round_bf16(rng.normal(0, 0.05, (E, 2 * I, H)).astype(np.float32))
    w2 = _round_bf16(rng.normal(0, 0.05, (E, H, I)).astype(np.float32))
    idx = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    w = rng.uniform(0.1, 1.0, (T, k))
    ops = oracle.MxOperands(x, w1, w2)
    y = oracle.mx_forward(ops, idx, w)
    *_, o = oracle.mx_expert_rows(ops, idx, np.arange(T * k))
    ref = (w.reshape(T * k, 1) * o).reshape(T, k, H).sum(axis=1)
    assert np.allclose(y, ref, rtol=1e-13, atol=1e-13)
    perm = rng.permutation(T)
    ops_p = oracle.MxOperands(x[perm], w1, w2)
    yp = oracle.mx_forward(ops_p, idx[perm], w[perm])
    assert np.array_equal(yp, y[perm])


def test_mx_forward_within_the_format_error_of_the_exact_forward():
    """E4M3 keeps 4 significant bits: each quantised operand is within 2^-4
    relative of its value, so the MX forward stays within a few per cent
    (relative Frobenius) of the exact forward and is not identical to it."""
    rng = np.random.default_rng(9)
    T, H, I, E, k = 16, 128, 128, 4, 2
    x = _round_bf16(rng.normal(0, 1, (T, H)).astype(np.float32))
    w1 = _round_bf16(rng.normal(0, 0.02, (E, 2 * I, H)).astype(np.float32))
    w2 = _round_bf16(rng.normal(0, 0.02, (E, H, I)).astype(np.float32))
    idx = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    w = rng.uniform(0.1, 1.0, (T, k))
    y_mx = oracle.mx_forward(oracle.MxOperands(x, w1, w2), idx, w)
    y = oracle.forward(x, w1, w2, idx, w)
    rel = np.linalg.norm(y_mx - y) / np.linalg.norm(y)
    assert 1e-3 < rel < 0.08, rel


# ------------------------------------------------------------- backward ----

def _deq(bits2d):
    c, s = oracle.mx_quantize(bits2d)
    return oracle.mx_dequantize(c, s)


def _deq_cols(mat):
    """MX values of a [n, C] float matrix quantised along its rows (down each
    column) in blocks of 32 from row 0, the last block padded with zeros: the
    columns are transposed, padded and fed to the row quantiser."""
    n, C = mat.shape
    npad = (n + 31) // 32 * 32
    t = np.zeros((C, npad), np.float32)
    t[:, :n] = mat.T
    return _deq(_round_bf16(t))[:, :n].T      # values already bf16: RNE is exact


def _bwd_setup(seed, T=12, H=64, I=64, E=3, k=2):
    rng = np.random.default_rng(seed)
    x = _round_bf16(rng.normal(0, 1, (T, H)).astype(np.float32))
    w1 = _round_bf16(rng.normal(0, 0.05, (E, 2 * I, H)).astype(np.float32))
    w2 = _round_bf16(rng.normal(0, 0.05, (E, H, I)).astype(np.float32))
    dy = _round_bf16(rng.normal(0, 1, (T, H)).astype(np.float32))
    idx = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    w = rng.uniform(0.1, 1.0, (T, k))
    return x, w1, w2, dy, idx, w


def _numpy_mx_backward(x, w1, w2, dy, idx, w):
    """dx (expert part), dw [T,k], dW1, dW2 of the MXFP8 backward from the
    quantiser and dense fp64 matmuls."""
    T, H = x.shape
    E, twoI, _ = w1.shape
    I = twoI // 2
    k = idx.shape[1]
    Xd, DYd = _deq(x), _deq(dy)
    W1d = _deq(w1.reshape(E * twoI, H)).reshape(E, twoI, H)
    W2d = _deq(w2.reshape(E * H, I)).reshape(E, H, I)
    W2c = _deq(np.ascontiguousarray(w2.transpose(0, 2, 1)).reshape(E * I, H)).reshape(E, I, H)
    W1c = _deq(np.ascontiguousarray(w1.transpose(0, 2, 1)).reshape(E * H, twoI)).reshape(E, H, twoI)
    dx = np.zeros((T, H))
    dw = np.zeros((T, k))
    rows = {e: [] for e in range(E)}
    for f in range(T * k):
        t, j = divmod(f, k)
        e = idx[t, j]
        h = Xd[t] @ W1d[e].T
        g, u = h[:I], h[I:]
        ab = _bf16_value(_round_bf16((g * scipy.special.expit(g) * u).astype(np.float32)))
        dAp = DYd[t] @ W2c[e].T
        dw[t, j] = dAp @ ab
        dA = w[t, j] * dAp
        # the SwiGLU backward reads h as saved: g, u rounded to fp32, then bf16
        gb = _bf16_value(_round_bf16(g.astype(np.float32)))
        ub = _bf16_value(_round_bf16(u.astype(np.float32)))
        sg = scipy.special.expit(gb)
        dh = np.concatenate([dA * ub * sg * (1 + gb * (1 - sg)), dA * gb * sg])
        dhb = _round_bf16(dh.astype(np.float32))
        dx[t] += _deq(dhb[None, :])[0] @ W1c[e].T
        dyw = _bf16_value(_round_bf16((w[t, j] * _bf16_value(dy[t])).astype(np.float32)))
        rows[e].append((_bf16_value(dhb), ab, dyw, _bf16_value(x[t])))
    dW1 = np.zeros((E, twoI, H))
    dW2 = np.zeros((E, H, I))
    for e, rs in rows.items():
        if not rs:
            continue
        DH, A, DYW, XG = (np.stack([r[q] for r in rs]) for q in range(4))
        dW1[e] = _deq_cols(DH).T @ _deq_cols(XG)
        dW2[e] = _deq_cols(DYW).T @ _deq_cols(A)
    return dx, dw, dW1, dW2


def _numpy_mx_backward_abs(x, w1, w2, dy, idx, w):
    """As _numpy_mx_backward, with dW1 / dW2 formed from the magnitudes of
    their MX operands (the sums of |terms|)."""
    T, H = x.shape
    E, twoI, _ = w1.shape
    I = twoI // 2
    k = idx.shape[1]
    Xd, DYd = _deq(x), _deq(dy)
    W1d = _deq(w1.reshape(E * twoI, H)).reshape(E, twoI, H)
    W2c = _deq(np.ascontiguousarray(w2.transpose(0, 2, 1)).reshape(E * I, H)).reshape(E, I, H)
    rows = {e: [] for e in range(E)}
    for f in range(T * k):
        t, j = divmod(f, k)
        e = idx[t, j]
        h = Xd[t] @ W1d[e].T
        g, u = h[:I], h[I:]
        ab = _bf16_value(_round_bf16((g * scipy.special.expit(g) * u).astype(np.float32)))
        dA = w[t, j] * (DYd[t] @ W2c[e].T)
        gb = _bf16_value(_round_bf16(g.astype(np.float32)))
        ub = _bf16_value(_round_bf16(u.astype(np.float32)))
        sg = scipy.special.expit(gb)
        dh = np.concatenate([dA * ub * sg * (1 + gb * (1 - sg)), dA * gb * sg])
        dyw = _bf16_value(_round_bf16((w[t, j] * _bf16_value(dy[t])).astype(np.float32)))
        rows[e].append((_bf16_value(_round_bf16(dh.astype(np.float32))), ab, dyw,
                        _bf16_value(x[t])))
    aW1 = np.zeros((E, twoI, H))
    aW2 = np.zeros((E, H, I))
    for e, rs in rows.items():
        if not rs:
            continue
        DH, A, DYW, XG = (np.stack([r[q] for r in rs]) for q in range(4))
        aW1[e] = np.abs(_deq_cols(DH)).T @ np.abs(_deq_cols(XG))
        aW2[e] = np.abs(_deq_cols(DYW)).T @ np.abs(_deq_cols(A))
    return None, None, aW1, aW2


def test_mx_backward_tokens_against_numpy():
    x, w1, w2, dy, idx, w = _bwd_setup(21)
    T, E, k = x.shape[0], w1.shape[0], idx.shape[1]
    ops = oracle.MxBackwardOperands(x, w1, w2, dy)
    counts = np.bincount(idx.ravel(), minlength=E).astype(np.int32)
    logits = np.random.default_rng(4).normal(0, 1, (T, E))
    # softmax router, no renorm, no aux: dp at the chosen experts is dw itself
    dx, dl = oracle.mx_backward_tokens(ops, None, logits, idx, counts, w, score=oracle.SOFTMAX,
                                       renorm=False, scale=1.0, coeff=0.0, d_aux=0.0)
    dx_ref, dw_ref, _, _ = _numpy_mx_backward(x, w1, w2, dy, idx, w)
    assert np.allclose(dx, dx_ref, rtol=1e-9, atol=1e-12)
    p = scipy.special.softmax(logits, axis=1)
    dp = np.zeros((T, E))
    np.put_along_axis(dp, idx.astype(np.int64), dw_ref, axis=1)
    dl_ref = p * (dp - (dp * p).sum(1, keepdims=True))
    assert np.allclose(dl, dl_ref, rtol=1e-9, atol=1e-12)


def test_mx_weight_grad_elements_against_numpy():
    x, w1, w2, dy, idx, w = _bwd_setup(22, T=40, E=3, k=2)     # ~27 rows per expert: a ragged block
    E, twoI, H = w1.shape
    I = twoI // 2
    ops = oracle.MxBackwardOperands(x, w1, w2, dy)
    _, _, dW1, dW2 = _numpy_mx_backward(x, w1, w2, dy, idx, w)
    rng = np.random.default_rng(5)
    which, ee, rr, cc = [], [], [], []
    for e in range(E):
        for wh, nr, nc in ((1, twoI, H), (2, H, I)):
            which += [wh] * 16
            ee += [e] * 16
            rr += rng.integers(0, nr, 16).tolist()
            cc += rng.integers(0, nc, 16).tolist()
    got = oracle.mx_weight_grad_elements(ops, x, dy, idx, w, which, ee, rr, cc)
    which, ee, rr, cc = map(np.array, (which, ee, rr, cc))
    ref = np.where(which == 1, dW1[ee, np.minimum(rr, twoI - 1), np.minimum(cc, H - 1)],
                   dW2[ee, np.minimum(rr, H - 1), np.minimum(cc, I - 1)])
    assert np.allclose(got, ref, rtol=1e-9, atol=1e-12)


def test_mx_weight_grad_lines_against_numpy():
    """Whole rows of dW1 and columns of dW2 of the MXFP8 backward against the
    numpy formulation (ragged last 32-row block included)."""
    x, w1, w2, dy, idx, w = _bwd_setup(24, T=40, E=3, k=2)
    E, twoI, H = w1.shape
    I = twoI // 2
    ops = oracle.MxBackwardOperands(x, w1, w2, dy)
    _, _, dW1, dW2 = _numpy_mx_backward(x, w1, w2, dy, idx, w)
    ee = np.repeat(np.arange(E), 3)
    rows = np.tile([0, I + 3, twoI - 1], E)
    cols = np.tile([0, 17, I - 1], E)
    l1, m1 = oracle.mx_weight_grad_lines(ops, x, dy, idx, w, np.ones_like(ee), ee, rows,
                                         with_magnitude=True)
    l2 = oracle.mx_weight_grad_lines(ops, x, dy, idx, w, np.full_like(ee, 2), ee, cols)
    assert np.allclose(l1, dW1[ee, rows, :], rtol=1e-9, atol=1e-12)
    assert np.allclose(l2, dW2[ee, :, cols], rtol=1e-9, atol=1e-12)
    # the magnitudes: the same sums over |terms| (numpy formulation, |operands|)
    _, _, aW1, _ = _numpy_mx_backward_abs(x, w1, w2, dy, idx, w)
    assert np.allclose(m1, aW1[ee, rows, :], rtol=1e-9, atol=1e-12)
    assert (m1 >= np.abs(l1) - 1e-12).all()


def test_mx_backward_within_the_format_error_of_the_exact_backward():
    x, w1, w2, dy, idx, w = _bwd_setup(23, T=16, H=128, I=128, E=4, k=2)
    T, E = x.shape[0], w1.shape[0]
    ops = oracle.MxBackwardOperands(x, w1, w2, dy)
    counts = np.bincount(idx.ravel(), minlength=E).astype(np.int32)
    logits = np.random.default_rng(6).normal(0, 1, (T, E))
    # the routing weights the bf16 oracle derives from the logits (softmax, no renorm)
    w = np.take_along_axis(scipy.special.softmax(logits, axis=1), idx.astype(np.int64), axis=1)
    kw = dict(score=oracle.SOFTMAX, renorm=False, scale=1.0, coeff=0.01, d_aux=1.0)
    dx_mx, _ = oracle.mx_backward_tokens(ops, None, logits, idx, counts, w, **kw)
    dx, _ = oracle.backward_tokens(x, None, logits, w1, w2, idx, counts, dy, **kw)
    rel = np.linalg.norm(dx_mx - dx) / np.linalg.norm(dx)
    assert 1e-3 < rel < 0.1, rel


def test_backward_operands_from_experts_match_full():
    """The sparse-expert operands equal the full ones on the given experts and
    are zero elsewhere (so outputs that read only those experts agree)."""
    rng = np.random.default_rng(0)
    T, H, I, E = 20, 64, 64, 4
    bits = lambda a: (np.asarray(a, np.float32).view(np.uint32) >> 16).astype(np.uint16)
    x, dy = bits(rng.normal(0, 1, (T, H))), bits(rng.normal(0, 1, (T, H)))
    w1, w2 = bits(rng.normal(0, .05, (E, 2 * I, H))), bits(rng.normal(0, .05, (E, H, I)))
    full = oracle.MxBackwardOperands(x, w1, w2, dy)
    ex = np.array([1, 3])
    sp = oracle.MxBackwardOperands.from_experts(x, dy, E, ex, w1[ex], w2[ex])
    for n in ("xq", "xs", "dyq", "dys"):
        assert np.array_equal(getattr(full, n), getattr(sp, n)), n
    for n, rows in (("w1", 2 * I), ("w2", H), ("w2c", I), ("w1c", H)):
        for suf in "qs":
            a = getattr(full, n + suf).reshape(E, rows, -1)
            b = getattr(sp, n + suf).reshape(E, rows, -1)
            assert np.array_equal(a[ex], b[ex]) and not b[[0, 2]].any(), n + suf
