"""CPU oracle for the MoE expert path -- TEST INFRASTRUCTURE ONLY.

Only the test-suite, the smoke check in ``__graft_entry__`` and the CPU-baseline
leg of ``bench.py`` may import this package.  The product path (the HIP library
and its Python binding) never imports, links or calls anything here, and this
package imports nothing from the product path.

The arithmetic lives in ``moe_oracle.c`` (plain C, double precision, per-token
loops); this module only builds that file with gcc, loads it with ctypes and
marshals numpy arrays.  bf16 tensors are passed as ``uint16`` bit patterns.

Parity status of each function (what pins it, in ``tests/test_oracle_*.py``):
  logits               -- pinned: E=1 / dense reduction and per-element brute force
  selection_scores     -- pinned: monotonicity / bias closed forms
  topk                 -- pinned: brute-force subset enumeration, all-equal closed form
  weights              -- pinned: sum identities, E=1 closed form
  permute              -- pinned: `even` routing closed form (MegaMoE page,
                          force-load-balancing table), golden fixture
  even_topk            -- pinned: the same hand-worked golden fixture (its idx
                          lines), equal counts, weights against numpy softmax
  aux                  -- pinned: uniform-probability closed form (aux == coeff),
                          E=1 closed form.  The formula itself is a reading (the
                          pages name a "standard aux_loss" without a formula).
  forward              -- pinned: E=1/k=1 dense SwiGLU MLP, token-permutation
                          invariance, linearity in w2
  expert_rows          -- pinned: y = sum_j w_j o_j against forward
  backward_tokens, weight_grads, weight_grad_elements, weight_grad_lines,
  router_weight_grad   -- pinned: central finite differences of the forward and
                          an independent torch fp64 autograd formulation
  e4m3_values          -- pinned: the E4M3 points the OCP MX format fixes (zero,
                          smallest subnormal, smallest normal, one, 448, NaN),
                          strict monotonicity over all finite codes
  mx_quantize          -- pinned: hand-worked golden blocks, round trip of every
                          finite code, the half-spacing error bound and the
                          scale range, exactness on representable inputs
  mx_expert_rows, mx_forward
                       -- pinned: exact integer GEMMs on MX-representable inputs,
                          y = sum_j w_j o_j against mx_forward, the MX error
                          bound against the exact forward
  mx_backward_tokens, mx_weight_grad_elements, mx_weight_grad_lines
                       -- pinned: a numpy formulation from the quantiser and
                          dense matmuls (expert part of dx, dW1, dW2), the
                          router part through the bf16 oracle's pinned code,
                          and the distance to the exact backward
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
# MOE_ORACLE_LIBRARY may name another build of the same source (the
# sanitizer build of tests/test_sanitizers.py); it is loaded as it is.
_LIB_ENV = os.environ.get("MOE_ORACLE_LIBRARY")
_LIB = _LIB_ENV or os.path.join(_HERE, "libmoe_oracle.so")

SOFTMAX = 0
SIGMOID = 1

_lib = None


def build(force: bool = True, out: Optional[str] = None, sanitize: bool = False) -> str:
    """Compile moe_oracle.c into libmoe_oracle.so (gcc, OpenMP, no fast-math),
    or with sanitize=True into `out` with AddressSanitizer and
    UndefinedBehaviorSanitizer (a CPU build for tests/test_sanitizers.py)."""
    lib = out or _LIB
    if _LIB_ENV and out is None:
        return lib
    if force or not os.path.exists(lib) or os.path.getmtime(lib) < os.path.getmtime(_SRC):
        tmp = lib + ".tmp%d" % os.getpid()
        opt = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
               "-fno-sanitize-recover=undefined"] if sanitize else ["-O2"]
        cmd = (["gcc"] + opt + ["-std=c11", "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wextra",
                                "-o", tmp, _SRC, "-lm"])
        subprocess.run(cmd, check=True)
        os.replace(tmp, lib)
    return lib


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not _LIB_ENV and (not os.path.exists(_LIB) or
                         os.path.getmtime(_LIB) < os.path.getmtime(_SRC)):
        build(force=True)
    lib = ctypes.CDLL(_LIB)
    P = ctypes.c_void_p
    i64, i32, f64 = ctypes.c_int64, ctypes.c_int32, ctypes.c_double
    sig = {
        "oracle_logits": [i64, i32, i32, P, P, P],
        "oracle_selection_scores": [i64, i32, i32, P, P, P],
        "oracle_topk": [i64, i32, i32, i32, i32, P, P],
        "oracle_even_topk": [i64, i32, i32, P],
        "oracle_weights": [i64, i32, i32, i32, i32, f64, P, P, P],
        "oracle_permute": [i64, i32, i32, P, P, P, P, P],
        "oracle_aux": [i64, i32, i32, i32, f64, P, P],
        "oracle_forward": [i64, i32, i32, i32, i32, P, P, P, P, P, i64, P, P],
        "oracle_backward_tokens": [i64, i32, i32, i32, i32, i32, i32, f64, f64, f64,
                                   P, P, P, P, P, P, P, P, i64, P, P, P],
        "oracle_weight_grads": [i64, i32, i32, i32, i32, P, P, P, P, P, P, i32, P,
                                i64, P, P, P],
        "oracle_weight_grad_elements": [i64, i32, i32, i32, P, P, P, P, P, P, i64,
                                        P, P, P, P, P],
        "oracle_weight_grad_lines": [i64, i32, i32, i32, P, P, P, P, P, P, i64, P, P, P, P],
        "oracle_router_weight_grad": [i64, i32, i32, P, P, P],
        "oracle_expert_rows": [i32, i32, i32, P, P, P, P, i64, P, P, P, P, P],
        "oracle_mx_quantize": [i64, i64, P, P, P],
        "oracle_mx_expert_rows": [i32, i32, i32, P, P, P, P, P, P, P, i64, P, P, P, P, P, P, P],
        "oracle_mx_forward": [i32, i32, i32, P, P, P, P, P, P, P, P, i64, P, P],
        "oracle_mx_backward_tokens": [i64, i32, i32, i32, i32, i32, i32, f64, f64, f64,
                                      P, P, P, P, P] + [P] * 12 + [i64, P, P, P],
        "oracle_mx_weight_grad_elements": [i64, i32, i32, i32, P, P, P, P] + [P] * 8
                                          + [i64, P, P, P, P, P],
        "oracle_mx_weight_grad_lines": [i64, i32, i32, i32, P, P, P, P] + [P] * 8
                                       + [i64, P, P, P, P, P],
    }
    for name, args in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = None
    lib.oracle_aux.restype = f64
    lib.oracle_e4m3_value.argtypes = [ctypes.c_uint8]
    lib.oracle_e4m3_value.restype = f64
    _lib = lib
    return lib


def _c(a: Optional[np.ndarray], dtype) -> Optional[np.ndarray]:
    if a is None:
        return None
    return np.ascontiguousarray(a, dtype=dtype)


def _p(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def logits(x: np.ndarray, Wr: np.ndarray) -> np.ndarray:
    """l = x . Wr^T in double.  x [T,H] bf16 bits (uint16), Wr [E,H] fp32."""
    x = _c(x, np.uint16)
    Wr = _c(Wr, np.float32)
    T, H = x.shape
    E = Wr.shape[0]
    out = np.empty((T, E), np.float64)
    _load().oracle_logits(T, H, E, _p(x), _p(Wr), _p(out))
    return out


def selection_scores(logits32: np.ndarray, score: int, bias: Optional[np.ndarray] = None) -> np.ndarray:
    """fp32 selection scores from fp32 logits (S = l, or fp32(sigmoid(l)) + b)."""
    l32 = _c(logits32, np.float32)
    T, E = l32.shape
    b = _c(bias, np.float32)
    out = np.empty((T, E), np.float32)
    _load().oracle_selection_scores(T, E, score, _p(l32), _p(b), _p(out))
    return out


def topk(S: np.ndarray, k: int, n_groups: int = 1, topk_groups: int = 1) -> np.ndarray:
    """Group-limited top-k on fp32 scores -> int32 [T,k], best first."""
    S = _c(S, np.float32)
    T, E = S.shape
    out = np.empty((T, k), np.int32)
    _load().oracle_topk(T, E, k, n_groups, topk_groups, _p(S), _p(out))
    return out


def even_topk(T: int, E: int, k: int) -> np.ndarray:
    """`even` forced routing: slot (t, j) -> expert (t*k + j) % E, int32 [T,k]."""
    out = np.empty((T, k), np.int32)
    _load().oracle_even_topk(T, E, k, _p(out))
    return out


def weights(logits64: np.ndarray, idx: np.ndarray, score: int, renorm: bool, scale: float) -> np.ndarray:
    """Routing weights [T,k] in double from double logits and chosen indices."""
    l = _c(logits64, np.float64)
    idx = _c(idx, np.int32)
    T, E = l.shape
    k = idx.shape[1]
    out = np.empty((T, k), np.float64)
    _load().oracle_weights(T, E, k, score, int(bool(renorm)), float(scale), _p(l), _p(idx), _p(out))
    return out


def permute(idx: np.ndarray, E: int):
    """-> counts [E], offsets [E+1], row_map [T*k], pos [T*k] (all int32)."""
    idx = _c(idx, np.int32)
    T, k = idx.shape
    counts = np.empty(E, np.int32)
    offsets = np.empty(E + 1, np.int32)
    row_map = np.empty(T * k, np.int32)
    pos = np.empty(T * k, np.int32)
    _load().oracle_permute(T, k, E, _p(idx), _p(counts), _p(offsets), _p(row_map), _p(pos))
    return counts, offsets, row_map, pos


def aux(logits64: np.ndarray, counts: np.ndarray, k: int, score: int, coeff: float) -> float:
    l = _c(logits64, np.float64)
    counts = _c(counts, np.int32)
    T, E = l.shape
    return float(_load().oracle_aux(T, E, k, score, float(coeff), _p(l), _p(counts)))


def _toks(toks, T):
    if toks is None:
        return None, T
    t = _c(np.asarray(toks), np.int64)
    return t, t.shape[0]


def forward(x, w1, w2, idx, w, toks=None) -> np.ndarray:
    """y [ntok,H] double for the listed tokens (all when toks is None)."""
    x = _c(x, np.uint16)
    w1 = _c(w1, np.uint16)
    w2 = _c(w2, np.uint16)
    idx = _c(idx, np.int32)
    w = _c(w, np.float64)
    T, H = x.shape
    E, twoI, _ = w1.shape
    I = twoI // 2
    k = idx.shape[1]
    tk, n = _toks(toks, T)
    y = np.empty((n, H), np.float64)
    _load().oracle_forward(T, H, I, E, k, _p(x), _p(w1), _p(w2), _p(idx), _p(w), n, _p(tk), _p(y))
    return y


def backward_tokens(x, Wr, logits64, w1, w2, idx, counts, dy, *, score, renorm, scale,
                    coeff, d_aux=1.0, toks=None):
    """-> dx [ntok,H], dlogits [ntok,E] (double).  Wr may be None (logits supplied)."""
    x = _c(x, np.uint16)
    Wr = _c(Wr, np.float32)
    l = _c(logits64, np.float64)
    w1 = _c(w1, np.uint16)
    w2 = _c(w2, np.uint16)
    idx = _c(idx, np.int32)
    counts = _c(counts, np.int32)
    dy = _c(dy, np.uint16)
    T, H = x.shape
    E, twoI, _ = w1.shape
    I = twoI // 2
    k = idx.shape[1]
    tk, n = _toks(toks, T)
    dx = np.empty((n, H), np.float64)
    dl = np.empty((n, E), np.float64)
    _load().oracle_backward_tokens(T, H, I, E, k, score, int(bool(renorm)), float(scale),
                                   float(coeff), float(d_aux), _p(x), _p(Wr), _p(l), _p(w1),
                                   _p(w2), _p(idx), _p(counts), _p(dy), n, _p(tk), _p(dx), _p(dl))
    return dx, dl


def weight_grads(x, w1, w2, idx, w, dy, experts=None, toks=None):
    """-> dW1 [ne,2I,H], dW2 [ne,H,I] (double) for the listed experts."""
    x = _c(x, np.uint16)
    w1 = _c(w1, np.uint16)
    w2 = _c(w2, np.uint16)
    idx = _c(idx, np.int32)
    w = _c(w, np.float64)
    dy = _c(dy, np.uint16)
    T, H = x.shape
    E, twoI, _ = w1.shape
    I = twoI // 2
    k = idx.shape[1]
    ex = None if experts is None else _c(np.asarray(experts), np.int32)
    ne = E if ex is None else ex.shape[0]
    tk, n = _toks(toks, T)
    dW1 = np.empty((ne, twoI, H), np.float64)
    dW2 = np.empty((ne, H, I), np.float64)
    _load().oracle_weight_grads(T, H, I, E, k, _p(x), _p(w1), _p(w2), _p(idx), _p(w), _p(dy),
                                ne, _p(ex), n, _p(tk), _p(dW1), _p(dW2))
    return dW1, dW2


def weight_grad_elements(x, w1, w2, idx, w, dy, which, ee, rr, cc) -> np.ndarray:
    """Single elements of dW1 (which=1, [e,n,h]) or dW2 (which=2, [e,h,i])."""
    x = _c(x, np.uint16)
    w1 = _c(w1, np.uint16)
    w2 = _c(w2, np.uint16)
    idx = _c(idx, np.int32)
    w = _c(w, np.float64)
    dy = _c(dy, np.uint16)
    which = _c(which, np.int32)
    ee = _c(ee, np.int32)
    rr = _c(rr, np.int32)
    cc = _c(cc, np.int32)
    T, H = x.shape
    I = w2.shape[2]
    k = idx.shape[1]
    out = np.empty(which.shape[0], np.float64)
    _load().oracle_weight_grad_elements(T, H, I, k, _p(x), _p(w1), _p(w2), _p(idx), _p(w), _p(dy),
                                        which.shape[0], _p(which), _p(ee), _p(rr), _p(cc), _p(out))
    return out


def weight_grad_lines(x, w1, w2, idx, w, dy, which, ee, rr) -> np.ndarray:
    """Whole lines of the weight gradients, [n, H] double: row rr of dW1[ee]
    (which=1) or column rr of dW2[ee] (which=2)."""
    x = _c(x, np.uint16)
    w1 = _c(w1, np.uint16)
    w2 = _c(w2, np.uint16)
    idx = _c(idx, np.int32)
    w = _c(w, np.float64)
    dy = _c(dy, np.uint16)
    which, ee, rr = (_c(np.asarray(v), np.int32) for v in (which, ee, rr))
    T, H = x.shape
    I = w2.shape[2]
    k = idx.shape[1]
    out = np.empty((which.shape[0], H), np.float64)
    _load().oracle_weight_grad_lines(T, H, I, k, _p(x), _p(w1), _p(w2), _p(idx), _p(w), _p(dy),
                                     which.shape[0], _p(which), _p(ee), _p(rr), _p(out))
    return out


def expert_rows(x, w1, w2, idx, slots):
    """Per flat slot f = t*k + j: (g, u, a, o) in double, see moe_oracle.c."""
    x = _c(x, np.uint16)
    w1 = _c(w1, np.uint16)
    w2 = _c(w2, np.uint16)
    idx = _c(idx, np.int32)
    sl = _c(np.asarray(slots), np.int64)
    H = x.shape[1]
    I = w2.shape[2]
    k = idx.shape[1]
    n = sl.shape[0]
    g = np.empty((n, I)); u = np.empty((n, I)); a = np.empty((n, I)); o = np.empty((n, H))
    _load().oracle_expert_rows(H, I, k, _p(x), _p(w1), _p(w2), _p(idx), n, _p(sl), _p(g), _p(u),
                               _p(a), _p(o))
    return g, u, a, o


def router_weight_grad(x, dlogits64) -> np.ndarray:
    x = _c(x, np.uint16)
    dl = _c(dlogits64, np.float64)
    T, H = x.shape
    E = dl.shape[1]
    out = np.empty((E, H), np.float64)
    _load().oracle_router_weight_grad(T, H, E, _p(x), _p(dl), _p(out))
    return out


def route(logits64: np.ndarray, *, score: int, k: int, n_groups: int = 1, topk_groups: int = 1,
          bias=None, renorm: bool = False, scale: float = 1.0, coeff: float = 0.0,
          logits32: Optional[np.ndarray] = None, route_mode: str = "learned"):
    """Full router of the oracle: fp32 selection, top-k, weights, permutation, aux.

    ``logits32`` is the fp32 logits tensor the decision is taken on; by default
    the double logits rounded to fp32.  ``route_mode="even"`` replaces the
    decision by the `even` forced routing (groups then play no part).
    """
    l32 = np.asarray(logits64, np.float32) if logits32 is None else np.asarray(logits32, np.float32)
    S = selection_scores(l32, score, bias)
    if route_mode == "even":
        idx = even_topk(l32.shape[0], l32.shape[1], k)
    elif route_mode == "learned":
        idx = topk(S, k, n_groups, topk_groups)
    else:
        raise ValueError(f"unknown route_mode {route_mode}")
    E = l32.shape[1]
    w = weights(logits64, idx, score, renorm, scale)
    counts, offsets, row_map, pos = permute(idx, E)
    a = aux(logits64, counts, k, score, coeff)
    return dict(S=S, idx=idx, w=w, counts=counts, offsets=offsets, row_map=row_map,
                pos=pos, aux=a)


# ------------------------------------------------------------------ MXFP8 ----

def e4m3_values() -> np.ndarray:
    """The value of every E4M3 code 0..255 (NaN for 0x7F / 0xFF)."""
    lib = _load()
    return np.array([lib.oracle_e4m3_value(c) for c in range(256)], np.float64)


def mx_quantize(src: np.ndarray):
    """Row-wise MXFP8 of a bf16 matrix [R, K] (K % 32 == 0): codes [R, K] uint8,
    scales [R, K/32] uint8 (E8M0, 2^(s-127)), blocks in natural order."""
    src = _c(src, np.uint16)
    R, K = src.shape
    assert K % 32 == 0
    codes = np.empty((R, K), np.uint8)
    scales = np.empty((R, K // 32), np.uint8)
    _load().oracle_mx_quantize(R, K, _p(src), _p(codes), _p(scales))
    return codes, scales


def mx_dequantize(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """The values an MX matrix stands for (double)."""
    vals = e4m3_values()[codes]
    sc = np.ldexp(1.0, scales.astype(np.int64) - 127)
    return vals * np.repeat(sc, 32, axis=-1)


class MxOperands:
    """x, w1 and w2 quantised along their contraction dimensions."""

    def __init__(self, x, w1, w2):
        x = _c(x, np.uint16)
        w1 = _c(w1, np.uint16)
        w2 = _c(w2, np.uint16)
        T, H = x.shape
        E, twoI, _ = w1.shape
        self.H, self.I, self.E = H, twoI // 2, E
        self.xq, self.xs = mx_quantize(x)
        self.w1q, self.w1s = mx_quantize(w1.reshape(E * twoI, H))
        self.w2q, self.w2s = mx_quantize(w2.reshape(E * H, self.I))

    def ptrs(self):
        return (_p(self.xq), _p(self.xs), _p(self.w1q), _p(self.w1s), _p(self.w2q),
                _p(self.w2s))


def mx_expert_rows(ops: MxOperands, idx, slots):
    """Per flat slot f = t*k + j of the MXFP8 path: g, u, a (double [n, I]),
    aq [n, I], as [n, I/32] (a rounded to bf16 and MX-quantised), o [n, H]."""
    idx = _c(idx, np.int32)
    sl = _c(np.asarray(slots), np.int64)
    k = idx.shape[1]
    n = sl.shape[0]
    H, I = ops.H, ops.I
    g = np.empty((n, I)); u = np.empty((n, I)); a = np.empty((n, I)); o = np.empty((n, H))
    aq = np.empty((n, I), np.uint8)
    as_ = np.empty((n, I // 32), np.uint8)
    _load().oracle_mx_expert_rows(H, I, k, *ops.ptrs(), _p(idx), n, _p(sl), _p(g), _p(u), _p(a),
                                  _p(aq), _p(as_), _p(o))
    return g, u, a, aq, as_, o


def mx_forward(ops: MxOperands, idx, w, toks=None) -> np.ndarray:
    """y [ntok, H] (double) of the MXFP8 path for the listed tokens."""
    idx = _c(idx, np.int32)
    w = _c(w, np.float64)
    T, k = idx.shape
    tk, n = _toks(toks, T)
    y = np.empty((n, ops.H), np.float64)
    _load().oracle_mx_forward(ops.H, ops.I, k, *ops.ptrs(), _p(idx), _p(w), n, _p(tk), _p(y))
    return y


class MxBackwardOperands(MxOperands):
    """The forward's MX operands plus the backward's: dy along H, and the
    transposed weights w2[e]^T [I, H] along H and w1[e]^T [H, 2I] along 2I."""

    def __init__(self, x, w1, w2, dy):
        super().__init__(x, w1, w2)
        dy = _c(dy, np.uint16)
        w1 = _c(w1, np.uint16)
        w2 = _c(w2, np.uint16)
        E, H, I = self.E, self.H, self.I
        self.dyq, self.dys = mx_quantize(dy)
        self.w2cq, self.w2cs = mx_quantize(np.ascontiguousarray(w2.transpose(0, 2, 1)).reshape(E * I, H))
        self.w1cq, self.w1cs = mx_quantize(np.ascontiguousarray(w1.transpose(0, 2, 1)).reshape(E * H, 2 * I))

    def bwd_ptrs(self):
        return (_p(self.dyq), _p(self.dys), _p(self.w2cq), _p(self.w2cs), _p(self.w1cq),
                _p(self.w1cs))

    @classmethod
    def from_experts(cls, x, dy, E, experts, w1_parts, w2_parts):
        """Operands of a layer with E experts of which only `experts` are
        given (w1_parts [n, 2I, H], w2_parts [n, H, I], bf16 bits); the
        others stay zero.  The arrays have the full shapes, but np.zeros maps
        untouched pages lazily, so only the given experts take memory.  For
        outputs that read no other expert."""
        x, dy = _c(x, np.uint16), _c(dy, np.uint16)
        w1_parts, w2_parts = _c(w1_parts, np.uint16), _c(w2_parts, np.uint16)
        n, twoI, H = w1_parts.shape
        I = twoI // 2
        self = cls.__new__(cls)
        self.H, self.I, self.E = H, I, E
        self.xq, self.xs = mx_quantize(x)
        self.dyq, self.dys = mx_quantize(dy)
        for name, rows, K in (("w1", twoI, H), ("w2", H, I), ("w2c", I, H), ("w1c", H, twoI)):
            setattr(self, name + "q", np.zeros((E * rows, K), np.uint8))
            setattr(self, name + "s", np.zeros((E * rows, K // 32), np.uint8))
        for j, e in enumerate(np.asarray(experts).tolist()):
            parts = (("w1", w1_parts[j]), ("w2", w2_parts[j]), ("w2c", w2_parts[j].T),
                     ("w1c", w1_parts[j].T))
            for name, m in parts:
                q, sc = mx_quantize(np.ascontiguousarray(m))
                getattr(self, name + "q")[e * m.shape[0]:(e + 1) * m.shape[0]] = q
                getattr(self, name + "s")[e * m.shape[0]:(e + 1) * m.shape[0]] = sc
        return self


def mx_backward_tokens(ops: MxBackwardOperands, Wr, logits64, idx, counts, w, *, score, renorm,
                       scale, coeff, d_aux=1.0, toks=None):
    """-> dx [ntok,H], dlogits [ntok,E] (double) of the MXFP8 backward."""
    idx = _c(idx, np.int32)
    w = _c(w, np.float64)
    l = _c(logits64, np.float64)
    counts = _c(counts, np.int32)
    Wr = _c(Wr, np.float32)
    T, k = idx.shape
    E = l.shape[1]
    tk, n = _toks(toks, T)
    dx = np.empty((n, ops.H), np.float64)
    dl = np.empty((n, E), np.float64)
    _load().oracle_mx_backward_tokens(T, ops.H, ops.I, E, k, score, int(bool(renorm)), float(scale),
                                      float(coeff), float(d_aux), _p(Wr), _p(l), _p(idx),
                                      _p(counts), _p(w), *ops.ptrs(), *ops.bwd_ptrs(), n, _p(tk),
                                      _p(dx), _p(dl))
    return dx, dl


def mx_weight_grad_elements(ops: MxBackwardOperands, x, dy, idx, w, which, ee, rr, cc):
    """Single elements of the MXFP8 dW1 (which=1, [e,n,h]) or dW2 (which=2, [e,h,i])."""
    x = _c(x, np.uint16)
    dy = _c(dy, np.uint16)
    idx = _c(idx, np.int32)
    w = _c(w, np.float64)
    which, ee, rr, cc = (_c(np.asarray(v), np.int32) for v in (which, ee, rr, cc))
    T, k = idx.shape
    out = np.empty(which.shape[0], np.float64)
    _load().oracle_mx_weight_grad_elements(T, ops.H, ops.I, k, _p(x), _p(dy), _p(idx), _p(w),
                                           _p(ops.xq), _p(ops.xs), _p(ops.w1q), _p(ops.w1s),
                                           _p(ops.dyq), _p(ops.dys), _p(ops.w2cq), _p(ops.w2cs),
                                           which.shape[0], _p(which), _p(ee), _p(rr), _p(cc),
                                           _p(out))
    return out


def mx_weight_grad_lines(ops: MxBackwardOperands, x, dy, idx, w, which, ee, rr,
                         with_magnitude: bool = False):
    """Whole lines of the MXFP8 weight gradients, [n, H] double: row rr of
    dW1[ee] (which=1) or column rr of dW2[ee] (which=2).  With
    with_magnitude, also the sums of the terms' magnitudes (same shape)."""
    x = _c(x, np.uint16)
    dy = _c(dy, np.uint16)
    idx = _c(idx, np.int32)
    w = _c(w, np.float64)
    which, ee, rr = (_c(np.asarray(v), np.int32) for v in (which, ee, rr))
    T, k = idx.shape
    out = np.empty((which.shape[0], ops.H), np.float64)
    mag = np.empty_like(out) if with_magnitude else None
    _load().oracle_mx_weight_grad_lines(T, ops.H, ops.I, k, _p(x), _p(dy), _p(idx), _p(w),
                                        _p(ops.xq), _p(ops.xs), _p(ops.w1q), _p(ops.w1s),
                                        _p(ops.dyq), _p(ops.dys), _p(ops.w2cq), _p(ops.w2cs),
                                        which.shape[0], _p(which), _p(ee), _p(rr), _p(out),
                                        _p(mag))
    return (out, mag) if with_magnitude else out
