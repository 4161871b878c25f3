"""Python binding of libmoe (include/moe.h): argument marshalling only.

Every function here has the name of a C entry point, takes torch tensors that
already live on the GPU, passes their device pointers and the current HIP
stream to the library, and raises if the library reports an error.  No step of
the expert path runs in Python or in PyTorch: torch only owns the memory and
the stream.  If libmoe.so is missing, importing this module raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

# MOE_LIBRARY may name another build of the same library (a tuning variant).
_LIB_PATH = os.environ.get("MOE_LIBRARY") or os.path.join(
    os.path.dirname(os.path.abspath(__file__)), "libmoe.so")

MOE_SOFTMAX, MOE_SIGMOID = 0, 1
MOE_F32, MOE_BF16 = 0, 1
MOE_ROUTE_LEARNED, MOE_ROUTE_EVEN = 0, 1
MOE_PRECISION_BF16, MOE_PRECISION_SPLIT = 0, 1
(MOE_GEMM_UP_SWIGLU, MOE_GEMM_DOWN, MOE_GEMM_DOWN_DGRAD, MOE_GEMM_UP_DGRAD,
 MOE_GEMM_DOWN_WGRAD, MOE_GEMM_UP_WGRAD) = range(6)

_P = ctypes.c_void_p


class MoeConfig(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int64), ("H", ctypes.c_int32), ("I", ctypes.c_int32),
                ("E", ctypes.c_int32), ("k", ctypes.c_int32), ("n_groups", ctypes.c_int32),
                ("topk_groups", ctypes.c_int32), ("score", ctypes.c_int32),
                ("renorm", ctypes.c_int32), ("scale", ctypes.c_float),
                ("aux_coeff", ctypes.c_float), ("route_mode", ctypes.c_int32),
                ("precision", ctypes.c_int32)]


class MoeSaved(ctypes.Structure):
    _fields_ = [(n, _P) for n in ("logits", "topk_idx", "topk_w", "counts", "offsets",
                                  "row_map", "pos", "h", "a", "h_lo", "a_lo")]


class MoeGemmArgs(ctypes.Structure):
    _fields_ = [(n, _P) for n in ("x", "dy", "w1", "w2", "counts", "offsets", "row_map",
                                  "topk_w", "h", "a", "o", "dh", "dw_part", "dxp", "dW1",
                                  "dW2")] + [("dw_dtype", ctypes.c_int32),
                                             ("dw_accumulate", ctypes.c_int32)]


class MoeGemmMxArgs(ctypes.Structure):
    _fields_ = [(n, _P) for n in ("x_mx", "w1_mx", "w2_mx", "a_mx", "counts", "offsets",
                                  "row_map", "h", "a", "o")]


class MoeError(RuntimeError):
    pass


def _load():
    if not os.path.exists(_LIB_PATH):
        raise MoeError(f"{_LIB_PATH} is missing: build it with "
                       "`python -m grouped_gemm_expert_amd.build` (there is no fallback)")
    lib = ctypes.CDLL(_LIB_PATH)
    S = ctypes.c_int  # moe_status
    CFG = ctypes.POINTER(MoeConfig)
    sz = ctypes.c_size_t
    lib.moe_status_string.argtypes = [S]
    lib.moe_status_string.restype = ctypes.c_char_p
    lib.moe_version.argtypes = []
    lib.moe_version.restype = ctypes.c_char_p
    lib.moe_check_config.argtypes = [CFG]
    lib.moe_check_config.restype = S
    lib.moe_workspace_size.argtypes = [CFG, ctypes.POINTER(sz), ctypes.POINTER(sz)]
    lib.moe_workspace_size.restype = S
    lib.moe_dw_part_cols.argtypes = [CFG]
    lib.moe_dw_part_cols.restype = ctypes.c_int32
    lib.moe_router.argtypes = [CFG] + [_P] * 9 + [_P, sz, _P]
    lib.moe_router.restype = S
    lib.moe_permute.argtypes = [CFG] + [_P] * 5 + [_P, sz, _P]
    lib.moe_permute.restype = S
    lib.moe_permute_checked.argtypes = [CFG] + [_P] * 6 + [_P, sz, _P]
    lib.moe_permute_checked.restype = S
    lib.moe_saved_sizes.argtypes = [CFG, ctypes.POINTER(sz)]
    lib.moe_saved_sizes.restype = S
    lib.moe_forward_noalloc.argtypes = [CFG] + [_P] * 7 + [ctypes.POINTER(MoeSaved), _P]
    lib.moe_forward_noalloc.restype = S
    lib.moe_forward_noalloc_bytes.argtypes = [CFG, ctypes.POINTER(sz)]
    lib.moe_forward_noalloc_bytes.restype = S
    lib.moe_grouped_gemm.argtypes = [ctypes.c_int32, CFG, ctypes.POINTER(MoeGemmArgs), _P, sz, _P]
    lib.moe_grouped_gemm.restype = S
    lib.moe_swiglu.argtypes = [ctypes.c_int32, ctypes.c_int64, ctypes.c_int32, _P, _P, _P, _P]
    lib.moe_swiglu.restype = S
    lib.moe_combine.argtypes = [CFG, _P, _P, _P, _P, _P]
    lib.moe_combine.restype = S
    lib.moe_forward.argtypes = [CFG] + [_P] * 7 + [ctypes.POINTER(MoeSaved), _P, sz, _P]
    lib.moe_forward.restype = S
    lib.moe_backward.argtypes = ([CFG, ctypes.POINTER(MoeSaved)] + [_P] * 11
                                 + [ctypes.c_int32, ctypes.c_int32, _P, sz, _P])
    lib.moe_backward.restype = S
    SP = ctypes.POINTER(MoeSaved)
    I32 = ctypes.c_int32
    lib.moe_stage1_forward.argtypes = [CFG] + [_P] * 5 + [SP, _P, sz, _P]
    lib.moe_stage1_forward.restype = S
    lib.moe_stage2_forward.argtypes = [CFG, _P, SP, _P, _P, sz, _P]
    lib.moe_stage2_forward.restype = S
    lib.moe_stage2_backward.argtypes = [CFG, SP, _P, _P, _P, I32, I32, _P, sz, _P]
    lib.moe_stage2_backward.restype = S
    lib.moe_stage1_backward.argtypes = [CFG, SP] + [_P] * 8 + [I32, I32, _P, sz, _P]
    lib.moe_stage1_backward.restype = S
    lib.moe_set_stage_events.argtypes = [ctypes.c_int32, _P, _P]
    lib.moe_set_stage_events.restype = S
    lib.moe_grouped_gemm_mx.argtypes = [ctypes.c_int32, CFG, ctypes.POINTER(MoeGemmMxArgs), _P,
                                         sz, _P]
    lib.moe_grouped_gemm_mx.restype = S
    lib.moe_mx_size.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.POINTER(sz)]
    lib.moe_mx_size.restype = S
    lib.moe_mx_quantize.argtypes = [_P, ctypes.c_int64, ctypes.c_int64, _P, sz, _P]
    lib.moe_mx_quantize.restype = S
    lib.moe_stage1_forward_mx.argtypes = [CFG] + [_P] * 5 + [SP, _P, sz, _P]
    lib.moe_stage1_forward_mx.restype = S
    lib.moe_stage2_forward_mx.argtypes = [CFG, _P, SP, _P, _P, sz, _P]
    lib.moe_stage2_forward_mx.restype = S
    lib.moe_forward_mx.argtypes = [CFG] + [_P] * 7 + [SP, _P, sz, _P]
    lib.moe_forward_mx.restype = S
    lib.moe_mx_quantize_t.argtypes = [_P, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, _P, sz, _P]
    lib.moe_mx_quantize_t.restype = S
    lib.moe_mx_quantize_both.argtypes = [_P, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, _P, sz,
                                         _P, sz, _P]
    lib.moe_mx_quantize_both.restype = S
    lib.moe_stage2_backward_mx.argtypes = [CFG, SP, _P, _P, _P, I32, I32, _P, sz, _P]
    lib.moe_stage2_backward_mx.restype = S
    lib.moe_stage1_backward_mx.argtypes = [CFG, SP] + [_P] * 8 + [I32, I32, _P, sz, _P]
    lib.moe_stage1_backward_mx.restype = S
    lib.moe_backward_mx.argtypes = [CFG, SP] + [_P] * 11 + [I32, I32, _P, sz, _P]
    lib.moe_backward_mx.restype = S
    return lib


_lib = _load()

SYMBOLS = ("moe_status_string", "moe_version", "moe_check_config", "moe_workspace_size",
           "moe_saved_sizes", "moe_dw_part_cols", "moe_router", "moe_permute",
           "moe_permute_checked", "moe_forward_noalloc", "moe_forward_noalloc_bytes",
           "moe_grouped_gemm", "moe_swiglu",
           "moe_combine", "moe_forward", "moe_backward", "moe_stage1_forward",
           "moe_stage2_forward", "moe_stage2_backward", "moe_stage1_backward",
           "moe_set_stage_events", "moe_grouped_gemm_mx", "moe_mx_size", "moe_mx_quantize", "moe_stage1_forward_mx",
           "moe_stage2_forward_mx", "moe_forward_mx", "moe_mx_quantize_t", "moe_mx_quantize_both",
           "moe_stage2_backward_mx", "moe_stage1_backward_mx", "moe_backward_mx")

STAGES = {"up_swiglu": 0, "down": 1, "down_dgrad": 2, "up_dgrad": 3, "down_wgrad": 4,
          "up_wgrad": 5, "router_proj": 6, "router": 7, "permute": 8, "combine": 9,
          "router_bwd": 10, "unpermute": 11, "router_grads": 12, "mx_quant": 13,
          "operands_bwd2": 14, "operands_bwd1": 15}


def moe_set_stage_events(stage: int, start, stop):
    """Register torch.cuda.Event objects (or None) for a stage of the path."""
    sp = None if start is None else ctypes.c_void_p(start.cuda_event)
    ep = None if stop is None else ctypes.c_void_p(stop.cuda_event)
    _check(_lib.moe_set_stage_events(int(stage), sp, ep), "moe_set_stage_events")


def lib_path() -> str:
    return _LIB_PATH


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_contiguous():
        raise MoeError("tensor arguments must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _check(status: int, what: str):
    if status != 0:
        raise MoeError(f"{what}: {_lib.moe_status_string(status).decode()} (status {status})")


def config(T, H, I, E, k, n_groups=1, topk_groups=1, score="softmax", renorm=False,
           scale=1.0, aux_coeff=0.01, route="learned", precision="bf16") -> MoeConfig:
    sc = {"softmax": MOE_SOFTMAX, "sigmoid": MOE_SIGMOID}.get(score, score)
    rm = {"learned": MOE_ROUTE_LEARNED, "even": MOE_ROUTE_EVEN}.get(route, route)
    pr = {"bf16": MOE_PRECISION_BF16, "split": MOE_PRECISION_SPLIT}.get(precision, precision)
    return MoeConfig(int(T), int(H), int(I), int(E), int(k), int(n_groups), int(topk_groups),
                     int(sc), int(bool(renorm)), float(scale), float(aux_coeff), int(rm), int(pr))


def config_from_workload(w, T=None, precision=None) -> MoeConfig:
    """The layer config of a workload; precision defaults to the workload's."""
    return config(w.T if T is None else T, w.H, w.I, w.E, w.k, w.n_groups, w.topk_groups,
                  w.score, w.renorm, w.scale, w.aux_coeff, w.route,
                  w.precision if precision is None else precision)


def moe_version() -> str:
    return _lib.moe_version().decode()


def moe_check_config(cfg: MoeConfig) -> int:
    return int(_lib.moe_check_config(ctypes.byref(cfg)))


def moe_workspace_size(cfg: MoeConfig):
    f, b = ctypes.c_size_t(0), ctypes.c_size_t(0)
    _check(_lib.moe_workspace_size(ctypes.byref(cfg), ctypes.byref(f), ctypes.byref(b)),
           "moe_workspace_size")
    return int(f.value), int(b.value)


def moe_dw_part_cols(cfg: MoeConfig) -> int:
    return int(_lib.moe_dw_part_cols(ctypes.byref(cfg)))


def workspace(cfg: MoeConfig, which: str = "fwd", device="cuda") -> torch.Tensor:
    f, b = moe_workspace_size(cfg)
    n = f if which == "fwd" else b
    return torch.empty(max(n, 256), dtype=torch.uint8, device=device)


def moe_router(cfg, x, Wr, bias, logits, sel_scores, topk_idx, topk_w, counts, aux, ws,
               stream=None):
    _check(_lib.moe_router(ctypes.byref(cfg), _ptr(x), _ptr(Wr), _ptr(bias), _ptr(logits),
                           _ptr(sel_scores), _ptr(topk_idx), _ptr(topk_w), _ptr(counts),
                           _ptr(aux), _ptr(ws), ws.numel(), _stream(stream)), "moe_router")


def moe_permute(cfg, topk_idx, counts, offsets, row_map, pos, ws, stream=None):
    _check(_lib.moe_permute(ctypes.byref(cfg), _ptr(topk_idx), _ptr(counts), _ptr(offsets),
                            _ptr(row_map), _ptr(pos), _ptr(ws), ws.numel(), _stream(stream)),
           "moe_permute")


def moe_permute_checked(cfg, topk_idx, counts, offsets, row_map, pos, n_bad, ws, stream=None):
    _check(_lib.moe_permute_checked(ctypes.byref(cfg), _ptr(topk_idx), _ptr(counts),
                                    _ptr(offsets), _ptr(row_map), _ptr(pos), _ptr(n_bad),
                                    _ptr(ws), ws.numel(), _stream(stream)), "moe_permute_checked")


SAVED_N = 11


def moe_saved_sizes(cfg: MoeConfig) -> dict:
    """Bytes of each tensor of moe_saved, by name."""
    arr = (ctypes.c_size_t * SAVED_N)()
    _check(_lib.moe_saved_sizes(ctypes.byref(cfg), arr), "moe_saved_sizes")
    return {name: int(arr[i]) for i, (name, _) in enumerate(MoeSaved._fields_)}


def moe_grouped_gemm(op, cfg, ws, stream=None, dw_dtype=MOE_F32, dw_accumulate=False, **tensors):
    args = MoeGemmArgs()
    for name, t in tensors.items():
        if name not in dict(MoeGemmArgs._fields_):
            raise MoeError(f"unknown grouped-GEMM argument {name}")
        setattr(args, name, None if t is None else t.data_ptr())
    args.dw_dtype = dw_dtype
    args.dw_accumulate = int(bool(dw_accumulate))
    _check(_lib.moe_grouped_gemm(int(op), ctypes.byref(cfg), ctypes.byref(args), _ptr(ws),
                                 ws.numel(), _stream(stream)), "moe_grouped_gemm")


def moe_swiglu(backward, h, out, da=None, stream=None):
    M = h.shape[0]
    I = h.shape[1] // 2
    _check(_lib.moe_swiglu(int(bool(backward)), M, I, _ptr(h), _ptr(da), _ptr(out),
                           _stream(stream)), "moe_swiglu")


def moe_combine(cfg, o, topk_w, pos, y, stream=None):
    _check(_lib.moe_combine(ctypes.byref(cfg), _ptr(o), _ptr(topk_w), _ptr(pos), _ptr(y),
                            _stream(stream)), "moe_combine")


def _saved_struct(saved: dict) -> MoeSaved:
    s = MoeSaved()
    for name, _ in MoeSaved._fields_:
        t = saved.get(name)
        setattr(s, name, None if t is None else t.data_ptr())
    return s


def alloc_saved(cfg: MoeConfig, device="cuda") -> dict:
    """The forward's saved tensors (caller-owned; see moe_saved in moe.h),
    sized by moe_saved_sizes and shaped for use from torch."""
    T, E, k, I = cfg.T, cfg.E, cfg.k, cfg.I
    M = T * k
    shapes = {"logits": ((T, E), torch.float32), "topk_idx": ((T, k), torch.int32),
              "topk_w": ((T, k), torch.float32), "counts": ((E,), torch.int32),
              "offsets": ((E + 1,), torch.int32), "row_map": ((M,), torch.int32),
              "pos": ((M,), torch.int32), "h": ((M, 2 * I), torch.bfloat16),
              "a": ((M, I), torch.bfloat16), "h_lo": ((M, 2 * I), torch.bfloat16),
              "a_lo": ((M, I), torch.bfloat16)}
    sizes = moe_saved_sizes(cfg)
    out = {}
    for name, (shape, dt) in shapes.items():
        if name in ("h_lo", "a_lo") and sizes[name] == 0:
            continue                          # not used at this precision
        n = 1
        for d in shape:
            n *= d
        if n * torch.tensor([], dtype=dt).element_size() != sizes[name]:
            raise MoeError(f"moe_saved_sizes disagrees on {name}")
        # empty tensors still get one element so that every pointer is valid
        out[name] = torch.empty(shape if n else (1,) + tuple(shape[1:]), dtype=dt, device=device)
    return out


def moe_forward(cfg, x, Wr, bias, w1, w2, y, aux, saved: dict, ws, stream=None):
    s = _saved_struct(saved)
    _check(_lib.moe_forward(ctypes.byref(cfg), _ptr(x), _ptr(Wr), _ptr(bias), _ptr(w1),
                            _ptr(w2), _ptr(y), _ptr(aux), ctypes.byref(s), _ptr(ws), ws.numel(),
                            _stream(stream)), "moe_forward")


def moe_backward(cfg, saved: dict, x, Wr, w1, w2, dy, d_aux, dx, dlogits, dWr, dW1, dW2, ws,
                 dw_accumulate=False, stream=None):
    s = _saved_struct(saved)
    dw_dtype = MOE_BF16 if dW1.dtype == torch.bfloat16 else MOE_F32
    _check(_lib.moe_backward(ctypes.byref(cfg), ctypes.byref(s), _ptr(x), _ptr(Wr), _ptr(w1),
                             _ptr(w2), _ptr(dy), _ptr(d_aux), _ptr(dx), _ptr(dlogits), _ptr(dWr),
                             _ptr(dW1), _ptr(dW2), dw_dtype, int(bool(dw_accumulate)), _ptr(ws),
                             ws.numel(), _stream(stream)), "moe_backward")


NOALLOC_SCRATCH_BYTES = 64 << 20   # MOE_NOALLOC_SCRATCH_BYTES


def moe_forward_noalloc_bytes(cfg) -> int:
    b = ctypes.c_size_t(0)
    _check(_lib.moe_forward_noalloc_bytes(ctypes.byref(cfg), ctypes.byref(b)),
           "moe_forward_noalloc_bytes")
    return int(b.value)


def moe_forward_noalloc(cfg, x, Wr, bias, w1, w2, y, aux, saved: dict, stream=None):
    """moe_forward on the library's own scratch array (no workspace argument)."""
    s = _saved_struct(saved)
    _check(_lib.moe_forward_noalloc(ctypes.byref(cfg), _ptr(x), _ptr(Wr), _ptr(bias), _ptr(w1),
                                    _ptr(w2), _ptr(y), _ptr(aux), ctypes.byref(s),
                                    _stream(stream)), "moe_forward_noalloc")


def moe_stage1_forward(cfg, x, Wr, bias, w1, aux, saved: dict, ws, stream=None):
    s = _saved_struct(saved)
    _check(_lib.moe_stage1_forward(ctypes.byref(cfg), _ptr(x), _ptr(Wr), _ptr(bias), _ptr(w1),
                                   _ptr(aux), ctypes.byref(s), _ptr(ws), ws.numel(),
                                   _stream(stream)), "moe_stage1_forward")


def moe_stage2_forward(cfg, w2, saved: dict, y, ws, stream=None):
    s = _saved_struct(saved)
    _check(_lib.moe_stage2_forward(ctypes.byref(cfg), _ptr(w2), ctypes.byref(s), _ptr(y),
                                   _ptr(ws), ws.numel(), _stream(stream)), "moe_stage2_forward")


def moe_stage2_backward(cfg, saved: dict, w2, dy, dW2, ws, dw_accumulate=False, stream=None):
    s = _saved_struct(saved)
    dw_dtype = MOE_BF16 if dW2.dtype == torch.bfloat16 else MOE_F32
    _check(_lib.moe_stage2_backward(ctypes.byref(cfg), ctypes.byref(s), _ptr(w2), _ptr(dy),
                                    _ptr(dW2), dw_dtype, int(bool(dw_accumulate)), _ptr(ws),
                                    ws.numel(), _stream(stream)), "moe_stage2_backward")


def moe_stage1_backward(cfg, saved: dict, x, Wr, w1, d_aux, dx, dlogits, dWr, dW1, ws,
                        dw_accumulate=False, stream=None):
    s = _saved_struct(saved)
    dw_dtype = MOE_BF16 if dW1.dtype == torch.bfloat16 else MOE_F32
    _check(_lib.moe_stage1_backward(ctypes.byref(cfg), ctypes.byref(s), _ptr(x), _ptr(Wr),
                                    _ptr(w1), _ptr(d_aux), _ptr(dx), _ptr(dlogits), _ptr(dWr),
                                    _ptr(dW1), dw_dtype, int(bool(dw_accumulate)), _ptr(ws),
                                    ws.numel(), _stream(stream)), "moe_stage1_backward")


# ------------------------------------------------------------------ MXFP8 ----

def mx_kp(K: int) -> int:
    """K rounded up to the 128-column groups of an MX matrix."""
    return (K + 127) // 128 * 128


def moe_mx_size(rows: int, K: int) -> int:
    b = ctypes.c_size_t()
    _check(_lib.moe_mx_size(int(rows), int(K), ctypes.byref(b)), "moe_mx_size")
    return int(b.value)


def mx_alloc(rows: int, K: int, device="cuda") -> torch.Tensor:
    """An uninitialised MX-matrix buffer for a [rows, K] matrix (uint8)."""
    return torch.empty(max(moe_mx_size(rows, K), 1), dtype=torch.uint8, device=device)


def mx_views(buf: torch.Tensor, rows: int, K: int):
    """(codes [rows, Kp], scales [rows, Kp/32]) of an MX-matrix buffer: the
    codes as a view, the scales gathered from their 32-row-block layout into
    block order (a new tensor)."""
    Kp = mx_kp(K)
    gpr = Kp // 128
    rows_p = (rows + 31) // 32 * 32
    codes = buf[:rows * Kp].view(rows, Kp)
    raw = buf[rows * Kp:rows * Kp + rows_p * Kp // 32].view(rows_p // 32, gpr, 32, 4)
    words = raw.permute(0, 2, 1, 3).reshape(rows_p, gpr, 4)[:rows]   # [row][group][0, 2, 1, 3]
    scales = words[:, :, [0, 2, 1, 3]].reshape(rows, Kp // 32)
    return codes, scales


def moe_mx_quantize(src: torch.Tensor, dst: torch.Tensor, stream=None):
    """MX matrix of a bf16 matrix src [rows, K] (any leading shape is flattened
    into rows) into dst (uint8, moe_mx_size bytes)."""
    K = src.shape[-1]
    rows = src.numel() // K if K else 0
    _check(_lib.moe_mx_quantize(_ptr(src), rows, K, _ptr(dst), dst.numel(), _stream(stream)),
           "moe_mx_quantize")


def moe_mx_quantize_t(src: torch.Tensor, dst: torch.Tensor, stream=None):
    """MX matrix of every batch's transpose of src [batches, R, C] (bf16),
    stacked as [batches*C, R] along R, into dst (moe_mx_size bytes)."""
    B, R, C = src.shape
    _check(_lib.moe_mx_quantize_t(_ptr(src), B, R, C, _ptr(dst), dst.numel(), _stream(stream)),
           "moe_mx_quantize_t")


def moe_mx_quantize_both(src: torch.Tensor, dst: torch.Tensor, dst_t: torch.Tensor, stream=None):
    """Both MX forms of src [batches, R, C] (bf16) from one read: dst the MX
    matrix of [batches*R, C] along C, dst_t that of the stacked transposes
    [batches*C, R] along R (each moe_mx_size bytes)."""
    B, R, C = src.shape
    _check(_lib.moe_mx_quantize_both(_ptr(src), B, R, C, _ptr(dst), dst.numel(), _ptr(dst_t),
                                     dst_t.numel(), _stream(stream)), "moe_mx_quantize_both")


class MxWeightCache:
    """The MXFP8 forms of w1 and w2, rebuilt when either weight changes: the
    forward's (w1 along H, w2 along I) and, with backward=True, the
    transposed ones the backward's data gradients use (w1[e]^T along 2I,
    w2[e]^T along H).

    The key is each weight's storage, shape and in-place version counter; as
    with the pages' cache, that is not enough when an optimizer writes the
    weights without bumping the version, so `drop()` (once per optimizer step)
    forces the next `get` to quantise again."""

    def __init__(self, backward: bool = False):
        self._key = None
        self.backward = backward
        self.w1_mx = None
        self.w2_mx = None
        self.w1t_mx = None
        self.w2t_mx = None
        self.builds = 0

    @staticmethod
    def _k(w):
        return (w.data_ptr(), tuple(w.shape), w._version)

    def drop(self):
        self._key = None

    def get(self, w1: torch.Tensor, w2: torch.Tensor, stream=None):
        key = (self._k(w1), self._k(w2))
        if key != self._key:
            E, twoI, H = w1.shape
            I = w2.shape[2]
            if self.w1_mx is None or self.w1_mx.numel() != moe_mx_size(E * twoI, H):
                self.w1_mx = mx_alloc(E * twoI, H, w1.device)
            if self.w2_mx is None or self.w2_mx.numel() != moe_mx_size(E * H, I):
                self.w2_mx = mx_alloc(E * H, I, w2.device)
            if self.backward:
                # both forms of each weight from one read of it
                if self.w1t_mx is None or self.w1t_mx.numel() != moe_mx_size(E * H, twoI):
                    self.w1t_mx = mx_alloc(E * H, twoI, w1.device)
                if self.w2t_mx is None or self.w2t_mx.numel() != moe_mx_size(E * I, H):
                    self.w2t_mx = mx_alloc(E * I, H, w2.device)
                moe_mx_quantize_both(w1, self.w1_mx, self.w1t_mx, stream)
                moe_mx_quantize_both(w2, self.w2_mx, self.w2t_mx, stream)
            else:
                moe_mx_quantize(w1, self.w1_mx, stream)
                moe_mx_quantize(w2, self.w2_mx, stream)
            self._key = key
            self.builds += 1
        return self.w1_mx, self.w2_mx


def moe_forward_mx(cfg, x, Wr, bias, w1_mx, w2_mx, y, aux, saved: dict, ws, stream=None):
    s = _saved_struct(saved)
    _check(_lib.moe_forward_mx(ctypes.byref(cfg), _ptr(x), _ptr(Wr), _ptr(bias), _ptr(w1_mx),
                               _ptr(w2_mx), _ptr(y), _ptr(aux), ctypes.byref(s), _ptr(ws),
                               ws.numel(), _stream(stream)), "moe_forward_mx")


def moe_stage1_forward_mx(cfg, x, Wr, bias, w1_mx, aux, saved: dict, ws, stream=None):
    s = _saved_struct(saved)
    _check(_lib.moe_stage1_forward_mx(ctypes.byref(cfg), _ptr(x), _ptr(Wr), _ptr(bias),
                                      _ptr(w1_mx), _ptr(aux), ctypes.byref(s), _ptr(ws),
                                      ws.numel(), _stream(stream)), "moe_stage1_forward_mx")


def moe_stage2_forward_mx(cfg, w2_mx, saved: dict, y, ws, stream=None):
    s = _saved_struct(saved)
    _check(_lib.moe_stage2_forward_mx(ctypes.byref(cfg), _ptr(w2_mx), ctypes.byref(s), _ptr(y),
                                      _ptr(ws), ws.numel(), _stream(stream)),
           "moe_stage2_forward_mx")


def moe_grouped_gemm_mx(op: int, cfg, *, ws, counts, offsets, row_map=None, x_mx=None,
                        w1_mx=None, w2_mx=None, a_mx=None, h=None, a=None, o=None, stream=None):
    args = MoeGemmMxArgs(*[_ptr(t) for t in (x_mx, w1_mx, w2_mx, a_mx, counts, offsets, row_map,
                                              h, a, o)])
    _check(_lib.moe_grouped_gemm_mx(int(op), ctypes.byref(cfg), ctypes.byref(args), _ptr(ws),
                                    ws.numel(), _stream(stream)), "moe_grouped_gemm_mx")


def moe_backward_mx(cfg, saved: dict, x, Wr, w1t_mx, w2t_mx, dy, d_aux, dx, dlogits, dWr, dW1, dW2,
                    ws, dw_accumulate=False, stream=None):
    s = _saved_struct(saved)
    dw_dtype = MOE_BF16 if dW1.dtype == torch.bfloat16 else MOE_F32
    _check(_lib.moe_backward_mx(ctypes.byref(cfg), ctypes.byref(s), _ptr(x), _ptr(Wr),
                                _ptr(w1t_mx), _ptr(w2t_mx), _ptr(dy), _ptr(d_aux), _ptr(dx),
                                _ptr(dlogits), _ptr(dWr), _ptr(dW1), _ptr(dW2), dw_dtype,
                                int(bool(dw_accumulate)), _ptr(ws), ws.numel(), _stream(stream)),
           "moe_backward_mx")


def moe_stage2_backward_mx(cfg, saved: dict, w2t_mx, dy, dW2, ws, dw_accumulate=False,
                           stream=None):
    s = _saved_struct(saved)
    dw_dtype = MOE_BF16 if dW2.dtype == torch.bfloat16 else MOE_F32
    _check(_lib.moe_stage2_backward_mx(ctypes.byref(cfg), ctypes.byref(s), _ptr(w2t_mx), _ptr(dy),
                                       _ptr(dW2), dw_dtype, int(bool(dw_accumulate)), _ptr(ws),
                                       ws.numel(), _stream(stream)), "moe_stage2_backward_mx")


def moe_stage1_backward_mx(cfg, saved: dict, x, Wr, w1t_mx, d_aux, dx, dlogits, dWr, dW1, ws,
                           dw_accumulate=False, stream=None):
    s = _saved_struct(saved)
    dw_dtype = MOE_BF16 if dW1.dtype == torch.bfloat16 else MOE_F32
    _check(_lib.moe_stage1_backward_mx(ctypes.byref(cfg), ctypes.byref(s), _ptr(x), _ptr(Wr),
                                       _ptr(w1t_mx), _ptr(d_aux), _ptr(dx), _ptr(dlogits),
                                       _ptr(dWr), _ptr(dW1), dw_dtype, int(bool(dw_accumulate)),
                                       _ptr(ws), ws.numel(), _stream(stream)),
           "moe_stage1_backward_mx")
