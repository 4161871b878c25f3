// Internal header of libmoe: device helpers and the launch functions each
// translation unit exports to the host layer (api.cpp).  gfx950 only.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe.h"

#define MOE_DEV __device__ __forceinline__

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

namespace moe {

MOE_DEV float bf2f(uint16_t b) { return __uint_as_float(((uint32_t)b) << 16); }

// fp32 -> bf16 bits, round to nearest even (gfx950 converts in hardware).
MOE_DEV uint16_t f2bf(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }

// Two fp32 -> two bf16 in one 32-bit word (lo in the low half), both rounded
// to nearest even by a single v_cvt_pk_bf16_f32.
typedef __bf16 bf16x2_v __attribute__((ext_vector_type(2)));
typedef float f32x2_v __attribute__((ext_vector_type(2)));
MOE_DEV uint32_t pack_bf2(float lo, float hi)
{
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_v){lo, hi}, bf16x2_v));
}

// Logistic function of the SwiGLU activation and its derivative.  The
// hardware reciprocal (about 1 ulp) replaces the IEEE division's ten-odd
// instructions: every value it feeds is rounded to bf16 afterwards, and in the
// GEMM epilogues this arithmetic runs while the matrix cores idle.
MOE_DEV float sigmoidf_(float z) { return __builtin_amdgcn_rcpf(1.0f + __expf(-z)); }

// Ranking used everywhere in the router: larger value first, equal values
// -> lower index first.  idx < 0 marks an empty candidate that never wins.
// The router forms its selection scores through sel_key, so that NaN (a NaN
// input) ranks as -inf and the order stays total: every lane of an arg-max
// then agrees on the winner, and the top-k yields k valid experts.
MOE_DEV float sel_key(float v) { return v != v ? -INFINITY : v; }
MOE_DEV bool ranks_before(float va, int ia, float vb, int ib)
{
    if (ib < 0) return ia >= 0;
    if (ia < 0) return false;
    return va > vb || (va == vb && ia < ib);
}

// One step of a lane-permutation reduction under ranks_before: (v, i) takes
// the better of itself and the pair DPP control CTRL brings in.
template <int CTRL>
MOE_DEV void argmax_dpp_step(float &v, int &i)
{
    const float ov = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
    const int oi = __builtin_amdgcn_update_dpp(0, i, CTRL, 0xF, 0xF, false);
    if (ranks_before(ov, oi, v, i)) { v = ov; i = oi; }
}

// Wave-wide arg-max under ranks_before; every lane gets the winner.  Inside
// each row of 16 lanes by DPP lane permutations (swap neighbours, swap pairs,
// mirror the half-rows, mirror the row: after each step every lane holds the
// best of a group twice as large), then across the four rows by two
// shuffles.  ranks_before is a total order (value descending, index
// ascending), so the winner does not depend on the reduction order.
MOE_DEV void wave_argmax(float &v, int &i)
{
    argmax_dpp_step<0xB1>(v, i);   // quad_perm(1, 0, 3, 2)
    argmax_dpp_step<0x4E>(v, i);   // quad_perm(2, 3, 0, 1)
    argmax_dpp_step<0x141>(v, i);  // row_half_mirror
    argmax_dpp_step<0x140>(v, i);  // row_mirror
#pragma unroll
    for (int off = 16; off <= 32; off <<= 1) {
        float ov = __shfl_xor(v, off, 64);
        int oi = __shfl_xor(i, off, 64);
        if (ranks_before(ov, oi, v, i)) { v = ov; i = oi; }
    }
}

MOE_DEV float wave_sum(float v)
{
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}

MOE_DEV float wave_max(float v)
{
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
    return v;
}

__host__ __device__ inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// ---------------------------------------------------------------------------
// Launch functions (host side, one per kernel family).  All enqueue on
// `stream` and return hipGetLastError() of the launch.
// ---------------------------------------------------------------------------

// fill int32 / fp32 buffers with a value (small kernels instead of memset,
// so that captured graphs hold only kernel nodes)
hipError_t launch_fill_i32(int32_t *p, int64_t n, int32_t v, hipStream_t s);
hipError_t launch_fill_f32(float *p, int64_t n, float v, hipStream_t s);

// Router GEMMs on bf16 MFMA with exact three-way bf16 splits of the fp32
// operands (fp32-accurate products, fp32 accumulation).  The workspace sizes
// are what the two calls need (device memory, 256-byte aligned).
size_t router_ws_bytes_fwd(int64_t T, int32_t E, int32_t H);
size_t router_ws_bytes_bwd(int64_t T, int32_t E, int32_t H);
// logits[T, E] = x[T, H] . Wr[E, H]^T
hipError_t launch_router_logits(int64_t T, int32_t E, int32_t H, const uint16_t *x, const float *Wr,
                                float *logits, void *ws, hipStream_t s);
// dx[T, H] += dl[T, E] . Wr[E, H];  dWr[E, H] = dl^T . x  (if dWr)
hipError_t launch_router_grads(int64_t T, int32_t E, int32_t H, const float *dl, const uint16_t *x,
                               const float *Wr, float *dx, float *dWr, void *ws, hipStream_t s);

// router: selection + weights + counts + aux partial sums; then aux finalize
struct RouterArgs {
    int64_t T;
    int32_t E, k, G, kg, score, renorm, even;
    float scale, aux_coeff;
    const float *logits, *bias;
    float *sel, *topk_w;
    int32_t *topk_idx, *counts;
    float *aux, *prob_part;  // prob_part [nblk, E]: per-block aux column sums
    int32_t *cnt_part;       // [nblk, E]: per-block expert counts
    float *prob_slice;       // [aux_slices, E]: the partials summed in slices
    int32_t *cnt_slice;      // [aux_slices, E]
};
int64_t router_blocks(int64_t T);
int64_t aux_slices(int64_t T);
hipError_t launch_router(const RouterArgs &a, hipStream_t s);

// permute: histogram / scan / stable scatter
int64_t permute_chunks(int64_t M);
hipError_t launch_permute(int64_t M, int32_t E, const int32_t *idx, int32_t *counts,
                          int32_t *offsets, int32_t *row_map, int32_t *pos,
                          int32_t *chunk_hist, hipStream_t s);
// the same with expert ids checked: a slot whose expert is outside [0, E) is
// placed nowhere (pos = -1; row_map holds -1 past the placed rows) and
// counted in *n_bad (device); chunk_hist has E + 1 rows of permute_chunks(M)
hipError_t launch_permute_checked(int64_t M, int32_t E, const int32_t *idx, int32_t *counts,
                                  int32_t *offsets, int32_t *row_map, int32_t *pos,
                                  int32_t *chunk_hist, int32_t *n_bad, hipStream_t s);

// schedule: m-tile prefix sums for the grouped GEMMs and experts sorted by
// count (descending, ties -> lower index) for the weight-gradient GEMMs
struct Sched {
    int32_t *mt_off256;  // [E+1]
    int32_t *mt_off128;  // [E+1]
    int32_t *order;      // [E+1]; order[E] = number of non-empty experts
    int32_t *mt_a;       // [E+1] mixed m-tiling: 256-row tiles (decode_mtile_mixed)
    int32_t *mt_b;       // [E+1] mixed m-tiling: 257..320-row tiles
};

// Mixed m-tiling of an expert with c rows: its 257..320-row tile count (0 or
// 1: c > 256 leaving 1..64 rows past a multiple of 256) and its 256-row one.
MOE_DEV int mixed_tail_tiles(int c) { return c > 256 && (c & 255) >= 1 && (c & 255) <= 64 ? 1 : 0; }
MOE_DEV int mixed_head_tiles(int c) { return mixed_tail_tiles(c) ? c / 256 - 1 : (c + 255) / 256; }
hipError_t launch_schedule(int32_t E, const int32_t *counts, const Sched &sc, hipStream_t s);

struct GemmArgs {
    int64_t T, M;
    int32_t E, k, H, I;
    const int32_t *counts, *offsets, *row_map;
    const float *topk_w;
    const uint16_t *x, *dy, *w1, *w2;
    const float *wrow;         // per sorted row: topk_w of its slot
    uint16_t *h, *a, *dh;
    float *o, *dw_part, *dxp;
    // when set, dgrad1 writes its per-row partials of dx here in bf16
    // instead of to dxp (the fused backward; the per-op entry point keeps fp32)
    uint16_t *dxp_bf16;
    // when set, GEMM2 writes the expert outputs here in bf16 instead of to o
    // (the fused forward with bf16 intermediates; the per-op entry keeps fp32)
    uint16_t *o_bf16;
    void *dW1, *dW2;
    int32_t dw_bf16, dw_acc;
    Sched sched;
    // MXFP8 forward: MX matrices (codes, scales; layout in mxfmt.h) of x
    // [T, Hp], w1 [E*2I, Hp], w2 [E*H, Ip] and a [M, Ip]; Hp, Ip = H, I
    // rounded up to 128
    const uint8_t *xq, *xs, *w1q, *w1s, *w2q, *w2s;
    uint8_t *aq, *as_;
    int64_t Hp, Ip;
    // MXFP8 backward: MX matrices of dy [T, Hp], dh [M, 2Ip], w2^T per expert
    // [E*I, Hp] and w1^T per expert [E*H, 2Ip]; for the weight gradients, the
    // per-expert MX matrices of the two operands transposed (segA: rows of
    // dW, segB: its columns; expert e at R * 132 * mt_off128[e] bytes, R the
    // operand's row count, K = its routed rows padded to 128)
    const uint8_t *dyq, *dys, *dhq, *dhs, *w2cq, *w2cs, *w1cq, *w1cs;
    const uint8_t *segA, *segB;
    // bf16 weight gradients: each expert's rows of the two operands
    // transposed into K-major 128-deep chunks, [R][128] and [C][128] each,
    // expert e's first at R (C) * 128 * mt_off128[e] elements (see
    // launch_transpose_segments)
    const uint16_t *tA, *tB;
    // split intermediates (MOE_PRECISION_SPLIT): the bf16 remainders of h, a
    // and dh (v = hi + lo), and the weight gradients' second operand halves:
    // tA_lo (dh_lo, wgrad1) or tB_lo (the remainder of w*a, wgrad2), laid out
    // as tA / tB; the other operand's chunks serve both halves
    int32_t split;
    uint16_t *h_lo, *a_lo, *dh_lo;
    const uint16_t *tA_lo, *tB_lo;
};
int32_t dgrad2_cols(int32_t I);
hipError_t launch_grouped_gemm(int32_t op, const GemmArgs &g, hipStream_t s);
// MXFP8: quantise a bf16 matrix [rows, K] (K % 32 == 0) into the MX matrix at
// dst (codes [rows, Kp] then scales [rows, Kp/32]); the forward GEMMs on MX
// operands (op MOE_GEMM_UP_SWIGLU or MOE_GEMM_DOWN)
hipError_t launch_mx_quantize(const uint16_t *src, int64_t rows, int64_t K, uint8_t *dst,
                              hipStream_t s);
hipError_t launch_mx_gemm(int32_t op, const GemmArgs &g, hipStream_t s);
// MXFP8: both forms of src [B, R, C] from one read: dst_f the MX matrix of
// [B*R, C] (along C), dst_t that of the stacked transposes [B*C, R] (along R)
// (R % 32 == 0, C % 32 == 0)
hipError_t launch_mx_quantize_both(const uint16_t *src, int64_t B, int64_t R, int64_t C,
                                   uint8_t *dst_f, uint8_t *dst_t, hipStream_t s);
// MXFP8: the transposes of column segments of a bf16 matrix src (row stride
// C elements, C % 64 == 0) as MX matrices along the segment's rows.  Either
// nseg uniform segments of R rows, written as one MX matrix [nseg*C, Rp]
// (offsets == NULL), or the E expert segments of sorted rows given by
// offsets / mt128 (the 128-row m-tile prefix sums), each its own MX matrix
// [C, Kp_e] at C * 132 * mt128[e] bytes; gather (optional) maps a sorted row
// r to source row gather[r] / gk, and rw (optional) scales sorted row r by
// rw[r] first (the product rounded to bf16).  max_chunks bounds the 128-row
// chunks.
// src_lo (optional, bf16 transposer only): a second source of the same shape
// whose values are added to src's in fp32 before the scaling (a hi + lo
// pair); lo_part (bf16 transposer only): 0 stores bf16(v), 1 stores the
// remainder bf16(v - bf16(v)).
struct ColQuant {
    const uint16_t *src;
    int64_t C;
    const int32_t *gather;
    int32_t gk;
    const float *rw;
    int32_t nseg;
    int64_t R;
    const int32_t *offsets, *mt128;
    uint8_t *dst;
    const uint16_t *src_lo;
    int32_t lo_part;
};
hipError_t launch_mx_quantize_cols(const ColQuant &q, int64_t max_chunks, hipStream_t s);
// bf16: the same expert segments (offsets / mt128 mode) transposed without
// quantising, into dst in 128-row chunks: chunk j of expert e is [C][128]
// at C * 128 * (mt128[e] + j) elements, rows past its count zero.
hipError_t launch_transpose_segments(const ColQuant &q, int64_t max_chunks, uint16_t *dst,
                                     hipStream_t s);
// zero the weight gradient of every expert without rows (overwrite mode)
hipError_t launch_zero_empty(int32_t E, int64_t per_expert, const int32_t *counts, void *dW,
                             int32_t bf16, hipStream_t s);

// wrow[r] = topk_w[row_map[r]], the routing weight of each sorted row
hipError_t launch_row_weights(int64_t M, const int32_t *row_map, const float *topk_w, float *wrow,
                              hipStream_t s);

// elementwise / reductions
hipError_t launch_combine(int64_t T, int32_t k, int32_t H, const float *o, const float *w,
                          const int32_t *pos, float *y, hipStream_t s);
// the same with bf16 rows o (the backward's un-permute of bf16 dx partials)
hipError_t launch_combine_bf16(int64_t T, int32_t k, int32_t H, const uint16_t *o, const float *w,
                               const int32_t *pos, float *y, hipStream_t s);
hipError_t launch_swiglu(int32_t backward, int64_t M, int32_t I, const uint16_t *h,
                         const float *da, uint16_t *out, hipStream_t s);
struct RouterBwdArgs {
    int64_t T;
    int32_t E, k, score, renorm, ncols;
    float scale, aux_coeff;
    const float *logits, *topk_w, *dw_part, *d_aux;
    const int32_t *topk_idx, *counts, *pos;
    float *dlogits;
};
hipError_t launch_router_bwd(const RouterBwdArgs &a, hipStream_t s);

}  // namespace moe
