// Grouped bf16 GEMMs of the MoE expert path on gfx950 MFMA
// (v_mfma_f32_32x32x16_bf16, fp32 accumulation).
//
// Every GEMM is written as C[r, c] = sum_k A(r, k) * B(c, k), staged
// through double-buffered LDS tiles 64 deep in k that are filled by direct
// global->LDS copies.  Operands whose k index is contiguous in memory are
// copied row by row into [rows][64] tiles (KLoad) and read with 16-byte LDS
// reads; operands that are contiguous along the output dimension instead
// (the weights in dgrad, both operands in wgrad) are copied in their own
// layout into [64][rows] tiles (NLoad) and read with gfx950's transposing
// LDS reads.  16-byte chunks are XOR-swizzled so that fragment reads are free
// of bank conflicts.  Token rows are gathered through row_map while loading:
// dispatch is fused into the load, as the MegaMoE page (intro) fuses it into
// the first grouped GEMM.
//
// Scheduling: forward and dgrad GEMMs tile the sorted rows of each expert
// (M-grouped), in 256-row tiles except that an expert's last tile may hold
// 257..320 rows (the mixed m-tiling, decode_mtile_mixed); the per-expert
// m-tile prefix sums live on the device, the grid is sized from a host-side
// upper bound and surplus blocks exit.  The
// weight-gradient GEMMs tile the [rows x cols] output of each expert that has
// rows and loop over those rows (K-grouped), longest experts first; experts
// without rows are zeroed by a separate fill (overwrite) or left untouched
// (accumulate).  Block
// indices are remapped so that each of the 8 XCDs works on a contiguous run
// of tiles (neighbouring tiles share operand panels in that XCD's L2).
#include "bwd_epi.h"
#include "segtile.h"
#include "swiglu_epi.h"

namespace moe {

// Weight-gradient tile walk: tiles dealt to the XCDs in chunks of
// WGRAD_XCD_CHUNK, and inside an expert groups of WGRAD_GR row tiles sweep
// the column tiles (compile-time overridable for tuning builds).
#ifndef MOE_WGRAD_XCD_CHUNK
#define MOE_WGRAD_XCD_CHUNK 16
#endif
#ifndef MOE_WGRAD_GR
#define MOE_WGRAD_GR 4
#endif
constexpr int64_t WGRAD_XCD_CHUNK = MOE_WGRAD_XCD_CHUNK;
constexpr int WGRAD_GR = MOE_WGRAD_GR;

int64_t mgrid_blocks(int64_t M, int E, int BM, int nN)
{
    int64_t mt = M / BM + (M < E ? M : E) + 1;
    return grid_for(mt * nN);
}


// =========================================================================
// GEMM1 + SwiGLU:  h[r, n] = x[tok(r)] . w1[e, n, :],  a = silu(g) * u
// B tile rows: wave column wn covers gate columns i0 + wn*WN/2 + [0, WN/2)
// and the matching up columns, so each lane holds g and u of the same (r, i).
// =========================================================================
template <class C, bool SPLIT>
MOE_DEV void up_swiglu_tile(const GemmArgs &g, const MTile &t, lds_t *lds)
{
    const int I = g.I, H = g.H;
    const int tid = threadIdx.x, lane0 = tid & 63, wave0 = wave_uniform_id();
    KLoad<C::BM, C::NT> la;
    KLoad<C::BN, C::NT> lb;
    la.init(g.x, wave0);
    const uint16_t *w1e = g.w1 + (int64_t)t.e * 2 * I * H;
    lb.init(w1e, wave0);
    const int64_t i0 = (int64_t)t.nt * (C::BN / 2);
#pragma unroll
    for (int q = 0; q < la.NI; ++q) {
        int64_t m = t.m0 + la.row(q, lane0);
        if (m >= t.seg_end) m = t.seg_end - 1;
        la.set(q, lane0, (uint32_t)((g.row_map[m] / g.k) * (int64_t)H * 2));
    }
#pragma unroll
    for (int q = 0; q < lb.NI; ++q) {
        int r = lb.row(q, lane0);
        int wn = r / C::WN, qq = r % C::WN;
        int half = C::WN / 2;
        int64_t i = i0 + wn * half + (qq < half ? qq : qq - half);
        if (i >= I) i = I - 1;
        int64_t n = qq < half ? i : I + i;
        lb.set(q, lane0, (uint32_t)(n * H * 2));
    }
    Acc<C> acc;
    mainloop<C, false, false, false>(lds, H, la, lb, acc);

    swiglu_epilogue<C, false, SPLIT>(acc, lds, t, i0, I, g.h, g.a, nullptr, nullptr, 0, g.h_lo,
                                     g.a_lo);
}

// =========================================================================
// GEMM2:  o[r, c] = a[r] . w2[e, c, :]   (fp32 out)
// SPLIT: a is the pair a + a_lo, so the k loop runs twice over I: stages
// 0 .. I/64-1 read a, the next I/64 read a_lo, both against the same w2.
// =========================================================================
template <class C, bool SPLIT, bool BF16OUT = false>
MOE_DEV void down_tile(const GemmArgs &g, const MTile &t, lds_t *lds)
{
    const int I = g.I, H = g.H;
    const int tid = threadIdx.x, lane0 = tid & 63, wave0 = wave_uniform_id();
    KLoad<C::BM, C::NT> la;
    KLoad<C::BN, C::NT> lb;
    la.init(g.a, wave0);
    const uint16_t *w2e = g.w2 + (int64_t)t.e * H * I;
    lb.init(w2e, wave0);
#pragma unroll
    for (int q = 0; q < la.NI; ++q) {
        int64_t m = t.m0 + la.row(q, lane0);
        if (m >= t.seg_end) m = t.seg_end - 1;
        la.set(q, lane0, (uint32_t)(m * I * 2));
    }
    const int64_t n0 = (int64_t)t.nt * C::BN;
#pragma unroll
    for (int q = 0; q < lb.NI; ++q) {
        int64_t n = n0 + lb.row(q, lane0);
        if (n >= H) n = H - 1;
        lb.set(q, lane0, (uint32_t)(n * I * 2));
    }
    Acc<C> acc;
    if constexpr (SPLIT) {
        const int nI = I / BK;  // I % 64 == 0 (moe_check_config)
        const char *alo = (const char *)g.a_lo;
        pipeline<C, false, false, KLoad<C::BM, C::NT>::NI, KLoad<C::BN, C::NT>::NI>(
            lds, 0, 2 * nI,
            [&](int q, int st, lds_t *As) {
                const bool lo = st >= nI;
                la.issue_one(q, As, (int64_t)(lo ? st - nI : st) * BK, BK, lo ? alo : la.base);
            },
            [&](int q, int st, lds_t *Bs) {
                lb.issue_one(q, Bs, (int64_t)(st >= nI ? st - nI : st) * BK, BK, lb.base);
            },
            [](int, lds_t *, lds_t *) {}, acc);
    } else {
        mainloop<C, false, false, false>(lds, I, la, lb, acc);
    }
    if (BF16OUT || g.o_bf16) store_tile_f32<C>(acc, lds, g.o_bf16, t.m0, t.seg_end, n0, H);
    else store_tile_f32<C>(acc, lds, g.o, t.m0, t.seg_end, n0, H);
}

// =========================================================================
// dgrad of GEMM2 + row-dot + SwiGLU backward:
//   dA'[r, i] = dy[tok(r)] . w2[e, :, i];  dw_part[r, nt] = sum_i dA' a
//   dA = topk_w * dA';  dh = (dA u sig(g)(1 + g(1 - sig(g))) | dA silu(g))
// =========================================================================
template <class C, bool SPLIT>
MOE_DEV void down_dgrad_tile(const GemmArgs &g, const MTile &t, lds_t *lds)
{
    const int I = g.I, H = g.H;
    const int nN = (int)ceil_div(I, C::BN);
    const int tid = threadIdx.x, lane0 = tid & 63, wave0 = wave_uniform_id();
    KLoad<C::BM, C::NT> la;
    NLoad<C::BN, C::NT> lb;
    la.init(g.dy, wave0);
#pragma unroll
    for (int q = 0; q < la.NI; ++q) {
        int64_t m = t.m0 + la.row(q, lane0);
        if (m >= t.seg_end) m = t.seg_end - 1;
        la.set(q, lane0, (uint32_t)((g.row_map[m] / g.k) * (int64_t)H * 2));
    }
    const uint16_t *w2e = g.w2 + (int64_t)t.e * H * I;
    const int64_t n0 = (int64_t)t.nt * C::BN;
    // B(n = i, k = hh) = w2[e, hh, i]: k-row hh starts at w2e + hh*I
    lb.init(w2e, I, n0, I, wave0, lane0);
    Acc<C> acc;
    // a segment's last m-tile may be part-filled: the partial main loop skips
    // the A copies and MFMAs of its empty rows (3-4% on the dgrad GEMMs
    // under uniform routing; it does not pay in GEMM1 and GEMM2).  A 320-row
    // tile (257..320 rows) runs the full loop: its rows past the segment
    // repeat the last one.
    const int64_t rows = t.seg_end - t.m0;
    if (rows >= C::BM || C::BM == 320) mainloop<C, false, true, false>(lds, H, la, lb, acc);
    else mainloop<C, false, true, false, C::BM != 320>(lds, H, la, lb, acc, (int)rows);
    // the split form loads twice the rows' data, and the 320-row tile has
    // 32 more accumulators: half the rows a batch
    dgrad2_epilogue<C, SPLIT || C::BM == 320 ? 2 : 4, SPLIT>(acc, lds, t, n0, nN, I, g.h, g.a, g.wrow, g.dh,
                                             g.dw_part, g.h_lo, g.a_lo, g.dh_lo);
}

// =========================================================================
// dgrad of GEMM1:  dxp[r, c] = dh[r] . w1[e, :, c]   (fp32 out, or bf16 to
// g.dxp_bf16)
// =========================================================================
template <class C, bool BF16OUT = false>
MOE_DEV void up_dgrad_tile(const GemmArgs &g, const MTile &t, lds_t *lds)
{
    const int I = g.I, H = g.H;
    const int tid = threadIdx.x, lane0 = tid & 63, wave0 = wave_uniform_id();
    KLoad<C::BM, C::NT> la;
    NLoad<C::BN, C::NT> lb;
    la.init(g.dh, wave0);
#pragma unroll
    for (int q = 0; q < la.NI; ++q) {
        int64_t m = t.m0 + la.row(q, lane0);
        if (m >= t.seg_end) m = t.seg_end - 1;
        la.set(q, lane0, (uint32_t)(m * 2 * I * 2));
    }
    const uint16_t *w1e = g.w1 + (int64_t)t.e * 2 * I * H;
    const int64_t n0 = (int64_t)t.nt * C::BN;
    // B(n = hh, k = nn) = w1[e, nn, hh]: k-row nn starts at w1e + nn*H
    lb.init(w1e, H, n0, H, wave0, lane0);
    Acc<C> acc;
    const int64_t rows = t.seg_end - t.m0;  // part-filled last m-tile: as in down_dgrad_tile
    if (rows >= C::BM || C::BM == 320) mainloop<C, false, true, false>(lds, 2 * I, la, lb, acc);
    else mainloop<C, false, true, false, C::BM != 320>(lds, 2 * I, la, lb, acc, (int)rows);
    if (BF16OUT || g.dxp_bf16) store_tile_f32<C>(acc, lds, g.dxp_bf16, t.m0, t.seg_end, n0, H);
    else store_tile_f32<C>(acc, lds, g.dxp, t.m0, t.seg_end, n0, H);
}

// =========================================================================
// Kernels of the M-grouped GEMMs.  Single-shape kernels: 256-row tiles (or
// 128-row ones) of every row (mt_off256 / mt_off128).  Mixed kernels: both
// shapes of the mixed m-tiling in one launch (decode_mtile_mixed), each
// block one tile of either shape; their GEMM2 and dgrad1 store bf16 only
// (the forms the layer uses).  The two shapes' code sits side by side in
// one kernel; the 256-row path compiles as in the single-shape kernel
// (no spills) because the decoded tile is forced into scalar registers.
// =========================================================================
template <class C>
MOE_DEV bool decode_single(const GemmArgs &g, int nN, MTile &t)
{
    return decode_mtile<C::BM>(blockIdx.x, C::BM == 256 ? g.sched.mt_off256 : g.sched.mt_off128,
                               g.offsets, g.E, nN, t);
}

template <class C0, class C1>
struct Mixed {
    static_assert(C0::NT == C1::NT && C0::BM == 256 && C1::BM == 320 && C0::BN == C1::BN,
                  "256- and 320-row shapes of one n-tiling");
    static constexpr int NT = C0::NT;
    static constexpr int LDS_BYTES = C0::LDS_BYTES > C1::LDS_BYTES ? C0::LDS_BYTES : C1::LDS_BYTES;
};

#define MOE_MIXED_KERNEL(NAME, NCOLS, ...)                                                     \
    template <class M, class C0, class C1>                                                     \
    __global__ __launch_bounds__(M::NT) void NAME##_mixed(GemmArgs g)                          \
    {                                                                                          \
        __shared__ __attribute__((aligned(16))) char lds_raw[M::LDS_BYTES];                    \
        MTile t;                                                                               \
        const int cls = decode_mtile_mixed(blockIdx.x, g.sched.mt_a, g.sched.mt_b, g.offsets, \
                                           g.E, (int)(NCOLS), t);                              \
        if (cls == 0) NAME##_tile<C0, __VA_ARGS__>(g, t, (lds_t *)lds_raw);                    \
        else if (cls == 1) NAME##_tile<C1, __VA_ARGS__>(g, t, (lds_t *)lds_raw);               \
    }

template <class C, bool SPLIT>
__global__ __launch_bounds__(C::NT) void k_up_swiglu(GemmArgs g)
{
    __shared__ __attribute__((aligned(16))) char lds_raw[C::LDS_BYTES];
    MTile t;
    if (decode_single<C>(g, (int)ceil_div(g.I, C::BN / 2), t))
        up_swiglu_tile<C, SPLIT>(g, t, (lds_t *)lds_raw);
}
MOE_MIXED_KERNEL(up_swiglu, ceil_div(g.I, C0::BN / 2), false)

template <class C, bool SPLIT>
__global__ __launch_bounds__(C::NT) void k_down(GemmArgs g)
{
    __shared__ __attribute__((aligned(16))) char lds_raw[C::LDS_BYTES];
    MTile t;
    if (decode_single<C>(g, (int)ceil_div(g.H, C::BN), t)) down_tile<C, SPLIT>(g, t, (lds_t *)lds_raw);
}
MOE_MIXED_KERNEL(down, ceil_div(g.H, C0::BN), false, true)

template <class C, bool SPLIT>
__global__ __launch_bounds__(C::NT) void k_down_dgrad(GemmArgs g)
{
    __shared__ __attribute__((aligned(16))) char lds_raw[C::LDS_BYTES];
    MTile t;
    if (decode_single<C>(g, (int)ceil_div(g.I, C::BN), t))
        down_dgrad_tile<C, SPLIT>(g, t, (lds_t *)lds_raw);
}
MOE_MIXED_KERNEL(down_dgrad, ceil_div(g.I, C0::BN), false)

template <class C>
__global__ __launch_bounds__(C::NT) void k_up_dgrad(GemmArgs g)
{
    __shared__ __attribute__((aligned(16))) char lds_raw[C::LDS_BYTES];
    MTile t;
    if (decode_single<C>(g, (int)ceil_div(g.H, C::BN), t)) up_dgrad_tile<C>(g, t, (lds_t *)lds_raw);
}
MOE_MIXED_KERNEL(up_dgrad, ceil_div(g.H, C0::BN), true)

// =========================================================================
// Weight-gradient operands: the rows of each expert, transposed into a
// K-major matrix in 128-deep chunks: chunk j of expert e is [C][128]
// (element (c, k) at c * 128 + k; rows past the expert's count zero), at
// C * 128 * (mt128[e] + j) elements.  A block takes one chunk's 128 rows x
// NCT*64 columns through LDS (rows gathered and scaled on the way when
// asked; each source row gives NCT*128 contiguous bytes; NCT = 4 where the
// column count allows) and writes NCT*16 contiguous KB.  Four lanes share an
// output row (one column of the source): lane b of the four holds rows
// 32 i + 8 b .. 32 i + 8 b + 7 for i = 0..3, so each 16-byte store of a wave
// writes sixteen 64-byte runs of one 4 KB span.  The LDS rows are padded to
// 66 elements so that the column reads of the four lanes fall in different
// banks.
// =========================================================================
template <int NCT, bool SPLIT>
__global__ __launch_bounds__(256) void k_transpose_segments(ColQuant q, uint16_t *dst)
{
    __shared__ __attribute__((aligned(16))) uint16_t tile[NCT * SEG_ROWS][66];
    const int nct = (int)(q.C / (64 * NCT));
    const int ct = (blockIdx.x % nct) * NCT;
    __shared__ int32_t mt_s[SEG_MAX_E + 1];
    seg_stage_table(q, mt_s);
    __syncthreads();
    SegPos p;
    if (!seg_locate(q, mt_s, blockIdx.x / nct, p)) return;
    seg_load_tile<66, NCT, SPLIT>(q, p, ct, tile);
    __syncthreads();
    const int b = threadIdx.x & 3, c = threadIdx.x >> 2;
#pragma unroll
    for (int t = 0; t < NCT; ++t) {
        uint16_t *o = dst + q.C * SEG_ROWS * (p.chunk0 + p.j) + ((ct + t) * 64 + c) * SEG_ROWS;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r0 = 32 * i + 8 * b;
            uint32_t z[4];
#pragma unroll
            for (int e = 0; e < 4; ++e)
                z[e] = (uint32_t)tile[t * SEG_ROWS + r0 + 2 * e][c] |
                       ((uint32_t)tile[t * SEG_ROWS + r0 + 2 * e + 1][c] << 16);
            *(u32x4_t *)(o + r0) = u32x4_t{z[0], z[1], z[2], z[3]};
        }
    }
}

hipError_t launch_transpose_segments(const ColQuant &q, int64_t max_chunks, uint16_t *dst,
                                     hipStream_t s)
{
    // four (else two) column tiles a block where the columns allow it
    const int nct = (q.C / 64) % 4 == 0 ? 4 : (q.C / 64) % 2 == 0 ? 2 : 1;
    const int64_t blocks = max_chunks * (q.C / (64 * nct));
    if (blocks <= 0) return hipSuccess;
    const bool split = q.src_lo != nullptr || q.lo_part != 0;
    const dim3 grid((unsigned)blocks), block(256);
    if (nct == 4) {
        if (split) hipLaunchKernelGGL((k_transpose_segments<4, true>), grid, block, 0, s, q, dst);
        else hipLaunchKernelGGL((k_transpose_segments<4, false>), grid, block, 0, s, q, dst);
    } else if (nct == 2) {
        if (split) hipLaunchKernelGGL((k_transpose_segments<2, true>), grid, block, 0, s, q, dst);
        else hipLaunchKernelGGL((k_transpose_segments<2, false>), grid, block, 0, s, q, dst);
    } else {
        if (split) hipLaunchKernelGGL((k_transpose_segments<1, true>), grid, block, 0, s, q, dst);
        else hipLaunchKernelGGL((k_transpose_segments<1, false>), grid, block, 0, s, q, dst);
    }
    return hipGetLastError();
}

// =========================================================================
// Weight gradients (K-grouped over each expert's rows).
//   DOWN:  dW2[e, hh, i] (+)= sum_r topk_w(r) dy[tok(r), hh] a[r, i]
//   UP:    dW1[e, n, hh] (+)= sum_r dh[r, n] x[tok(r), hh]
// Output tile rows come from operand A (tA: w*dy or dh), columns from
// operand B (tB: a or x), both the expert's K-major chunks written by
// k_transpose_segments, so the tile is the forward one: row-contiguous
// copies and 16-byte fragment reads, no index loads, no partial stage.
// Stage s (64 k) of a row r lies at byte (s/2) * rows * 256 + r * 256 +
// (s%2) * 128 of the expert's area.
// SPLIT: the k loop runs twice over the expert's rows; the second pass reads
// the remainder half of the split operand (UP: tA_lo, the remainder of dh;
// DOWN: tB_lo, the remainder of w*a) and the same chunks of the other one.
// =========================================================================
template <class C, bool UP, bool SPLIT>
__global__ __launch_bounds__(C::NT) void k_wgrad(GemmArgs g)
{
    __shared__ __attribute__((aligned(16))) char lds_raw[C::LDS_BYTES];
    lds_t *lds = (lds_t *)lds_raw;
    const int I = g.I, H = g.H;
    const int R = UP ? 2 * I : H;   // output rows
    const int Cc = UP ? H : I;      // output cols
    const int nR = (int)ceil_div(R, C::BM), nC = (int)ceil_div(Cc, C::BN);
    const int64_t tpe = (int64_t)nR * nC;
    const int64_t total = (int64_t)g.sched.order[g.E] * tpe;  // non-empty experts only
    const int64_t L = xcd_remap<WGRAD_XCD_CHUNK>(blockIdx.x, total);
    if (L < 0) return;
    const int e = g.sched.order[L / tpe];
    // inside one expert: groups of GR row tiles sweep all column tiles, so
    // the tiles running together share A and B panels in L2
    constexpr int GR = WGRAD_GR;
    const int64_t rest = L % tpe;
    const int64_t grp = rest / ((int64_t)GR * nC);
    const int64_t first = grp * GR;
    const int64_t gr = nR - first < GR ? nR - first : GR;
    const int64_t in = rest - grp * (int64_t)GR * nC;
    const int rt = (int)(first + in % gr), ct = (int)(in / gr);
    const int64_t r0 = (int64_t)rt * C::BM, c0 = (int64_t)ct * C::BN;
    const int lane = threadIdx.x & 63, wave = wave_uniform_id();
    const int32_t *mt = g.sched.mt_off128;
    const int nst = 2 * (mt[e + 1] - mt[e]);  // 64-k stages
    KLoad<C::BM, C::NT> la;
    KLoad<C::BN, C::NT> lb;
    la.init(g.tA + (int64_t)R * SEG_ROWS * mt[e], wave);
    lb.init(g.tB + (int64_t)Cc * SEG_ROWS * mt[e], wave);
#pragma unroll
    for (int q = 0; q < la.NI; ++q) {
        int64_t r = r0 + la.row(q, lane);
        if (r >= R) r = R - 1;
        la.set(q, lane, (uint32_t)(r * SEG_ROWS * 2));
    }
#pragma unroll
    for (int q = 0; q < lb.NI; ++q) {
        int64_t n = c0 + lb.row(q, lane);
        if (n >= Cc) n = Cc - 1;
        lb.set(q, lane, (uint32_t)(n * SEG_ROWS * 2));
    }
    auto stage_off = [](int s, int64_t rows) { return (int64_t)(s >> 1) * rows * 256 + (s & 1) * 128; };
    Acc<C> acc;
    if constexpr (SPLIT) {
        const char *alo = UP ? (const char *)(g.tA_lo + (int64_t)R * SEG_ROWS * mt[e]) : la.base;
        const char *blo = UP ? lb.base : (const char *)(g.tB_lo + (int64_t)Cc * SEG_ROWS * mt[e]);
        pipeline<C, false, false, KLoad<C::BM, C::NT>::NI, KLoad<C::BN, C::NT>::NI>(
            lds, 0, 2 * nst,
            [&](int q, int s, lds_t *As) {
                const bool lo = s >= nst;
                la.issue_one(q, As, 0, BK, (lo ? alo : la.base) + stage_off(lo ? s - nst : s, R));
            },
            [&](int q, int s, lds_t *Bs) {
                const bool lo = s >= nst;
                lb.issue_one(q, Bs, 0, BK, (lo ? blo : lb.base) + stage_off(lo ? s - nst : s, Cc));
            },
            [](int, lds_t *, lds_t *) {}, acc);
    } else {
        pipeline<C, false, false, KLoad<C::BM, C::NT>::NI, KLoad<C::BN, C::NT>::NI>(
            lds, 0, nst,
            [&](int q, int s, lds_t *As) { la.issue_one(q, As, 0, BK, la.base + stage_off(s, R)); },
            [&](int q, int s, lds_t *Bs) { lb.issue_one(q, Bs, 0, BK, lb.base + stage_off(s, Cc)); },
            [](int, lds_t *, lds_t *) {}, acc);
    }
    wgrad_epilogue<C, 8>(acc, lds, r0, c0, R, Cc, (int64_t)e * R * Cc, UP ? g.dW1 : g.dW2, g.dw_acc,
                      g.dw_bf16);
}

// ---------------------------------------------------------- empty experts ----
// dW[e] = 0 for every expert e without rows; grid (chunks, E), 16-byte stores.
__global__ __launch_bounds__(256) void k_zero_empty(int64_t per_expert, const int32_t *counts,
                                                    void *dW, int32_t bf16)
{
    const int e = blockIdx.y;
    if (counts[e] != 0) return;
    const int64_t bytes = per_expert * (bf16 ? 2 : 4);
    u32x4_t *p = (u32x4_t *)((char *)dW + (int64_t)e * bytes);
    const int64_t n = bytes / 16;
    const u32x4_t z = {0u, 0u, 0u, 0u};
    for (int64_t q = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; q < n;
         q += (int64_t)gridDim.x * blockDim.x)
        p[q] = z;
}

hipError_t launch_zero_empty(int32_t E, int64_t per_expert, const int32_t *counts, void *dW,
                             int32_t bf16, hipStream_t s)
{
    dim3 grid(64, (unsigned)E);
    k_zero_empty<<<grid, 256, 0, s>>>(per_expert, counts, dW, bf16);
    return hipGetLastError();
}

// ----------------------------------------------------------------- launch ----
// 256x256 output tiles computed by 8 waves (two a SIMD).  Wave tiles are
// 128 rows x 64 columns where the column operand is read with transposing LDS
// reads (down_dgrad, up_dgrad: the transposed operand then supplies the
// smaller fragment count), for up_swiglu and for the weight gradients.  GEMM2
// (down), whose epilogue is a plain fp32 store, runs four waves of 128 x 128
// (one a SIMD, accumulators in AGPRs): a third fewer fragment bytes read
// from LDS, +3% (the other ops lose on it).  Every op takes three B stage
// buffers (all 160 KB of LDS): the B copies of a stage get two stages to
// land.
// The mixed m-tiling's 257..320-row tiles run eight waves of 160 x 64 with
// two B stage buffers (2 x 40 KB of A, 2 x 32 KB of B), A fragments refilled
// in place.  In the mixed kernels GEMM2's 256-row tiles take eight waves (the
// two shapes share a launch); its split and fp32-output forms keep four.
using Tall = TileCfg<256, 256, 128, 64, 3>;
using Quad = TileCfg<256, 256, 128, 128, 3>;
using Tall320 = TileCfg<320, 256, 160, 64, 2>;
using MixT = Mixed<Tall, Tall320>;
using UpCfg = Tall;
using DownCfg = Quad;
using DownDgradCfg = Tall;
using UpDgradCfg = Tall;
using WgradCfg = Tall;

int32_t dgrad2_cols(int32_t I) { return (int32_t)ceil_div(I, DownDgradCfg::BN); }

template <class K>
static hipError_t launch_k(K kern, int64_t blocks, const GemmArgs &g, hipStream_t s, int nt)
{
    if (blocks <= 0) return hipSuccess;
    kern<<<(unsigned)blocks, nt, 0, s>>>(g);
    return hipGetLastError();
}

hipError_t launch_grouped_gemm(int32_t op, const GemmArgs &g, hipStream_t s)
{
    const bool sp = g.split != 0;
    switch (op) {
    // bf16 intermediates: the mixed m-tiling (GEMM2 and dgrad1 when they store
    // bf16); otherwise 256-row tiles
    case MOE_GEMM_UP_SWIGLU: {
        using C = UpCfg;
        const int64_t b = mgrid_blocks(g.M, g.E, C::BM, (int)ceil_div(g.I, C::BN / 2));
        return sp ? launch_k(k_up_swiglu<C, true>, b, g, s, C::NT)
                  : launch_k(up_swiglu_mixed<MixT, Tall, Tall320>, b, g, s, MixT::NT);
    }
    case MOE_GEMM_DOWN: {
        using C = DownCfg;
        const int64_t b = mgrid_blocks(g.M, g.E, C::BM, (int)ceil_div(g.H, C::BN));
        if (sp) return launch_k(k_down<C, true>, b, g, s, C::NT);
        return g.o_bf16 ? launch_k(down_mixed<MixT, Tall, Tall320>, b, g, s, MixT::NT)
                        : launch_k(k_down<C, false>, b, g, s, C::NT);
    }
    case MOE_GEMM_DOWN_DGRAD: {
        using C = DownDgradCfg;
        const int64_t b = mgrid_blocks(g.M, g.E, C::BM, (int)ceil_div(g.I, C::BN));
        return sp ? launch_k(k_down_dgrad<C, true>, b, g, s, C::NT)
                  : launch_k(down_dgrad_mixed<MixT, Tall, Tall320>, b, g, s, MixT::NT);
    }
    case MOE_GEMM_UP_DGRAD: {
        using C = UpDgradCfg;
        const int64_t b = mgrid_blocks(g.M, g.E, C::BM, (int)ceil_div(g.H, C::BN));
        return g.dxp_bf16 && !sp ? launch_k(up_dgrad_mixed<MixT, Tall, Tall320>, b, g, s, MixT::NT)
                                 : launch_k(k_up_dgrad<C>, b, g, s, C::NT);
    }
    case MOE_GEMM_DOWN_WGRAD: {
        using C = WgradCfg;
        const int64_t act = g.M < g.E ? g.M : g.E;  // non-empty experts, at most
        const int64_t b = grid_for<WGRAD_XCD_CHUNK>(act * ceil_div(g.H, C::BM) * ceil_div(g.I, C::BN));
        return sp ? launch_k(k_wgrad<C, false, true>, b, g, s, C::NT)
                  : launch_k(k_wgrad<C, false, false>, b, g, s, C::NT);
    }
    case MOE_GEMM_UP_WGRAD: {
        using C = WgradCfg;
        const int64_t act = g.M < g.E ? g.M : g.E;
        const int64_t b = grid_for<WGRAD_XCD_CHUNK>(act * ceil_div(2 * g.I, C::BM) * ceil_div(g.H, C::BN));
        return sp ? launch_k(k_wgrad<C, true, true>, b, g, s, C::NT)
                  : launch_k(k_wgrad<C, true, false>, b, g, s, C::NT);
    }
    default:
        return hipErrorInvalidValue;
    }
}

}  // namespace moe
