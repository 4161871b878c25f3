// Grouped bf16 GEMMs of the MoE expert path on gfx950 MFMA
// (v_mfma_f32_32x32x16_bf16, fp32 accumulation).
//
// Every GEMM is written as C[r, c] = sum_k A(r, k) * B(c, k), staged
// through double-buffered LDS tiles 64 deep in k.  Operands whose k index is
// contiguous in memory are copied row by row into [rows][64] tiles
// (RowLoader) and read with 16-byte LDS reads; operands that are contiguous
// along the output dimension instead (the weights in dgrad, both operands in
// wgrad) are copied in their own layout into [64][rows] tiles (ColLoader) and
// read with gfx950's transposing LDS reads.  16-byte chunks are XOR-swizzled
// so stores and fragment reads are free of bank conflicts.  Token rows are gathered through row_map while loading:
// dispatch is fused into the load, as the MegaMoE page (intro) fuses it into
// the first grouped GEMM.
//
// Scheduling: forward and dgrad GEMMs tile the sorted rows of each expert
// (M-grouped); the per-expert m-tile prefix sums live on the device, the
// grid is sized from a host-side upper bound and surplus blocks exit.  The
// weight-gradient GEMMs tile the [rows x cols] output of each expert that has
// rows and loop over those rows (K-grouped), longest experts first; experts
// without rows are zeroed by a separate fill (overwrite) or left untouched
// (accumulate).  Block
// indices are remapped so that each of the 8 XCDs works on a contiguous run
// of tiles (neighbouring tiles share operand panels in that XCD's L2).
#include "common.h"

namespace moe {

constexpr int BK = 64;  // k elements per LDS stage

// LDS is addressed through explicit local-address-space pointers so that the
// compiler emits ds_read / ds_write (a generic pointer would become FLAT).
typedef __attribute__((address_space(3))) char lds_t;
typedef __attribute__((address_space(3))) u32x4_t lds_u32x4;
typedef __attribute__((address_space(3))) bf16x8_t lds_bf16x8;
typedef __attribute__((address_space(3))) float lds_f32;

MOE_DEV int swz(int r) { return (r ^ (r >> 3)) & 7; }
MOE_DEV int lds_off(int r, int c) { return r * 128 + ((c ^ swz(r)) << 4); }

template <int BM_, int BN_, int WM_, int WN_>
struct TileCfg {
    static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_;
    static constexpr int WAVES_M = BM / WM, WAVES_N = BN / WN;
    static constexpr int NT = WAVES_M * WAVES_N * 64;
    static constexpr int FM = WM / 32, FN = WN / 32;
    static constexpr int LDS_BYTES = 2 * (BM + BN) * 128;
    static_assert(WM % 32 == 0 && WN % 32 == 0, "wave tile is a multiple of 32x32");
    static_assert(BM == 256 || BM == 128, "m-tile prefix sums exist for 256 and 128 rows");
};

#ifndef MOE_PREFETCH
#define MOE_PREFETCH 1
#endif

// ------------------------------------------------------------- loaders ----
// Both loaders keep two register sets, so the global loads of stage s+2 are
// issued while stage s is computed and stored to LDS at the end of stage s+1
// (two stages of latency cover).

// K-major tile: ROWS x 64 with k contiguous (128 bytes a row).  Thread tid
// owns chunk tid % 8 of rows tid/8 + i*(NT/8); each owned row has its own
// element offset from `base` (rows may be gathered).
template <int ROWS, int NT>
struct RowLoader {
    static constexpr int RSTEP = NT / 8;
    static constexpr int CPT = ROWS / RSTEP;
    static_assert(ROWS % RSTEP == 0, "rows split evenly");
    const uint16_t *base;
    uint32_t off[CPT];
    u32x4_t reg[MOE_PREFETCH][CPT];
    int c, r0;
    MOE_DEV void init(int tid, const uint16_t *b) { c = tid & 7; r0 = tid >> 3; base = b; }
    MOE_DEV int row(int i) const { return r0 + i * RSTEP; }
    template <int S>
    MOE_DEV void load(int64_t k0)
    {
        const uint16_t *p = base + k0 + c * 8;
#pragma unroll
        for (int i = 0; i < CPT; ++i) reg[S][i] = *(const u32x4_t *)(p + off[i]);
    }
    template <int S>
    MOE_DEV void store(lds_t *lds) const
    {
#pragma unroll
        for (int i = 0; i < CPT; ++i) *(lds_u32x4 *)(lds + lds_off(row(i), c)) = reg[S][i];
    }
};

// N-major tile: 64 k-rows x ROWS, the other index contiguous (ROWS*2 bytes a
// k-row), in the source's own layout; the MFMA fragments are read from it
// with transposing LDS reads.  16-byte chunk c of k-row k sits at
// nmaj_off(k, c): the chunk index is XORed with 4*(k % 4), which keeps both
// the row stores and the transposing reads free of bank conflicts.
template <int ROWS>
MOE_DEV int nmaj_off(int k, int c) { return k * (ROWS * 2) + ((c ^ ((k & 3) << 2)) << 4); }

// Element (n, k) of the stage starting at k0 is base[(k0 + k) * ld + n], zero
// where k0 + k >= klim or n >= nlim (nlim a multiple of 8).  Thread tid owns
// chunk tid % (ROWS/8) of k-rows tid/(ROWS/8) + i*(NT*8/ROWS).  Out-of-range
// reads are clamped to a valid address and zeroed with selects (no branches).
template <int ROWS, int NT>
struct ColLoader {
    static constexpr int CPR = ROWS / 8;
    static constexpr int KSTEP = NT / CPR;
    static constexpr int CPT = 64 / KSTEP;
    static_assert(NT % CPR == 0 && 64 % KSTEP == 0, "chunks split evenly");
    const uint16_t *base;
    int64_t ld, klim, ncol;
    bool nok;
    int c, k0r;
    u32x4_t reg[MOE_PREFETCH][CPT];
    MOE_DEV void init(int tid, const uint16_t *b, int64_t ld_, int64_t n0, int64_t nlim,
                      int64_t klim_)
    {
        base = b;
        ld = ld_;
        klim = klim_;
        c = tid % CPR;
        k0r = tid / CPR;
        const int64_t n = n0 + c * 8;
        nok = n < nlim;
        ncol = nok ? n : 0;
    }
    MOE_DEV int krow(int i) const { return k0r + i * KSTEP; }
    template <int S>
    MOE_DEV void load(int64_t k0)
    {
#pragma unroll
        for (int i = 0; i < CPT; ++i) {
            const int64_t k = k0 + krow(i);
            const bool ok = nok && k < klim;
            const int64_t kc = k < klim ? k : klim - 1;
            u32x4_t v = *(const u32x4_t *)(base + kc * ld + ncol);
#pragma unroll
            for (int q = 0; q < 4; ++q) v[q] = ok ? v[q] : 0u;
            reg[S][i] = v;
        }
    }
    template <int S>
    MOE_DEV void store(lds_t *lds) const
    {
#pragma unroll
        for (int i = 0; i < CPT; ++i) *(lds_u32x4 *)(lds + nmaj_off<ROWS>(krow(i), c)) = reg[S][i];
    }
};

// ------------------------------------------------------------ MFMA core ----
template <class C>
struct Acc {
    f32x16_t v[C::FM][C::FN];
    MOE_DEV void zero()
    {
#pragma unroll
        for (int i = 0; i < C::FM; ++i)
#pragma unroll
            for (int j = 0; j < C::FN; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r) v[i][j][r] = 0.f;
    }
};

// MFMA operand fragment for rows rbase + lane%32 and k = kk*16 + (lane/32)*8
// + [0, 8).  K-major tile: one 16-byte read.  N-major tile: two transposing
// reads; in each group of 16 lanes, lane 4r+q addresses k-row kb + r at
// columns 4q..4q+3 of its 16-column slice, and lane j receives the four
// k-values of column j.
MOE_DEV bf16x8_t frag_kmaj(const lds_t *T, int rbase, int kk, int lane)
{
    return *(const lds_bf16x8 *)(T + lds_off(rbase + (lane & 31), kk * 2 + (lane >> 5)));
}

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;

template <int ROWS>
MOE_DEV bf16x8_t frag_nmaj(const lds_t *T, int rbase, int kk, int lane)
{
    const int g = lane >> 4, j = lane & 15, r = j >> 2, q = j & 3;
    const int n = rbase + (g & 1) * 16 + 4 * q;
    const int k = kk * 16 + (g >> 1) * 8 + r;
    const int within = (q & 1) * 8;
    v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_v4i16 *)(T + nmaj_off<ROWS>(k, n >> 3) + within));
    v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_v4i16 *)(T + nmaj_off<ROWS>(k + 4, n >> 3) + within));
    typedef short v8i16 __attribute__((ext_vector_type(8)));
    v8i16 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    return __builtin_bit_cast(bf16x8_t, v);
}

// One 64-deep LDS stage: 4 MFMA k-steps of 16.
template <class C, bool A_NMAJ, bool B_NMAJ>
MOE_DEV void mma_stage(const lds_t *As, const lds_t *Bs, Acc<C> &acc, int wm, int wn, int lane)
{
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
        bf16x8_t a[C::FM], b[C::FN];
#pragma unroll
        for (int i = 0; i < C::FM; ++i)
            a[i] = A_NMAJ ? frag_nmaj<C::BM>(As, wm * C::WM + i * 32, kk, lane)
                          : frag_kmaj(As, wm * C::WM + i * 32, kk, lane);
#pragma unroll
        for (int j = 0; j < C::FN; ++j)
            b[j] = B_NMAJ ? frag_nmaj<C::BN>(Bs, wn * C::WN + j * 32, kk, lane)
                          : frag_kmaj(Bs, wn * C::WN + j * 32, kk, lane);
#pragma unroll
        for (int i = 0; i < C::FM; ++i)
#pragma unroll
            for (int j = 0; j < C::FN; ++j)
                acc.v[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b[j], a[i], acc.v[i][j], 0, 0, 0);
    }
}

template <int S>
struct SetTag {
    static constexpr int value = S;
};

#ifndef MOE_PREFETCH
#define MOE_PREFETCH 1
#endif

// Main loop over nk stages of 64 k.  Stage s computes from LDS buffer s%2.
// Prefetch distance 1: the loads of stage s+1 are issued before the MFMAs of
// stage s and stored to the other LDS buffer after them.  Prefetch distance 2
// (two register sets): the loads of stage s+2 fill register set s%2 while
// set (s+1)%2, loaded during stage s-1, is stored; unrolled by two so each
// register set index is static.
template <class C, bool A_NMAJ, bool B_NMAJ, class LA, class LB>
MOE_DEV void mainloop(lds_t *lds, int nk, LA &la, LB &lb, Acc<C> &acc)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = wave / C::WAVES_N, wn = wave % C::WAVES_N;
    lds_t *As[2] = {lds, lds + C::BM * 128};
    lds_t *Bs[2] = {lds + 2 * C::BM * 128, lds + 2 * C::BM * 128 + C::BN * 128};
    acc.zero();
    if (nk <= 0) return;
    la.template load<0>(0);
    lb.template load<0>(0);
#if MOE_PREFETCH == 2
    if (nk > 1) {
        la.template load<1>(BK);
        lb.template load<1>(BK);
    }
#endif
    la.template store<0>(As[0]);
    lb.template store<0>(Bs[0]);
    __syncthreads();
#if MOE_PREFETCH == 2
    auto step = [&](auto tag, int s) {
        constexpr int S = decltype(tag)::value;
        if (s + 2 < nk) {
            la.template load<S>((int64_t)(s + 2) * BK);
            lb.template load<S>((int64_t)(s + 2) * BK);
        }
        mma_stage<C, A_NMAJ, B_NMAJ>(As[S], Bs[S], acc, wm, wn, lane);
        if (s + 1 < nk) {
            la.template store<1 - S>(As[1 - S]);
            lb.template store<1 - S>(Bs[1 - S]);
        }
        __syncthreads();
    };
    int s = 0;
    for (; s + 1 < nk; s += 2) {
        step(SetTag<0>(), s);
        step(SetTag<1>(), s + 1);
    }
    if (s < nk) step(SetTag<0>(), s);
#else
    for (int s = 0; s < nk; ++s) {
        const int cur = s & 1;
        const bool more = s + 1 < nk;
        if (more) {
            la.template load<0>((int64_t)(s + 1) * BK);
            lb.template load<0>((int64_t)(s + 1) * BK);
        }
        mma_stage<C, A_NMAJ, B_NMAJ>(As[cur], Bs[cur], acc, wm, wn, lane);
        if (more) {
            la.template store<0>(As[cur ^ 1]);
            lb.template store<0>(Bs[cur ^ 1]);
        }
        __syncthreads();
    }
#endif
}

// The MFMA takes the B fragment as its first operand, so each 32x32 block
// holds the transposed product: element r of acc.v[i][j] is
//   tile row (from A) = wm*WM + i*32 + lane%32
//   tile col (from B) = wn*WN + j*32 + (r/4)*8 + (lane/32)*4 + r%4
// i.e. every lane owns one row and four runs of four consecutive columns,
// which the epilogues store as 8- or 16-byte vectors.
template <class C>
MOE_DEV int acc_row(int wm, int i, int lane) { return wm * C::WM + i * 32 + (lane & 31); }
template <class C>
MOE_DEV int acc_col(int wn, int j, int rg, int lane)
{
    return wn * C::WN + j * 32 + rg * 8 + (lane >> 5) * 4;
}

MOE_DEV uint64_t pack_bf4(float a, float b, float c, float d)
{
    return (uint64_t)pack_bf2(a, b) | ((uint64_t)pack_bf2(c, d) << 32);
}
MOE_DEV void unpack_bf4(uint64_t v, float (&o)[4])
{
    o[0] = bf2f((uint16_t)(v & 0xffffu));
    o[1] = bf2f((uint16_t)((v >> 16) & 0xffffu));
    o[2] = bf2f((uint16_t)((v >> 32) & 0xffffu));
    o[3] = bf2f((uint16_t)(v >> 48));
}

// ------------------------------------------------------- tile schedules ----
// XCD-aware remap of block b over `total` tiles.  Blocks are dispatched to
// the 8 XCDs round-robin (block b runs on XCD b % 8); consecutive tiles are
// dealt to the XCDs in chunks of XCD_CHUNK (the CUs of one XCD), so the tiles
// an XCD runs together are neighbours (they share operand panels in its L2)
// while tiles of unequal cost spread evenly over all XCDs.  The grid is a
// multiple of 8 * XCD_CHUNK and at least `total` rounded up to that.
constexpr int64_t XCD_CHUNK = 32;
MOE_DEV int64_t xcd_remap(int64_t b, int64_t total)
{
    const int64_t x = b & 7, j = b >> 3;
    const int64_t L = ((j / XCD_CHUNK) * 8 + x) * XCD_CHUNK + (j % XCD_CHUNK);
    return L < total ? L : -1;
}

int64_t grid_for(int64_t total) { return ceil_div(total, 8 * XCD_CHUNK) * 8 * XCD_CHUNK; }

struct MTile {
    int e;
    int64_t m0, seg_end;
    int nt;
};

// M-grouped tile L: groups of GM m-tiles sweep all n-tiles before moving on.
template <int BM>
MOE_DEV bool decode_mtile(int64_t b, const int32_t *mt_off, const int32_t *offsets, int E,
                          int nN, MTile &t)
{
    constexpr int GM = 4;
    const int64_t total_mt = mt_off[E];
    const int64_t total = total_mt * nN;
    int64_t L = xcd_remap(b, total);
    if (L < 0) return false;
    int64_t grp = L / ((int64_t)GM * nN);
    int64_t first = grp * GM;
    int64_t gm = total_mt - first < GM ? total_mt - first : GM;
    int64_t in = L - grp * (int64_t)GM * nN;
    int64_t mt = first + in % gm;
    t.nt = (int)(in / gm);
    int lo = 0, hi = E;  // largest e with mt_off[e] <= mt
    while (hi - lo > 1) {
        int mid = (lo + hi) >> 1;
        if (mt_off[mid] <= mt) lo = mid; else hi = mid;
    }
    t.e = lo;
    t.m0 = offsets[lo] + (mt - mt_off[lo]) * BM;
    t.seg_end = offsets[lo + 1];
    return true;
}

int64_t mgrid_blocks(int64_t M, int E, int BM, int nN)
{
    int64_t mt = M / BM + (M < E ? M : E) + 1;
    return grid_for(mt * nN);
}

// fp32 tile store: rows [m0, seg_end), columns [n0, n0 + BN) below ncols,
// row stride ncols; 16-byte stores.
template <class C>
MOE_DEV void store_rows_f32(const Acc<C> &acc, float *out, int64_t m0, int64_t seg_end, int64_t n0,
                            int64_t ncols, int wm, int wn, int lane)
{
#pragma unroll
    for (int i = 0; i < C::FM; ++i) {
        const int64_t m = m0 + acc_row<C>(wm, i, lane);
        if (m >= seg_end) continue;
#pragma unroll
        for (int j = 0; j < C::FN; ++j)
#pragma unroll
            for (int rg = 0; rg < 4; ++rg) {
                const int64_t col = n0 + acc_col<C>(wn, j, rg, lane);
                if (col >= ncols) continue;
                f32x4_t v = {acc.v[i][j][rg * 4], acc.v[i][j][rg * 4 + 1], acc.v[i][j][rg * 4 + 2],
                             acc.v[i][j][rg * 4 + 3]};
                *(f32x4_t *)(out + m * ncols + col) = v;
            }
    }
}

// =========================================================================
// GEMM1 + SwiGLU:  h[r, n] = x[tok(r)] . w1[e, n, :],  a = silu(g) * u
// B tile rows: wave column wn covers gate columns i0 + wn*WN/2 + [0, WN/2)
// and the matching up columns, so each lane holds g and u of the same (r, i).
// =========================================================================
template <class C>
__global__ __launch_bounds__(C::NT) void k_up_swiglu(GemmArgs g)
{
    __shared__ __attribute__((aligned(16))) char lds_raw[C::LDS_BYTES];
    lds_t *lds = (lds_t *)lds_raw;
    const int I = g.I, H = g.H;
    const int nN = (int)ceil_div(I, C::BN / 2);
    MTile t;
    if (!decode_mtile<C::BM>(blockIdx.x, C::BM == 256 ? g.sched.mt_off256 : g.sched.mt_off128, g.offsets, g.E, nN, t)) return;
    const int tid = threadIdx.x;
    RowLoader<C::BM, C::NT> la;
    RowLoader<C::BN, C::NT> lb;
    la.init(tid, g.x);
    const uint16_t *w1e = g.w1 + (int64_t)t.e * 2 * I * H;
    lb.init(tid, w1e);
    const int64_t i0 = (int64_t)t.nt * (C::BN / 2);
#pragma unroll
    for (int q = 0; q < la.CPT; ++q) {
        int64_t m = t.m0 + la.row(q);
        if (m >= t.seg_end) m = t.seg_end - 1;
        la.off[q] = (uint32_t)((g.row_map[m] / g.k) * (int64_t)H);
    }
#pragma unroll
    for (int q = 0; q < lb.CPT; ++q) {
        int r = lb.row(q);
        int wn = r / C::WN, qq = r % C::WN;
        int half = C::WN / 2;
        int64_t i = i0 + wn * half + (qq < half ? qq : qq - half);
        if (i >= I) i = I - 1;
        int64_t n = qq < half ? i : I + i;
        lb.off[q] = (uint32_t)(n * H);
    }
    Acc<C> acc;
    mainloop<C, false, false>(lds, H / BK, la, lb, acc);

    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave / C::WAVES_N, wn = wave % C::WAVES_N;
    constexpr int HF = C::FN / 2;
#pragma unroll
    for (int i = 0; i < C::FM; ++i) {
        const int64_t m = t.m0 + acc_row<C>(wm, i, lane);
        if (m >= t.seg_end) continue;
#pragma unroll
        for (int j = 0; j < HF; ++j)
#pragma unroll
            for (int rg = 0; rg < 4; ++rg) {
                // gate columns of wave column wn start at i0 + wn*WN/2
                const int64_t col = i0 + wn * (C::WN / 2) + j * 32 + rg * 8 + (lane >> 5) * 4;
                if (col >= I) continue;
                float gv[4], uv[4], av[4];
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    gv[q] = acc.v[i][j][rg * 4 + q];
                    uv[q] = acc.v[i][j + HF][rg * 4 + q];
                    av[q] = gv[q] * sigmoidf_(gv[q]) * uv[q];
                }
                if (g.h) {
                    *(uint64_t *)(g.h + m * 2 * I + col) = pack_bf4(gv[0], gv[1], gv[2], gv[3]);
                    *(uint64_t *)(g.h + m * 2 * I + I + col) = pack_bf4(uv[0], uv[1], uv[2], uv[3]);
                }
                *(uint64_t *)(g.a + m * I + col) = pack_bf4(av[0], av[1], av[2], av[3]);
            }
    }
}

// =========================================================================
// GEMM2:  o[r, c] = a[r] . w2[e, c, :]   (fp32 out)
// =========================================================================
template <class C>
__global__ __launch_bounds__(C::NT) void k_down(GemmArgs g)
{
    __shared__ __attribute__((aligned(16))) char lds_raw[C::LDS_BYTES];
    lds_t *lds = (lds_t *)lds_raw;
    const int I = g.I, H = g.H;
    const int nN = (int)ceil_div(H, C::BN);
    MTile t;
    if (!decode_mtile<C::BM>(blockIdx.x, C::BM == 256 ? g.sched.mt_off256 : g.sched.mt_off128, g.offsets, g.E, nN, t)) return;
    const int tid = threadIdx.x;
    RowLoader<C::BM, C::NT> la;
    RowLoader<C::BN, C::NT> lb;
    la.init(tid, g.a);
    const uint16_t *w2e = g.w2 + (int64_t)t.e * H * I;
    lb.init(tid, w2e);
#pragma unroll
    for (int q = 0; q < la.CPT; ++q) {
        int64_t m = t.m0 + la.row(q);
        if (m >= t.seg_end) m = t.seg_end - 1;
        la.off[q] = (uint32_t)(m * I);
    }
    const int64_t n0 = (int64_t)t.nt * C::BN;
#pragma unroll
    for (int q = 0; q < lb.CPT; ++q) {
        int64_t n = n0 + lb.row(q);
        if (n >= H) n = H - 1;
        lb.off[q] = (uint32_t)(n * I);
    }
    Acc<C> acc;
    mainloop<C, false, false>(lds, I / BK, la, lb, acc);
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave / C::WAVES_N, wn = wave % C::WAVES_N;
    store_rows_f32<C>(acc, g.o, t.m0, t.seg_end, n0, H, wm, wn, lane);
}

// =========================================================================
// dgrad of GEMM2 + row-dot + SwiGLU backward:
//   dA'[r, i] = dy[tok(r)] . w2[e, :, i];  dw_part[r, nt] = sum_i dA' a
//   dA = topk_w * dA';  dh = (dA u sig(g)(1 + g(1 - sig(g))) | dA silu(g))
// =========================================================================
template <class C>
__global__ __launch_bounds__(C::NT) void k_down_dgrad(GemmArgs g)
{
    __shared__ __attribute__((aligned(16))) char lds_raw[C::LDS_BYTES];
    lds_t *lds = (lds_t *)lds_raw;
    const int I = g.I, H = g.H;
    const int nN = (int)ceil_div(I, C::BN);
    MTile t;
    if (!decode_mtile<C::BM>(blockIdx.x, C::BM == 256 ? g.sched.mt_off256 : g.sched.mt_off128, g.offsets, g.E, nN, t)) return;
    const int tid = threadIdx.x;
    RowLoader<C::BM, C::NT> la;
    ColLoader<C::BN, C::NT> lb;
    la.init(tid, g.dy);
#pragma unroll
    for (int q = 0; q < la.CPT; ++q) {
        int64_t m = t.m0 + la.row(q);
        if (m >= t.seg_end) m = t.seg_end - 1;
        la.off[q] = (uint32_t)((g.row_map[m] / g.k) * (int64_t)H);
    }
    const uint16_t *w2e = g.w2 + (int64_t)t.e * H * I;
    const int64_t n0 = (int64_t)t.nt * C::BN;
    // B(n = i, k = hh) = w2[e, hh, i]: k-row hh starts at w2e + hh*I
    lb.init(tid, w2e, I, n0, I, H);
    Acc<C> acc;
    mainloop<C, false, true>(lds, H / BK, la, lb, acc);
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave / C::WAVES_N, wn = wave % C::WAVES_N;
    lds_f32 *red = (lds_f32 *)lds;  // [WAVES_N][BM]; the LDS tiles are free now
#pragma unroll
    for (int i = 0; i < C::FM; ++i) {
        const int rl = acc_row<C>(wm, i, lane);
        const int64_t m = t.m0 + rl;
        const bool mok = m < t.seg_end;
        const float wgt = mok ? g.wrow[m] : 0.f;
        float part = 0.f;
#pragma unroll
        for (int j = 0; j < C::FN; ++j)
#pragma unroll
            for (int rg = 0; rg < 4; ++rg) {
                const int64_t col = n0 + acc_col<C>(wn, j, rg, lane);
                if (!mok || col >= I) continue;
                float gv[4], uv[4], av[4], dg[4], du[4];
                unpack_bf4(*(const uint64_t *)(g.h + m * 2 * I + col), gv);
                unpack_bf4(*(const uint64_t *)(g.h + m * 2 * I + I + col), uv);
                unpack_bf4(*(const uint64_t *)(g.a + m * I + col), av);
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const float dap = acc.v[i][j][rg * 4 + q];
                    part += dap * av[q];
                    const float da = wgt * dap;
                    const float sg = sigmoidf_(gv[q]);
                    dg[q] = da * uv[q] * sg * (1.0f + gv[q] * (1.0f - sg));
                    du[q] = da * gv[q] * sg;
                }
                *(uint64_t *)(g.dh + m * 2 * I + col) = pack_bf4(dg[0], dg[1], dg[2], dg[3]);
                *(uint64_t *)(g.dh + m * 2 * I + I + col) = pack_bf4(du[0], du[1], du[2], du[3]);
            }
        // lanes l and l+32 hold the same row
        part += __shfl_xor(part, 32, 64);
        if (lane < 32) red[wn * C::BM + rl] = part;
    }
    __syncthreads();
    for (int rl = tid; rl < C::BM; rl += C::NT) {
        const int64_t m = t.m0 + rl;
        if (m >= t.seg_end) continue;
        float v = 0.f;
#pragma unroll
        for (int w = 0; w < C::WAVES_N; ++w) v += red[w * C::BM + rl];
        g.dw_part[m * nN + t.nt] = v;
    }
}

// =========================================================================
// dgrad of GEMM1:  dxp[r, c] = dh[r] . w1[e, :, c]   (fp32 out)
// =========================================================================
template <class C>
__global__ __launch_bounds__(C::NT) void k_up_dgrad(GemmArgs g)
{
    __shared__ __attribute__((aligned(16))) char lds_raw[C::LDS_BYTES];
    lds_t *lds = (lds_t *)lds_raw;
    const int I = g.I, H = g.H;
    const int nN = (int)ceil_div(H, C::BN);
    MTile t;
    if (!decode_mtile<C::BM>(blockIdx.x, C::BM == 256 ? g.sched.mt_off256 : g.sched.mt_off128, g.offsets, g.E, nN, t)) return;
    const int tid = threadIdx.x;
    RowLoader<C::BM, C::NT> la;
    ColLoader<C::BN, C::NT> lb;
    la.init(tid, g.dh);
#pragma unroll
    for (int q = 0; q < la.CPT; ++q) {
        int64_t m = t.m0 + la.row(q);
        if (m >= t.seg_end) m = t.seg_end - 1;
        la.off[q] = (uint32_t)(m * 2 * I);
    }
    const uint16_t *w1e = g.w1 + (int64_t)t.e * 2 * I * H;
    const int64_t n0 = (int64_t)t.nt * C::BN;
    // B(n = hh, k = nn) = w1[e, nn, hh]: k-row nn starts at w1e + nn*H
    lb.init(tid, w1e, H, n0, H, 2 * I);
    Acc<C> acc;
    mainloop<C, false, true>(lds, 2 * I / BK, la, lb, acc);
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave / C::WAVES_N, wn = wave % C::WAVES_N;
    store_rows_f32<C>(acc, g.dxp, t.m0, t.seg_end, n0, H, wm, wn, lane);
}

// =========================================================================
// Weight gradients (K-grouped over each expert's rows).
//   DOWN:  dW2[e, hh, i] (+)= sum_r topk_w(r) dy[tok(r), hh] a[r, i]
//   UP:    dW1[e, n, hh] (+)= sum_r dh[r, n] x[tok(r), hh]
// Output tile rows come from operand A, columns from operand B; both are
// transposed loads over k = routed row.  The token rows are read from
// per-sorted-row copies (dyw = topk_w * dy[tok], xg = x[tok]) written by the
// gather pre-pass, so the k loop has no index loads.
// =========================================================================
template <class C, bool UP>
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
    const int64_t L = xcd_remap(blockIdx.x, total);
    if (L < 0) return;
    const int e = g.sched.order[L / tpe];
    // inside one expert: groups of GR row tiles sweep all column tiles, so
    // the tiles running together share A and B panels in L2
    constexpr int GR = 4;
    const int64_t rest = L % tpe;
    const int64_t grp = rest / ((int64_t)GR * nC);
    const int64_t first = grp * GR;
    const int64_t gr = nR - first < GR ? nR - first : GR;
    const int64_t in = rest - grp * (int64_t)GR * nC;
    const int rt = (int)(first + in % gr), ct = (int)(in / gr);
    const int64_t seg0 = g.offsets[e], seg1 = g.offsets[e + 1];
    const int64_t cnt = seg1 - seg0;
    const int64_t r0 = (int64_t)rt * C::BM, c0 = (int64_t)ct * C::BN;
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave / C::WAVES_N, wn = wave % C::WAVES_N;
    const int64_t dW_off = (int64_t)e * R * Cc;
    void *dWv = UP ? g.dW1 : g.dW2;
    // Operands are row-major per sorted row: A rows of length R, B rows of
    // length Cc (DOWN: w*dy gathered, a;  UP: dh, x gathered); k = sorted row
    // of this expert, so the loaders start at row seg0 and stop at seg1.
    const uint16_t *Ab = (UP ? g.dh : g.dyw) + seg0 * R;
    const uint16_t *Bb = (UP ? g.xg : g.a) + seg0 * Cc;
    ColLoader<C::BM, C::NT> la;
    ColLoader<C::BN, C::NT> lb;
    la.init(tid, Ab, R, r0, R, cnt);
    lb.init(tid, Bb, Cc, c0, Cc, cnt);
    const int nk = (int)ceil_div(cnt, BK);
    Acc<C> acc;
    mainloop<C, true, true>(lds, nk, la, lb, acc);
#pragma unroll
    for (int i = 0; i < C::FM; ++i) {
        const int64_t rr = r0 + acc_row<C>(wm, i, lane);
        if (rr >= R) continue;
#pragma unroll
        for (int j = 0; j < C::FN; ++j)
#pragma unroll
            for (int rg = 0; rg < 4; ++rg) {
                const int64_t cc = c0 + acc_col<C>(wn, j, rg, lane);
                if (cc >= Cc) continue;
                const int64_t o = dW_off + rr * Cc + cc;
                f32x4_t v = {acc.v[i][j][rg * 4], acc.v[i][j][rg * 4 + 1], acc.v[i][j][rg * 4 + 2],
                             acc.v[i][j][rg * 4 + 3]};
                if (g.dw_bf16) {
                    uint64_t *p = (uint64_t *)((uint16_t *)dWv + o);
                    if (g.dw_acc) {
                        float old[4];
                        unpack_bf4(*p, old);
                        v[0] += old[0]; v[1] += old[1]; v[2] += old[2]; v[3] += old[3];
                    }
                    *p = pack_bf4(v[0], v[1], v[2], v[3]);
                } else {
                    f32x4_t *p = (f32x4_t *)((float *)dWv + o);
                    if (g.dw_acc) v += *p;
                    *p = v;
                }
            }
    }
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
#ifndef MOE_TILE_BM
#define MOE_TILE_BM 256
#define MOE_TILE_BN 256
#define MOE_TILE_WM 64
#define MOE_TILE_WN 128
#endif
// 256x256 output tiles, 8 waves of 64x128 by default (two waves per SIMD)
using Big = TileCfg<MOE_TILE_BM, MOE_TILE_BN, MOE_TILE_WM, MOE_TILE_WN>;

int32_t dgrad2_cols(int32_t I) { return (int32_t)ceil_div(I, Big::BN); }

template <class K>
static hipError_t launch_k(K kern, int64_t blocks, const GemmArgs &g, hipStream_t s, int nt)
{
    if (blocks <= 0) return hipSuccess;
    kern<<<(unsigned)blocks, nt, 0, s>>>(g);
    return hipGetLastError();
}

hipError_t launch_grouped_gemm(int32_t op, const GemmArgs &g, hipStream_t s)
{
    using C = Big;
    switch (op) {
    case MOE_GEMM_UP_SWIGLU:
        return launch_k(k_up_swiglu<C>, mgrid_blocks(g.M, g.E, C::BM, (int)ceil_div(g.I, C::BN / 2)),
                        g, s, C::NT);
    case MOE_GEMM_DOWN:
        return launch_k(k_down<C>, mgrid_blocks(g.M, g.E, C::BM, (int)ceil_div(g.H, C::BN)), g, s, C::NT);
    case MOE_GEMM_DOWN_DGRAD:
        return launch_k(k_down_dgrad<C>, mgrid_blocks(g.M, g.E, C::BM, (int)ceil_div(g.I, C::BN)),
                        g, s, C::NT);
    case MOE_GEMM_UP_DGRAD:
        return launch_k(k_up_dgrad<C>, mgrid_blocks(g.M, g.E, C::BM, (int)ceil_div(g.H, C::BN)), g, s, C::NT);
    case MOE_GEMM_DOWN_WGRAD: {
        const int64_t act = g.M < g.E ? g.M : g.E;  // non-empty experts, at most
        int64_t total = act * ceil_div(g.H, C::BM) * ceil_div(g.I, C::BN);
        return launch_k(k_wgrad<C, false>, grid_for(total), g, s, C::NT);
    }
    case MOE_GEMM_UP_WGRAD: {
        const int64_t act = g.M < g.E ? g.M : g.E;
        int64_t total = act * ceil_div(2 * g.I, C::BM) * ceil_div(g.H, C::BN);
        return launch_k(k_wgrad<C, true>, grid_for(total), g, s, C::NT);
    }
    default:
        return hipErrorInvalidValue;
    }
}

}  // namespace moe
