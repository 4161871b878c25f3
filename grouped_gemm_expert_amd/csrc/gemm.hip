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

// ------------------------------------------------------------- loaders ----
// Operand tiles go from global memory straight into LDS (gfx950
// global_load_lds_dwordx4): lane l of a wave writes bytes [16 l, 16 l + 16)
// of a 1 KB LDS block whose address is uniform over the wave (it travels in
// M0), so each loader picks, per lane, the 16 global bytes that belong at
// that LDS position under the tile's swizzle.  The copies run asynchronously
// while the MFMAs of the previous stage execute; there are no staging
// registers and no ds_write in the main loop.

MOE_DEV int wave_uniform_id() { return __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6)); }

// The copy is issued from inline assembly: the compiler then does not track
// it, so it inserts no vmcnt wait in front of the LDS reads of the other
// buffer (it cannot prove that those do not alias the copy's destination);
// the main loop waits for its copies itself (wait_copies) before the barrier
// that publishes them.  M0 carries the LDS block address.
MOE_DEV void copy16_to_lds(const char *src, lds_t *dst_block)
{
    const uint32_t m0v = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)dst_block);
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off"
                 :
                 : "v"(src), "s"(m0v)
                 : "memory", "m0");
}

// Wait until every global->LDS copy this wave issued has landed: s_waitcnt
// vmcnt(0) (expcnt and lgkmcnt fields left at their maxima).
MOE_DEV void wait_copies() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// K-major tile: ROWS x 64 with k contiguous (128 bytes a row; chunk c of row r
// at lds_off(r, c)).  1 KB block q holds rows 8q .. 8q+7; wave w fills blocks
// w*NI .. w*NI+NI-1, and its lane l takes row 8q + l/8 at physical chunk l%8,
// i.e. logical chunk (l%8) ^ swz(row).  off[i] is the byte offset of that
// lane's 16 bytes from `base` at k = 0 (rows may be gathered).
template <int ROWS, int NT>
struct KLoad {
    static constexpr int NI = ROWS / 8 / (NT / 64);
    static_assert(NI * 8 * (NT / 64) == ROWS, "1 KB blocks split evenly over the waves");
    const char *base;
    uint32_t off[NI];
    int q0;
    MOE_DEV void init(const void *b, int wave) { base = (const char *)b; q0 = wave * NI; }
    MOE_DEV int row(int i, int lane) const { return (q0 + i) * 8 + (lane >> 3); }
    MOE_DEV void set(int i, int lane, uint32_t row_bytes)
    {
        off[i] = row_bytes + ((uint32_t)((lane & 7) ^ swz(row(i, lane))) << 4);
    }
    MOE_DEV void issue(lds_t *tile, int64_t k0, int) const
    {
        const char *p = base + k0 * 2;
#pragma unroll
        for (int i = 0; i < NI; ++i) copy16_to_lds(p + off[i], tile + (q0 + i) * 1024);
    }
    MOE_DEV void zero_tail(lds_t *, int) const {}
};

// N-major tile: 64 k-rows x ROWS, the other index contiguous (ROWS*2 bytes a
// k-row), in the source's own layout; the MFMA fragments are read from it
// with transposing LDS reads.  16-byte chunk c of k-row k sits at
// nmaj_off(k, c): the chunk index is XORed with 4*(k % 4), which keeps the
// transposing reads free of bank conflicts.
template <int ROWS>
MOE_DEV int nmaj_off(int k, int c) { return k * (ROWS * 2) + ((c ^ ((k & 3) << 2)) << 4); }

// 1 KB block q holds k-rows q*KPB .. q*KPB+KPB-1; lane l takes k-row
// q*KPB + l/CPR at physical chunk l%CPR, logical chunk (l%CPR) ^ 4*(k%4).
// Element (n, k) of the stage at k0 is at byte ((k0 + k) * ld + n) * 2 from
// base.  k-rows at or past the stage's valid count are read from its last
// valid row and zeroed in LDS once landed (zero_tail), so a partial last
// stage adds nothing; columns at or past nlim are read from column 0: they
// feed only output rows/columns that are never stored.
template <int ROWS, int NT>
struct NLoad {
    static constexpr int CPR = ROWS / 8;
    static constexpr int KPB = 64 / CPR;
    static constexpr int NI = 64 / KPB / (NT / 64);
    static_assert(NI * KPB * (NT / 64) == 64, "1 KB blocks split evenly over the waves");
    const char *base;
    uint32_t ldb;       // bytes per k-row
    uint32_t ncol[NI];  // byte offset of the lane's 8 columns in block i
    int q0, lane;
    MOE_DEV int krow(int i) const { return (q0 + i) * KPB + lane / CPR; }
    MOE_DEV void init(const void *b, int64_t ld, int64_t n0, int64_t nlim, int wave, int ln)
    {
        base = (const char *)b;
        ldb = (uint32_t)(ld * 2);
        q0 = wave * NI;
        lane = ln;
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const int k = krow(i);
            const int c = (lane % CPR) ^ ((k & 3) << 2);
            int64_t n = n0 + c * 8;
            if (n >= nlim) n = 0;
            ncol[i] = (uint32_t)(n * 2);
        }
    }
    MOE_DEV void issue(lds_t *tile, int64_t k0, int kvalid) const
    {
        const char *p = base + k0 * (int64_t)ldb;
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            int k = krow(i);
            if (k >= kvalid) k = kvalid - 1;
            copy16_to_lds(p + (uint32_t)k * ldb + ncol[i], tile + (q0 + i) * 1024);
        }
    }
    MOE_DEV void zero_tail(lds_t *tile, int kvalid) const
    {
        const u32x4_t z = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int i = 0; i < NI; ++i)
            if (krow(i) >= kvalid) *(lds_u32x4 *)(tile + (q0 + i) * 1024 + lane * 16) = z;
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

// Main loop over the K/64 stages, two LDS buffers.  Stage s: issue the
// copies of stage s+1 into the other buffer (free: every wave passed the
// barrier that ended stage s-1), run the MFMAs of stage s, wait for this
// wave's copies, zero a partial last stage's tail rows (KTAIL), barrier.
// One barrier a stage covers both hazards: the next stage's data has landed
// for every wave, and no wave still reads the buffer the stage after will
// overwrite.
template <class C, bool A_NMAJ, bool B_NMAJ, bool KTAIL, class LA, class LB>
MOE_DEV void mainloop(lds_t *lds, int64_t K, const LA &la, const LB &lb, Acc<C> &acc)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = wave / C::WAVES_N, wn = wave % C::WAVES_N;
    lds_t *As[2] = {lds, lds + C::BM * 128};
    lds_t *Bs[2] = {lds + 2 * C::BM * 128, lds + 2 * C::BM * 128 + C::BN * 128};
    acc.zero();
    const int nk = (int)ceil_div(K, BK);
    if (nk <= 0) return;
    auto kvalid = [&](int s) -> int {
        const int64_t rem = K - (int64_t)s * BK;
        return KTAIL ? (rem < BK ? (int)rem : BK) : BK;
    };
    auto fill = [&](int s, int buf) {
        la.issue(As[buf], (int64_t)s * BK, kvalid(s));
        lb.issue(Bs[buf], (int64_t)s * BK, kvalid(s));
    };
    auto land = [&](int s, int buf) {
        wait_copies();
        if (KTAIL && kvalid(s) < BK) {
            la.zero_tail(As[buf], kvalid(s));
            lb.zero_tail(Bs[buf], kvalid(s));
        }
    };
    fill(0, 0);
    land(0, 0);
    __syncthreads();
    for (int s = 0; s < nk; ++s) {
        const int cur = s & 1;
        const bool more = s + 1 < nk;
        if (more) fill(s + 1, cur ^ 1);
        mma_stage<C, A_NMAJ, B_NMAJ>(As[cur], Bs[cur], acc, wm, wn, lane);
        if (more) land(s + 1, cur ^ 1);
        __syncthreads();
    }
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
    mainloop<C, false, false, false>(lds, I, la, lb, acc);
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
    mainloop<C, false, true, false>(lds, H, la, lb, acc);
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
    mainloop<C, false, true, false>(lds, 2 * I, la, lb, acc);
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
    NLoad<C::BM, C::NT> la;
    NLoad<C::BN, C::NT> lb;
    la.init(Ab, R, r0, R, wave_uniform_id(), lane);
    lb.init(Bb, Cc, c0, Cc, wave_uniform_id(), lane);
    Acc<C> acc;
    mainloop<C, true, true, true>(lds, cnt, la, lb, acc);
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
// 256x256 output tiles computed by 8 waves (two a SIMD).  Wave tiles are
// 128 rows x 64 columns where the column operand is read with transposing LDS
// reads (down_dgrad, up_dgrad: the transposed operand then supplies the
// smaller fragment count) and for up_swiglu; 64 x 128 elsewhere.
using Tall = TileCfg<256, 256, 128, 64>;
using Wide = TileCfg<256, 256, 64, 128>;

int32_t dgrad2_cols(int32_t I) { return (int32_t)ceil_div(I, Tall::BN); }

template <class K>
static hipError_t launch_k(K kern, int64_t blocks, const GemmArgs &g, hipStream_t s, int nt)
{
    if (blocks <= 0) return hipSuccess;
    kern<<<(unsigned)blocks, nt, 0, s>>>(g);
    return hipGetLastError();
}

hipError_t launch_grouped_gemm(int32_t op, const GemmArgs &g, hipStream_t s)
{
    switch (op) {
    case MOE_GEMM_UP_SWIGLU: {
        using C = Tall;
        return launch_k(k_up_swiglu<C>, mgrid_blocks(g.M, g.E, C::BM, (int)ceil_div(g.I, C::BN / 2)),
                        g, s, C::NT);
    }
    case MOE_GEMM_DOWN: {
        using C = Wide;
        return launch_k(k_down<C>, mgrid_blocks(g.M, g.E, C::BM, (int)ceil_div(g.H, C::BN)), g, s, C::NT);
    }
    case MOE_GEMM_DOWN_DGRAD: {
        using C = Tall;
        return launch_k(k_down_dgrad<C>, mgrid_blocks(g.M, g.E, C::BM, (int)ceil_div(g.I, C::BN)),
                        g, s, C::NT);
    }
    case MOE_GEMM_UP_DGRAD: {
        using C = Tall;
        return launch_k(k_up_dgrad<C>, mgrid_blocks(g.M, g.E, C::BM, (int)ceil_div(g.H, C::BN)), g, s, C::NT);
    }
    case MOE_GEMM_DOWN_WGRAD: {
        using C = Wide;
        const int64_t act = g.M < g.E ? g.M : g.E;  // non-empty experts, at most
        int64_t total = act * ceil_div(g.H, C::BM) * ceil_div(g.I, C::BN);
        return launch_k(k_wgrad<C, false>, grid_for(total), g, s, C::NT);
    }
    case MOE_GEMM_UP_WGRAD: {
        using C = Wide;
        const int64_t act = g.M < g.E ? g.M : g.E;
        int64_t total = act * ceil_div(2 * g.I, C::BM) * ceil_div(g.H, C::BN);
        return launch_k(k_wgrad<C, true>, grid_for(total), g, s, C::NT);
    }
    default:
        return hipErrorInvalidValue;
    }
}

}  // namespace moe
