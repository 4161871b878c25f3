// Grouped bf16 GEMMs of the MoE expert path on gfx950 MFMA
// (v_mfma_f32_32x32x16_bf16, fp32 accumulation).
//
// Every GEMM is written as C[r, c] = sum_k A(r, k) * B(c, k): both operands
// are staged through LDS as [rows][64] bf16 tiles (k contiguous, 128 bytes a
// row, 16-byte chunks XOR-swizzled so that MFMA fragment reads and transposed
// stores are free of bank conflicts).  Operands whose k index is contiguous
// in memory are copied row by row (RowLoader); operands whose rows are
// contiguous along the output dimension instead (the weights in dgrad, both
// operands in wgrad) are loaded as 8x8 blocks and transposed in registers
// (TransLoader).  Token rows are gathered through row_map while loading:
// dispatch is fused into the load, as the MegaMoE page (intro) fuses it into
// the first grouped GEMM.
//
// Scheduling: forward and dgrad GEMMs tile the sorted rows of each expert
// (M-grouped); the per-expert m-tile prefix sums live on the device, the
// grid is sized from a host-side upper bound and surplus blocks exit.  The
// weight-gradient GEMMs tile each expert's [rows x cols] output and loop over
// its routed rows (K-grouped), longest experts first; an expert with no rows
// gets exact zeros (overwrite) or is left untouched (accumulate).  Block
// indices are remapped so that each of the 8 XCDs works on a contiguous run
// of tiles (neighbouring tiles share operand panels in that XCD's L2).
#include "common.h"

namespace moe {

constexpr int BK = 64;  // k elements per LDS stage

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
};

// ------------------------------------------------------------- loaders ----
// ROWS x 64 tile from rows with contiguous k.  Thread tid owns chunk tid % 8
// of rows tid/8 + i*(NT/8).
template <int ROWS, int NT>
struct RowLoader {
    static constexpr int RSTEP = NT / 8;
    static constexpr int CPT = ROWS / RSTEP;
    static_assert(ROWS % RSTEP == 0, "rows split evenly");
    const uint16_t *base;
    uint32_t off[CPT];  // element offset of each owned row from base
    u32x4_t reg[CPT];
    int c, r0;
    MOE_DEV void init(int tid, const uint16_t *b) { c = tid & 7; r0 = tid >> 3; base = b; }
    MOE_DEV int row(int i) const { return r0 + i * RSTEP; }
    MOE_DEV void load(int64_t k0)
    {
        const uint16_t *p = base + k0 + c * 8;
#pragma unroll
        for (int i = 0; i < CPT; ++i) reg[i] = *(const u32x4_t *)(p + off[i]);
    }
    MOE_DEV void store(char *lds) const
    {
#pragma unroll
        for (int i = 0; i < CPT; ++i) *(u32x4_t *)(lds + lds_off(row(i), c)) = reg[i];
    }
};

// ROWS x 64 tile whose source has rows along k: element (n, k) sits at
// kptr(k)[n].  Each thread loads 8 k-rows x 8 n (8 x 16 bytes), transposes in
// registers and stores 8 tile rows' chunk.  A null kptr row and columns at or
// beyond `nlim` read as zeros (nlim is a multiple of 8); an optional per-k-row
// scale multiplies the row (in fp32, rounded to bf16).
template <int ROWS, int NT>
struct TransLoader {
    static constexpr int NB = ROWS / 8;
    static constexpr int BLOCKS = NB * 8;
    static constexpr int BPT = (BLOCKS + NT - 1) / NT;
    u32x4_t reg[BPT][8];
    int tid;
    MOE_DEV void init(int t) { tid = t; }
    MOE_DEV bool has(int i) const { return BLOCKS % NT == 0 || tid + i * NT < BLOCKS; }
    MOE_DEV int nb(int i) const { return (tid + i * NT) % NB; }
    MOE_DEV int kb(int i) const { return (tid + i * NT) / NB; }
    // rowptr(kk) -> pointer to element n=0 of k-row k0+kk (or nullptr), scale(kk)
    template <class RowPtr, class Scale>
    MOE_DEV void load(int64_t n0, int64_t nlim, RowPtr rowptr, Scale scale)
    {
#pragma unroll
        for (int i = 0; i < BPT; ++i) {
            if (!has(i)) continue;
            const int64_t n = n0 + nb(i) * 8;
            const bool nok = n < nlim;
#pragma unroll
            for (int r = 0; r < 8; ++r) {
                int kk = kb(i) * 8 + r;
                const uint16_t *p = nok ? rowptr(kk) : nullptr;
                u32x4_t v = {0u, 0u, 0u, 0u};
                if (p) v = *(const u32x4_t *)(p + n);
                float s = scale(kk);
                if (s != 1.0f) {
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        uint32_t d = v[q];
                        v[q] = pack_bf2(bf2f((uint16_t)(d & 0xffffu)) * s,
                                        bf2f((uint16_t)(d >> 16)) * s);
                    }
                }
                reg[i][r] = v;
            }
        }
    }
    MOE_DEV void store(char *lds) const
    {
#pragma unroll
        for (int i = 0; i < BPT; ++i) {
            if (!has(i)) continue;
#pragma unroll
            for (int n = 0; n < 8; ++n) {
                u32x4_t o;
#pragma unroll
                for (int kp = 0; kp < 4; ++kp) {
                    uint32_t lo = reg[i][2 * kp][n >> 1], hi = reg[i][2 * kp + 1][n >> 1];
                    o[kp] = (n & 1) ? ((lo >> 16) | (hi & 0xffff0000u))
                                    : ((lo & 0xffffu) | (hi << 16));
                }
                *(u32x4_t *)(lds + lds_off(nb(i) * 8 + n, kb(i))) = o;
            }
        }
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

// One 64-deep LDS stage: 4 MFMA k-steps of 16.
template <class C>
MOE_DEV void mma_stage(const char *As, const char *Bs, Acc<C> &acc, int wm, int wn, int lane)
{
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
        const int ch = kk * 2 + (lane >> 5);
        bf16x8_t a[C::FM], b[C::FN];
#pragma unroll
        for (int i = 0; i < C::FM; ++i) {
            int r = wm * C::WM + i * 32 + (lane & 31);
            a[i] = *(const bf16x8_t *)(As + lds_off(r, ch));
        }
#pragma unroll
        for (int j = 0; j < C::FN; ++j) {
            int r = wn * C::WN + j * 32 + (lane & 31);
            b[j] = *(const bf16x8_t *)(Bs + lds_off(r, ch));
        }
#pragma unroll
        for (int i = 0; i < C::FM; ++i)
#pragma unroll
            for (int j = 0; j < C::FN; ++j)
                acc.v[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc.v[i][j], 0, 0, 0);
    }
}

// Software-pipelined main loop over nk stages: global loads for stage s+1 are
// issued before the MFMAs of stage s and land in the other LDS buffer after.
template <class C, class LoadA, class LoadB>
MOE_DEV void mainloop(char *lds, int nk, LoadA &&loadA, LoadB &&loadB, Acc<C> &acc)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = wave / C::WAVES_N, wn = wave % C::WAVES_N;
    char *As[2] = {lds, lds + C::BM * 128};
    char *Bs[2] = {lds + 2 * C::BM * 128, lds + 2 * C::BM * 128 + C::BN * 128};
    acc.zero();
    if (nk <= 0) return;
    loadA(0, As[0], true, false);
    loadB(0, Bs[0], true, false);
    loadA(0, As[0], false, true);
    loadB(0, Bs[0], false, true);
    __syncthreads();
    for (int s = 0; s < nk; ++s) {
        const int cur = s & 1;
        const bool more = s + 1 < nk;
        if (more) {
            loadA(s + 1, As[cur ^ 1], true, false);
            loadB(s + 1, Bs[cur ^ 1], true, false);
        }
        mma_stage<C>(As[cur], Bs[cur], acc, wm, wn, lane);
        if (more) {
            loadA(s + 1, As[cur ^ 1], false, true);
            loadB(s + 1, Bs[cur ^ 1], false, true);
        }
        __syncthreads();
    }
}

// Element (i, j, r) of the accumulators <-> tile coordinates:
//   row = wm*WM + i*32 + (r/4)*8 + (lane/32)*4 + r%4,  col = wn*WN + j*32 + lane%32
template <class C>
MOE_DEV int acc_row(int wm, int i, int r, int lane)
{
    return wm * C::WM + i * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
}
template <class C>
MOE_DEV int acc_col(int wn, int j, int lane) { return wn * C::WN + j * 32 + (lane & 31); }

// ------------------------------------------------------- tile schedules ----
// XCD-aware remap of block b over `total` tiles (grid >= total rounded up to
// 8): XCD x (= b % 8) gets tiles [x*q, (x+1)*q) with q = ceil(total/8).
MOE_DEV int64_t xcd_remap(int64_t b, int64_t total)
{
    int64_t q = (total + 7) >> 3;
    int64_t t8 = q << 3;
    if (b >= t8) return -1;
    int64_t L = (b & 7) * q + (b >> 3);
    return L < total ? L : -1;
}

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
    int64_t total = mt * nN;
    return ceil_div(total, 8) * 8;
}

// =========================================================================
// GEMM1 + SwiGLU:  h[r, n] = x[tok(r)] . w1[e, n, :],  a = silu(g) * u
// B tile rows: wave column wn covers gate columns i0 + wn*WN/2 + [0, WN/2)
// and the matching up columns, so each lane holds g and u of the same (r, i).
// =========================================================================
template <class C>
__global__ __launch_bounds__(C::NT) void k_up_swiglu(GemmArgs g)
{
    __shared__ __attribute__((aligned(16))) char lds[C::LDS_BYTES];
    const int I = g.I, H = g.H;
    const int nN = (int)ceil_div(I, C::BN / 2);
    MTile t;
    if (!decode_mtile<C::BM>(blockIdx.x, g.sched.mt_off256, g.offsets, g.E, nN, t)) return;
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
    mainloop<C>(
        lds, H / BK,
        [&](int s, char *dst, bool ld, bool st) { if (ld) la.load((int64_t)s * BK); if (st) la.store(dst); },
        [&](int s, char *dst, bool ld, bool st) { if (ld) lb.load((int64_t)s * BK); if (st) lb.store(dst); },
        acc);

    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave / C::WAVES_N, wn = wave % C::WAVES_N;
    constexpr int HF = C::FN / 2;
#pragma unroll
    for (int i = 0; i < C::FM; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int64_t m = t.m0 + acc_row<C>(wm, i, r, lane);
            if (m >= t.seg_end) continue;
#pragma unroll
            for (int j = 0; j < HF; ++j) {
                const int64_t col = i0 + wn * (C::WN / 2) + j * 32 + (lane & 31);
                if (col >= I) continue;
                const float gv = acc.v[i][j][r], uv = acc.v[i][j + HF][r];
                const float av = gv * sigmoidf_(gv) * uv;
                if (g.h) {
                    g.h[m * 2 * I + col] = f2bf(gv);
                    g.h[m * 2 * I + I + col] = f2bf(uv);
                }
                g.a[m * I + col] = f2bf(av);
            }
        }
}

// =========================================================================
// GEMM2:  o[r, c] = a[r] . w2[e, c, :]   (fp32 out)
// =========================================================================
template <class C>
__global__ __launch_bounds__(C::NT) void k_down(GemmArgs g)
{
    __shared__ __attribute__((aligned(16))) char lds[C::LDS_BYTES];
    const int I = g.I, H = g.H;
    const int nN = (int)ceil_div(H, C::BN);
    MTile t;
    if (!decode_mtile<C::BM>(blockIdx.x, g.sched.mt_off256, g.offsets, g.E, nN, t)) return;
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
    mainloop<C>(
        lds, I / BK,
        [&](int s, char *dst, bool ld, bool st) { if (ld) la.load((int64_t)s * BK); if (st) la.store(dst); },
        [&](int s, char *dst, bool ld, bool st) { if (ld) lb.load((int64_t)s * BK); if (st) lb.store(dst); },
        acc);
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave / C::WAVES_N, wn = wave % C::WAVES_N;
#pragma unroll
    for (int i = 0; i < C::FM; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int64_t m = t.m0 + acc_row<C>(wm, i, r, lane);
            if (m >= t.seg_end) continue;
#pragma unroll
            for (int j = 0; j < C::FN; ++j) {
                const int64_t col = n0 + acc_col<C>(wn, j, lane);
                if (col < H) g.o[m * H + col] = acc.v[i][j][r];
            }
        }
}

// =========================================================================
// dgrad of GEMM2 + row-dot + SwiGLU backward:
//   dA'[r, i] = dy[tok(r)] . w2[e, :, i];  dw_part[r, nt] = sum_i dA' a
//   dA = topk_w * dA';  dh = (dA u sig(g)(1 + g(1 - sig(g))) | dA silu(g))
// =========================================================================
template <class C>
__global__ __launch_bounds__(C::NT) void k_down_dgrad(GemmArgs g)
{
    __shared__ __attribute__((aligned(16))) char lds[C::LDS_BYTES];
    const int I = g.I, H = g.H;
    const int nN = (int)ceil_div(I, C::BN);
    MTile t;
    if (!decode_mtile<C::BM>(blockIdx.x, g.sched.mt_off256, g.offsets, g.E, nN, t)) return;
    const int tid = threadIdx.x;
    RowLoader<C::BM, C::NT> la;
    TransLoader<C::BN, C::NT> lb;
    la.init(tid, g.dy);
    lb.init(tid);
#pragma unroll
    for (int q = 0; q < la.CPT; ++q) {
        int64_t m = t.m0 + la.row(q);
        if (m >= t.seg_end) m = t.seg_end - 1;
        la.off[q] = (uint32_t)((g.row_map[m] / g.k) * (int64_t)H);
    }
    const uint16_t *w2e = g.w2 + (int64_t)t.e * H * I;
    const int64_t n0 = (int64_t)t.nt * C::BN;
    // B(n = i, k = hh) = w2[e, hh, i]: k-row hh starts at w2e + hh*I
    Acc<C> acc;
    mainloop<C>(
        lds, H / BK,
        [&](int s, char *dst, bool ld, bool st) { if (ld) la.load((int64_t)s * BK); if (st) la.store(dst); },
        [&](int s, char *dst, bool ld, bool st) {
            if (ld)
                lb.load(n0, I,
                        [&](int kk) -> const uint16_t * { return w2e + ((int64_t)s * BK + kk) * I; },
                        [](int) { return 1.0f; });
            if (st) lb.store(dst);
        },
        acc);
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave / C::WAVES_N, wn = wave % C::WAVES_N;
    float *red = (float *)lds;  // [WAVES_N][BM]; the LDS tiles are free now
#pragma unroll
    for (int i = 0; i < C::FM; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int rl = acc_row<C>(wm, i, r, lane);
            const int64_t m = t.m0 + rl;
            const bool mok = m < t.seg_end;
            const float wgt = mok ? g.topk_w[g.row_map[m]] : 0.f;
            float part = 0.f;
#pragma unroll
            for (int j = 0; j < C::FN; ++j) {
                const int64_t col = n0 + acc_col<C>(wn, j, lane);
                if (!mok || col >= I) continue;
                const float dap = acc.v[i][j][r];
                const float gv = bf2f(g.h[m * 2 * I + col]);
                const float uv = bf2f(g.h[m * 2 * I + I + col]);
                const float av = bf2f(g.a[m * I + col]);
                part += dap * av;
                const float da = wgt * dap;
                const float sg = sigmoidf_(gv);
                g.dh[m * 2 * I + col] = f2bf(da * uv * sg * (1.0f + gv * (1.0f - sg)));
                g.dh[m * 2 * I + I + col] = f2bf(da * gv * sg);
            }
#pragma unroll
            for (int off = 16; off >= 1; off >>= 1) part += __shfl_xor(part, off, 64);
            if ((lane & 31) == 0) red[wn * C::BM + rl] = part;
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
    __shared__ __attribute__((aligned(16))) char lds[C::LDS_BYTES];
    const int I = g.I, H = g.H;
    const int nN = (int)ceil_div(H, C::BN);
    MTile t;
    if (!decode_mtile<C::BM>(blockIdx.x, g.sched.mt_off256, g.offsets, g.E, nN, t)) return;
    const int tid = threadIdx.x;
    RowLoader<C::BM, C::NT> la;
    TransLoader<C::BN, C::NT> lb;
    la.init(tid, g.dh);
    lb.init(tid);
#pragma unroll
    for (int q = 0; q < la.CPT; ++q) {
        int64_t m = t.m0 + la.row(q);
        if (m >= t.seg_end) m = t.seg_end - 1;
        la.off[q] = (uint32_t)(m * 2 * I);
    }
    const uint16_t *w1e = g.w1 + (int64_t)t.e * 2 * I * H;
    const int64_t n0 = (int64_t)t.nt * C::BN;
    // B(n = hh, k = nn) = w1[e, nn, hh]: k-row nn starts at w1e + nn*H
    Acc<C> acc;
    mainloop<C>(
        lds, 2 * I / BK,
        [&](int s, char *dst, bool ld, bool st) { if (ld) la.load((int64_t)s * BK); if (st) la.store(dst); },
        [&](int s, char *dst, bool ld, bool st) {
            if (ld)
                lb.load(n0, H,
                        [&](int kk) -> const uint16_t * { return w1e + ((int64_t)s * BK + kk) * H; },
                        [](int) { return 1.0f; });
            if (st) lb.store(dst);
        },
        acc);
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave / C::WAVES_N, wn = wave % C::WAVES_N;
#pragma unroll
    for (int i = 0; i < C::FM; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int64_t m = t.m0 + acc_row<C>(wm, i, r, lane);
            if (m >= t.seg_end) continue;
#pragma unroll
            for (int j = 0; j < C::FN; ++j) {
                const int64_t col = n0 + acc_col<C>(wn, j, lane);
                if (col < H) g.dxp[m * H + col] = acc.v[i][j][r];
            }
        }
}

// =========================================================================
// Weight gradients (K-grouped over each expert's rows).
//   DOWN:  dW2[e, hh, i] (+)= sum_r topk_w(r) dy[tok(r), hh] a[r, i]
//   UP:    dW1[e, n, hh] (+)= sum_r dh[r, n] x[tok(r), hh]
// Output tile rows come from operand A, columns from operand B; both are
// transposed loads over k = routed row.
// =========================================================================
template <class C, bool UP>
__global__ __launch_bounds__(C::NT) void k_wgrad(GemmArgs g)
{
    __shared__ __attribute__((aligned(16))) char lds[C::LDS_BYTES];
    const int I = g.I, H = g.H;
    const int R = UP ? 2 * I : H;   // output rows
    const int Cc = UP ? H : I;      // output cols
    const int nR = (int)ceil_div(R, C::BM), nC = (int)ceil_div(Cc, C::BN);
    const int64_t tpe = (int64_t)nR * nC;
    const int64_t total = (int64_t)g.E * tpe;
    const int64_t L = xcd_remap(blockIdx.x, total);
    if (L < 0) return;
    const int e = g.sched.order[L / tpe];
    const int64_t rest = L % tpe;
    const int rt = (int)(rest / nC), ct = (int)(rest % nC);
    const int64_t seg0 = g.offsets[e], seg1 = g.offsets[e + 1];
    const int64_t cnt = seg1 - seg0;
    const int64_t r0 = (int64_t)rt * C::BM, c0 = (int64_t)ct * C::BN;
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave / C::WAVES_N, wn = wave % C::WAVES_N;
    const int64_t dW_off = (int64_t)e * R * Cc;
    void *dWv = UP ? g.dW1 : g.dW2;
    if (cnt == 0) {
        if (g.dw_acc) return;
        // exact zeros for an expert without rows
        for (int q = tid; q < C::BM * C::BN; q += C::NT) {
            const int64_t rr = r0 + q / C::BN, cc = c0 + q % C::BN;
            if (rr >= R || cc >= Cc) continue;
            const int64_t o = dW_off + rr * Cc + cc;
            if (g.dw_bf16) ((uint16_t *)dWv)[o] = 0;
            else ((float *)dWv)[o] = 0.f;
        }
        return;
    }
    TransLoader<C::BM, C::NT> la;
    TransLoader<C::BN, C::NT> lb;
    la.init(tid);
    lb.init(tid);
    const int nk = (int)ceil_div(cnt, BK);
    Acc<C> acc;
    mainloop<C>(
        lds, nk,
        [&](int s, char *dst, bool ld, bool st) {
            if (ld)
                la.load(r0, R,
                        [&](int kk) -> const uint16_t * {
                            const int64_t m = seg0 + (int64_t)s * BK + kk;
                            if (m >= seg1) return nullptr;
                            if (UP) return g.dh + m * 2 * I;
                            return g.dy + (int64_t)(g.row_map[m] / g.k) * H;
                        },
                        [&](int kk) -> float {
                            if (UP) return 1.0f;
                            const int64_t m = seg0 + (int64_t)s * BK + kk;
                            return m < seg1 ? g.topk_w[g.row_map[m]] : 1.0f;
                        });
            if (st) la.store(dst);
        },
        [&](int s, char *dst, bool ld, bool st) {
            if (ld)
                lb.load(c0, Cc,
                        [&](int kk) -> const uint16_t * {
                            const int64_t m = seg0 + (int64_t)s * BK + kk;
                            if (m >= seg1) return nullptr;
                            if (UP) return g.x + (int64_t)(g.row_map[m] / g.k) * H;
                            return g.a + m * I;
                        },
                        [](int) { return 1.0f; });
            if (st) lb.store(dst);
        },
        acc);
#pragma unroll
    for (int i = 0; i < C::FM; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int64_t rr = r0 + acc_row<C>(wm, i, r, lane);
            if (rr >= R) continue;
#pragma unroll
            for (int j = 0; j < C::FN; ++j) {
                const int64_t cc = c0 + acc_col<C>(wn, j, lane);
                if (cc >= Cc) continue;
                const int64_t o = dW_off + rr * Cc + cc;
                float v = acc.v[i][j][r];
                if (g.dw_bf16) {
                    uint16_t *p = (uint16_t *)dWv;
                    if (g.dw_acc) v += bf2f(p[o]);
                    p[o] = f2bf(v);
                } else {
                    float *p = (float *)dWv;
                    if (g.dw_acc) v += p[o];
                    p[o] = v;
                }
            }
        }
}

// ----------------------------------------------------------------- launch ----
using Big = TileCfg<256, 256, 128, 128>;  // 4 waves, 128x128 per wave

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
        int64_t total = (int64_t)g.E * ceil_div(g.H, C::BM) * ceil_div(g.I, C::BN);
        return launch_k(k_wgrad<C, false>, ceil_div(total, 8) * 8, g, s, C::NT);
    }
    case MOE_GEMM_UP_WGRAD: {
        int64_t total = (int64_t)g.E * ceil_div(2 * g.I, C::BM) * ceil_div(g.H, C::BN);
        return launch_k(k_wgrad<C, true>, ceil_div(total, 8) * 8, g, s, C::NT);
    }
    default:
        return hipErrorInvalidValue;
    }
}

}  // namespace moe
