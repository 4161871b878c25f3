// Router GEMMs on bf16 MFMA with fp32-accurate products.
//
// The router works in fp32: logits l = x . Wr^T (x bf16, Wr fp32), and in the
// backward dWr = dl^T . x and dx += dl . Wr (dl fp32).  Each fp32 operand is
// split exactly into three bf16 parts, v = hi + mid + lo (each part the
// round-to-nearest bf16 of what the previous parts leave), so that every
// product of two parts is exact in fp32 and the MFMA's fp32 accumulation
// gives the sum with fp32 rounding, as a plain fp32 GEMM would.  The logits
// decide the routing and take all three parts; the gradients feed no
// decision and take the first two (hi + mid holds 16 of the 24 significand
// bits: each product is within 2^-15 of its fp32 value, relative):
//   l   = sum_p  x  . Wr_p^T                      (3 products)
//   dWr = sum_{p<2}  dl_p^T . x                    (2 products)
//   dx += sum_{p+q<=1} dl_p . Wr_q                 (3 products)
// The products run as one pipeline over a concatenated list of K stages;
// outputs with few tiles split that list over several blocks (split-K) whose
// partial sums a second kernel adds in a fixed order, so results are
// deterministic.
#include "bwd_epi.h"

namespace moe {

constexpr int DENSE_MAX_TERMS = 6;

struct DenseArgs {
    int64_t M, N, K;   // C is M x N; every term sums over K
    int64_t lda, ldb;  // elements per row of the A / B part arrays
    int32_t nterms, splits;
    int64_t spt;       // stages per term, ceil(K / 64)
    const uint16_t *A[DENSE_MAX_TERMS], *B[DENSE_MAX_TERMS];
    float *C;          // splits == 1: C (+)= A . B^T, row stride N
    int32_t accumulate;
    float *part;       // splits > 1: part[s][M][N]
};

using DenseTile = TileCfg<256, 256, 64, 128>;

// Tile (mt, nt) and split s of block b.  A-operand rows come from A_NMAJ ?
// k-rows of lda elements (element (m, k) at A[k * lda + m]) : m-rows (element
// (m, k) at A[m * lda + k]); likewise for B with n.
template <class C, bool A_NMAJ, bool B_NMAJ>
__global__ __launch_bounds__(C::NT) void k_dense(DenseArgs d)
{
    __shared__ __attribute__((aligned(16))) char lds_raw[C::LDS_BYTES];
    lds_t *lds = (lds_t *)lds_raw;
    const int64_t tM = ceil_div(d.M, C::BM), tN = ceil_div(d.N, C::BN);
    const int64_t L = xcd_remap(blockIdx.x, tM * tN * d.splits);
    if (L < 0) return;
    const int s = (int)(L % d.splits);
    const int64_t tile = L / d.splits;
    const int64_t m0 = (tile / tN) * C::BM, n0 = (tile % tN) * C::BN;
    const int64_t nst = d.spt * d.nterms;
    const int v0 = (int)(nst * s / d.splits), v1 = (int)(nst * (s + 1) / d.splits);

    const int tid = threadIdx.x, lane = tid & 63, wave0 = wave_uniform_id();
    typename std::conditional<A_NMAJ, NLoad<C::BM, C::NT>, KLoad<C::BM, C::NT>>::type la;
    typename std::conditional<B_NMAJ, NLoad<C::BN, C::NT>, KLoad<C::BN, C::NT>>::type lb;
    if constexpr (A_NMAJ) {
        la.init(nullptr, d.lda, m0, d.M, wave0, lane);
    } else {
        la.init(nullptr, wave0);
#pragma unroll
        for (int q = 0; q < la.NI; ++q) {
            int64_t m = m0 + la.row(q, lane);
            if (m >= d.M) m = d.M - 1;
            la.set(q, lane, (uint32_t)(m * d.lda * 2));
        }
    }
    if constexpr (B_NMAJ) {
        lb.init(nullptr, d.ldb, n0, d.N, wave0, lane);
    } else {
        lb.init(nullptr, wave0);
#pragma unroll
        for (int q = 0; q < lb.NI; ++q) {
            int64_t n = n0 + lb.row(q, lane);
            if (n >= d.N) n = d.N - 1;
            lb.set(q, lane, (uint32_t)(n * d.ldb * 2));
        }
    }
    auto kvalid = [&](int v) -> int {
        const int64_t rem = d.K - (v % d.spt) * BK;
        return rem < BK ? (int)rem : BK;
    };
    Acc<C> acc;
    pipeline<C, A_NMAJ, B_NMAJ, decltype(la)::NI, decltype(lb)::NI>(
        lds, v0, v1,
        [&](int q, int v, lds_t *As) {
            la.issue_one(q, As, (v % d.spt) * BK, kvalid(v), (const char *)d.A[v / d.spt]);
        },
        [&](int q, int v, lds_t *Bs) {
            lb.issue_one(q, Bs, (v % d.spt) * BK, kvalid(v), (const char *)d.B[v / d.spt]);
        },
        [&](int v, lds_t *As, lds_t *Bs) {
            // K-major operands are read from rows padded with zeros past K
            const int kv = kvalid(v);
            if (kv < BK) {
                la.zero_tail(As, kv);
                lb.zero_tail(Bs, kv);
            }
        },
        acc);

    float *out = d.splits > 1 ? d.part + (int64_t)s * d.M * d.N : d.C;
    const bool add = d.splits == 1 && d.accumulate;
    const bool vec = (d.N & 3) == 0;
    if (vec) {
        // through the LDS staging tile: row-contiguous 16-byte loads (when
        // adding) and stores, 4 rows a wave at a time
        wgrad_epilogue<C, 4>(acc, lds, m0, n0, (int)d.M, (int)d.N, 0, out, add ? 1 : 0, 0);
        return;
    }
    const int wm = (tid >> 6) / C::WAVES_N, wn = (tid >> 6) % C::WAVES_N;
#pragma unroll
    for (int i = 0; i < C::FM; ++i) {
        const int64_t m = m0 + acc_row<C>(wm, i, lane);
        if (m >= d.M) continue;
#pragma unroll
        for (int j = 0; j < C::FN; ++j)
#pragma unroll
            for (int rg = 0; rg < 4; ++rg) {
                const int64_t col = n0 + acc_col<C>(wn, j, rg, lane);
                if (col >= d.N) continue;
                float *p = out + m * d.N + col;
                f32x4_t v = {acc.v[i][j][rg * 4], acc.v[i][j][rg * 4 + 1], acc.v[i][j][rg * 4 + 2],
                             acc.v[i][j][rg * 4 + 3]};
                if (vec) {
                    if (add) v += *(f32x4_t *)p;
                    *(f32x4_t *)p = v;
                } else {
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        if (col + q < d.N) p[q] = add ? p[q] + v[q] : v[q];
                }
            }
    }
}

// C[i] (+)= sum_s part[s][i], s ascending.
__global__ __launch_bounds__(256) void k_reduce_splits(int64_t n, int32_t splits, const float *part,
                                                       float *C, int32_t accumulate)
{
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * blockDim.x) {
        float v = accumulate ? C[i] : 0.f;
        for (int s = 0; s < splits; ++s) v += part[(int64_t)s * n + i];
        C[i] = v;
    }
}

// out[p][r][c] = part p of src[r][c] (c < cols), 0 for cols <= c < ld_out:
// hi = bf16(v), mid = bf16(v - hi), lo = bf16(v - hi - mid), each difference
// exact in fp32.
__global__ __launch_bounds__(256) void k_split3(int64_t rows, int64_t cols, int64_t ld_out,
                                                const float *src, uint16_t *out)
{
    const int64_t n = rows * ld_out;
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * blockDim.x) {
        const int64_t r = i / ld_out, c = i % ld_out;
        uint16_t h = 0, md = 0, lo = 0;
        if (c < cols) {
            const float v = src[r * cols + c];
            h = f2bf(v);
            const float r1 = v - bf2f(h);
            md = f2bf(r1);
            lo = f2bf(r1 - bf2f(md));
        }
        out[i] = h;
        out[n + i] = md;
        out[2 * n + i] = lo;
    }
}

static int64_t blocks_for(int64_t n) { return ceil_div(n, 256) < 4096 ? ceil_div(n, 256) : 4096; }

// Split count: double while the grid has fewer than 256 blocks and every
// split keeps at least 8 stages.
static int32_t dense_splits(int64_t M, int64_t N, int64_t stages)
{
    using C = DenseTile;
    const int64_t tiles = ceil_div(M, C::BM) * ceil_div(N, C::BN);
    int32_t s = 1;
    while (tiles * s < 256 && stages / (2 * s) >= 8) s *= 2;
    return s;
}

static int64_t pad64(int64_t v) { return ceil_div(v, 64) * 64; }

template <bool A_NMAJ, bool B_NMAJ>
static hipError_t run_dense(DenseArgs d, hipStream_t s)
{
    using C = DenseTile;
    const int64_t total = ceil_div(d.M, C::BM) * ceil_div(d.N, C::BN) * d.splits;
    if (total <= 0) return hipSuccess;
    k_dense<C, A_NMAJ, B_NMAJ><<<(unsigned)grid_for(total), C::NT, 0, s>>>(d);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || d.splits == 1) return e;
    const int64_t n = d.M * d.N;
    k_reduce_splits<<<(unsigned)blocks_for(n), 256, 0, s>>>(n, d.splits, d.part, d.C, d.accumulate);
    return hipGetLastError();
}

static hipError_t split3(int64_t rows, int64_t cols, int64_t ld_out, const float *src, uint16_t *out,
                         hipStream_t s)
{
    const int64_t n = rows * ld_out;
    if (n == 0) return hipSuccess;
    k_split3<<<(unsigned)blocks_for(n), 256, 0, s>>>(rows, cols, ld_out, src, out);
    return hipGetLastError();
}

// ------------------------------------------------------------ workspaces ----
// forward: Wr parts [3][E][H] bf16, logits partials [splits][T][E] fp32
// backward: Wr parts, dl parts [3][T][pad64(E)] bf16, dWr partials
//           [splits][E][H] fp32
static size_t al256(size_t b) { return (b + 255) / 256 * 256; }

size_t router_ws_bytes_fwd(int64_t T, int32_t E, int32_t H)
{
    const int32_t sp = dense_splits(T, E, 3 * ceil_div(H, BK));
    return al256((size_t)3 * E * H * 2) + (sp > 1 ? al256((size_t)sp * T * E * 4) : 0);
}

size_t router_ws_bytes_bwd(int64_t T, int32_t E, int32_t H)
{
    const int32_t sp = dense_splits(E, H, 2 * ceil_div(T, BK));
    return al256((size_t)3 * E * H * 2) + al256((size_t)3 * T * pad64(E) * 2) +
           (sp > 1 ? al256((size_t)sp * E * H * 4) : 0);
}

hipError_t launch_router_logits(int64_t T, int32_t E, int32_t H, const uint16_t *x, const float *Wr,
                                float *logits, void *ws, hipStream_t s)
{
    if (T == 0) return hipSuccess;
    char *p = (char *)ws;
    uint16_t *wsp = (uint16_t *)p;
    p += al256((size_t)3 * E * H * 2);
    hipError_t e = split3(E, H, H, Wr, wsp, s);
    if (e != hipSuccess) return e;
    DenseArgs d = {};
    d.M = T;
    d.N = E;
    d.K = H;
    d.lda = H;
    d.ldb = H;
    d.nterms = 3;
    d.spt = ceil_div(H, BK);
    d.splits = dense_splits(T, E, 3 * d.spt);
    for (int t = 0; t < 3; ++t) {
        d.A[t] = x;
        d.B[t] = wsp + (int64_t)t * E * H;
    }
    d.C = logits;
    d.accumulate = 0;
    d.part = (float *)p;
    return run_dense<false, false>(d, s);
}

hipError_t launch_router_grads(int64_t T, int32_t E, int32_t H, const float *dl, const uint16_t *x,
                               const float *Wr, float *dx, float *dWr, void *ws, hipStream_t s)
{
    if (T == 0) return hipSuccess;
    const int64_t Ep = pad64(E);
    char *p = (char *)ws;
    uint16_t *wsp = (uint16_t *)p;
    p += al256((size_t)3 * E * H * 2);
    uint16_t *dsp = (uint16_t *)p;
    p += al256((size_t)3 * T * Ep * 2);
    hipError_t e = split3(E, H, H, Wr, wsp, s);
    if (e == hipSuccess) e = split3(T, E, Ep, dl, dsp, s);
    if (e != hipSuccess) return e;
    const uint16_t *Wp[3] = {wsp, wsp + (int64_t)E * H, wsp + 2 * (int64_t)E * H};
    const uint16_t *Dp[3] = {dsp, dsp + T * Ep, dsp + 2 * T * Ep};

    // dx[t, h] += sum_e dl[t, e] Wr[e, h]: A = dl parts (t rows, e padded),
    // B(h, e) = Wr parts read along e (N-major)
    DenseArgs d = {};
    d.M = T;
    d.N = H;
    d.K = E;
    d.lda = Ep;
    d.ldb = H;
    const int pq[3][2] = {{0, 0}, {0, 1}, {1, 0}};
    d.nterms = 3;
    for (int t = 0; t < 3; ++t) {
        d.A[t] = Dp[pq[t][0]];
        d.B[t] = Wp[pq[t][1]];
    }
    d.spt = ceil_div(E, BK);
    d.splits = 1;
    d.C = dx;
    d.accumulate = 1;
    e = run_dense<false, true>(d, s);
    if (e != hipSuccess || !dWr) return e;

    // dWr[e, h] = sum_t dl[t, e] x[t, h]: both operands read along t (N-major)
    DenseArgs g = {};
    g.M = E;
    g.N = H;
    g.K = T;
    g.lda = Ep;
    g.ldb = H;
    g.nterms = 2;
    for (int t = 0; t < 2; ++t) {
        g.A[t] = Dp[t];
        g.B[t] = x;
    }
    g.spt = ceil_div(T, BK);
    g.splits = dense_splits(E, H, 2 * g.spt);
    g.C = dWr;
    g.accumulate = 0;
    g.part = (float *)p;
    return run_dense<true, true>(g, s);
}

}  // namespace moe
