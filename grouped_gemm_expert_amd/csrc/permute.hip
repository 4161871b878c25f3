// Dispatch bookkeeping on one GPU: per-chunk expert histograms, a scan that
// turns them into counts / offsets / per-chunk bases, and a stable scatter
// that writes row_map (sorted row -> flat slot) and pos (its inverse).
// Integer-only and deterministic: the result is the unique stable order
// (experts ascending, flat slots ascending inside one expert).
//
// The one-GPU form of the MegaMoE page's token dispatch (intro: dispatch is
// fused into the first grouped GEMM; here the GEMM gathers rows through
// row_map, so no permuted copy of the tokens is written).
#include "common.h"

namespace moe {

constexpr int PM_CHUNK = 1024;   // flat slots per block
constexpr int PM_THREADS = 256;  // 4 waves x 256 slots (4 rounds of 64)
constexpr int PM_EMAX = 1024;

int64_t permute_chunks(int64_t M) { return ceil_div(M, PM_CHUNK); }

// chunk_hist[e * nchunks + c] = slots of chunk c routed to expert e.
// CHECKED: a slot whose expert lies outside [0, E) is read as data only and
// counted in row E (the caller's histogram area then has E + 1 rows); no
// address is ever formed from it.
template <bool CHECKED>
__global__ __launch_bounds__(PM_THREADS) void k_hist(int64_t M, int32_t E, const int32_t *idx,
                                                      int32_t *chunk_hist, int64_t nchunks)
{
    __shared__ int32_t hist[PM_EMAX + 1];
    for (int e = threadIdx.x; e <= E; e += PM_THREADS) hist[e] = 0;
    __syncthreads();
    const int64_t base = (int64_t)blockIdx.x * PM_CHUNK;
#pragma unroll
    for (int i = 0; i < PM_CHUNK / PM_THREADS; ++i) {
        int64_t f = base + threadIdx.x + i * PM_THREADS;
        if (f < M) {
            int32_t v = idx[f];
            if (CHECKED && (uint32_t)v >= (uint32_t)E) v = E;
            atomicAdd(&hist[v], 1);
        }
    }
    __syncthreads();
    const int rows = CHECKED ? E + 1 : E;
    for (int e = threadIdx.x; e < rows; e += PM_THREADS)
        chunk_hist[(int64_t)e * nchunks + blockIdx.x] = hist[e];
}

// Block-wide exclusive scan for 1024 threads (16 waves).
MOE_DEV int32_t block_excl_scan_1024(int32_t v, int32_t *tmp /* >= 16 */, int32_t &total)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int32_t incl = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        int32_t o = __shfl_up(incl, off, 64);
        if (lane >= off) incl += o;
    }
    if (lane == 63) tmp[wave] = incl;
    __syncthreads();
    int32_t wbase = 0, all = 0;
    for (int w = 0; w < 16; ++w) {
        int32_t tw = tmp[w];
        if (w < wave) wbase += tw;
        all += tw;
    }
    __syncthreads();
    total = all;
    return wbase + incl - v;
}

// One wave per histogram row (expert e, or with CHECKED the out-of-range row
// E): the row's chunk counts become exclusive chunk bases in place, 64
// chunks per step with a running carry, and its total goes to counts[e]
// (row E: *n_bad).
constexpr int SC_WAVES = 4;
__global__ __launch_bounds__(64 * SC_WAVES) void k_scan_rows(int32_t rows, int32_t E,
                                                             int32_t *chunk_hist, int64_t nchunks,
                                                             int32_t *counts, int32_t *n_bad)
{
    const int lane = threadIdx.x & 63;
    const int e = blockIdx.x * SC_WAVES + (threadIdx.x >> 6);
    if (e >= rows) return;  // wave-uniform
    int32_t *row = chunk_hist + (int64_t)e * nchunks;
    int32_t carry = 0;
    for (int64_t c0 = 0; c0 < nchunks; c0 += 64) {
        const int64_t c = c0 + lane;
        const int32_t v = c < nchunks ? row[c] : 0;
        int32_t incl = v;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            int32_t o = __shfl_up(incl, off, 64);
            if (lane >= off) incl += o;
        }
        if (c < nchunks) row[c] = carry + incl - v;
        carry += __shfl(incl, 63, 64);
    }
    if (lane == 0) {
        if (e < E) counts[e] = carry;
        else *n_bad = carry;
    }
}

// Stable scatter.  Every block first turns counts into the exclusive expert
// offsets in LDS (block 0 also writes them out, offsets[E] = the number of
// slots placed).  Wave w of block c then handles flat slots
// [c*1024 + w*256, +256) in 4 rounds of 64 lanes; ranks inside a round come
// from a match mask built with one ballot per key bit, ranks across rounds
// from per-wave running counters in LDS, ranks across waves from a prefix
// over those counters, and ranks across chunks from the scanned histogram.
// CHECKED: a slot whose expert lies outside [0, E) takes the key of "no
// slot" (it is placed nowhere) and gets pos = -1.
template <bool CHECKED>
__global__ __launch_bounds__(1024) void k_scatter(int64_t M, int32_t E, const int32_t *idx,
                                                  const int32_t *chunk_base, int64_t nchunks,
                                                  const int32_t *counts, int32_t *offsets,
                                                  int32_t *row_map, int32_t *pos)
{
    __shared__ int32_t cnt[16][PM_EMAX];
    __shared__ int32_t off_s[PM_EMAX];
    __shared__ int32_t tmp[16];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int e0 = threadIdx.x;
    {
        int32_t total;
        const int32_t o = block_excl_scan_1024(e0 < E ? counts[e0] : 0, tmp, total);
        if (e0 < E) off_s[e0] = o;
        if (blockIdx.x == 0) {
            if (e0 < E) offsets[e0] = o;
            if (e0 == 0) offsets[E] = total;
        }
    }
    for (int e = threadIdx.x; e < E; e += 1024)
#pragma unroll
        for (int w = 0; w < 16; ++w) cnt[w][e] = 0;
    __syncthreads();

    // 16 waves x 64 slots: one round of 64 lanes each
    const int64_t f = (int64_t)blockIdx.x * PM_CHUNK + wave * 64 + lane;
    const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    int32_t kv = PM_EMAX;  // 11-bit key; PM_EMAX = no slot
    if (f < M) {
        kv = idx[f];
        if (CHECKED && (uint32_t)kv >= (uint32_t)E) {
            kv = PM_EMAX;
            pos[f] = -1;
        }
    }
    uint64_t match = ~0ull;
#pragma unroll
    for (int b = 0; b < 11; ++b) {
        uint64_t bb = __ballot((kv >> b) & 1);
        match &= ((kv >> b) & 1) ? bb : ~bb;
    }
    const int32_t rank = __popcll(match & lt_mask);
    // the lowest lane of each key group writes the wave's count of that key
    if (kv < PM_EMAX && rank == 0) cnt[wave][kv] = __popcll(match);
    __syncthreads();
    if (kv >= PM_EMAX) return;
    int32_t wb = 0;
    for (int w = 0; w < wave; ++w) wb += cnt[w][kv];
    const int32_t dst = off_s[kv] + chunk_base[(int64_t)kv * nchunks + blockIdx.x] + wb + rank;
    row_map[dst] = (int32_t)f;
    pos[f] = dst;
}

template <bool CHECKED>
static hipError_t permute_impl(int64_t M, int32_t E, const int32_t *idx, int32_t *counts,
                               int32_t *offsets, int32_t *row_map, int32_t *pos,
                               int32_t *chunk_hist, int32_t *n_bad, hipStream_t s)
{
    const int64_t nch = permute_chunks(M);
    if (nch > 0) {
        k_hist<CHECKED><<<(unsigned)nch, PM_THREADS, 0, s>>>(M, E, idx, chunk_hist, nch);
        hipError_t err = hipGetLastError();
        if (err != hipSuccess) return err;
    }
    const int32_t rows = CHECKED ? E + 1 : E;
    if (nch > 0) {
        k_scan_rows<<<(unsigned)ceil_div(rows, SC_WAVES), 64 * SC_WAVES, 0, s>>>(
            rows, E, chunk_hist, nch, counts, n_bad);
    } else {
        // no slots: zero counts (and the out-of-range count)
        hipError_t err = launch_fill_i32(counts, E, 0, s);
        if (err != hipSuccess) return err;
        if (CHECKED) err = launch_fill_i32(n_bad, 1, 0, s);
        if (err != hipSuccess) return err;
        // offsets from the zero counts
        k_scatter<CHECKED><<<1, 1024, 0, s>>>(0, E, idx, chunk_hist, 0, counts, offsets,
                                              row_map, pos);
        return hipGetLastError();
    }
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    if (CHECKED) {
        // rows past the placed slots hold -1
        err = launch_fill_i32(row_map, M, -1, s);
        if (err != hipSuccess) return err;
    }
    k_scatter<CHECKED><<<(unsigned)nch, 1024, 0, s>>>(M, E, idx, chunk_hist, nch, counts, offsets,
                                                      row_map, pos);
    return hipGetLastError();
}

hipError_t launch_permute(int64_t M, int32_t E, const int32_t *idx, int32_t *counts,
                          int32_t *offsets, int32_t *row_map, int32_t *pos,
                          int32_t *chunk_hist, hipStream_t s)
{
    return permute_impl<false>(M, E, idx, counts, offsets, row_map, pos, chunk_hist, nullptr, s);
}

hipError_t launch_permute_checked(int64_t M, int32_t E, const int32_t *idx, int32_t *counts,
                                  int32_t *offsets, int32_t *row_map, int32_t *pos,
                                  int32_t *chunk_hist, int32_t *n_bad, hipStream_t s)
{
    return permute_impl<true>(M, E, idx, counts, offsets, row_map, pos, chunk_hist, n_bad, s);
}

// ------------------------------------------------------------- schedule ----
// mt_off*[e] = sum_{e' < e} ceil(counts[e'] / BM) for BM = 256 and 128,
// mt_a / mt_b the same sums of the mixed m-tiling's 256-row and 320-row
// tile counts (mixed_head_tiles / mixed_tail_tiles),
// order[] = the experts with rows in the order the weight-gradient GEMMs
// visit them, and order[E] = their number (the empty experts follow).
// Experts are ranked by count descending (ties -> lower expert index).  With
// SHORT_ROWS > 0 the experts with fewer rows than that (their tiles are
// mostly the fp32 read-modify-write of dW, memory-bound) are spread among
// the longer ones (MFMA-bound) instead of all coming last: short expert j
// goes after long expert ceil((j+1) nb / ns) - 1 (nb long, ns short), so
// the memory-bound tiles run beside MFMA-bound ones and the launch still
// ends on short tiles.  Measured against all short experts last: the
// DeepSeek-V3-style routing's dW2 pass 1.5% faster (5 short experts of 14;
// with a 1024-row threshold, 4 of them, 2% slower), the Zipf-skewed one's
// weight gradients 2-5% faster.
#ifndef MOE_WGRAD_SHORT_ROWS
#define MOE_WGRAD_SHORT_ROWS 2048
#endif
constexpr int32_t WGRAD_SHORT_ROWS = MOE_WGRAD_SHORT_ROWS;

__global__ __launch_bounds__(1024) void k_schedule(int32_t E, const int32_t *counts,
                                                   int32_t *mt256, int32_t *mt128,
                                                   int32_t *order, int32_t *mt_a, int32_t *mt_b)
{
    __shared__ int32_t tmp[16];
    __shared__ int32_t sc[PM_EMAX];
    const int e = threadIdx.x;
    int32_t c = (e < E) ? counts[e] : 0;
    if (e < E) sc[e] = c;
    int32_t total;
    int32_t o256 = block_excl_scan_1024((c + 255) / 256, tmp, total);
    if (e < E) mt256[e] = o256;
    if (e == E - 1) mt256[E] = total;
    int32_t o128 = block_excl_scan_1024((c + 127) / 128, tmp, total);
    if (e < E) mt128[e] = o128;
    if (e == E - 1) mt128[E] = total;
    const int32_t oa = block_excl_scan_1024(mixed_head_tiles(c), tmp, total);
    if (e < E) mt_a[e] = oa;
    if (e == E - 1) mt_a[E] = total;
    const int32_t ob = block_excl_scan_1024(mixed_tail_tiles(c), tmp, total);
    if (e < E) mt_b[e] = ob;
    if (e == E - 1) mt_b[E] = total;
    __syncthreads();
    // rank of expert er: S threads (consecutive lanes of one wave) each count
    // the experts ahead of it among every S-th one, then add up by shuffles
    int S = 1;
    while (S < 64 && 2 * S * E <= 1024) S *= 2;
    const int er = e / S, part = e % S;
    int32_t rank = 0;
    if (er < E) {
        const int32_t ce = sc[er];
        for (int j = part; j < E; j += S) {
            const int32_t cj = sc[j];
            rank += (cj > ce) || (cj == ce && j < er);
        }
    }
    for (int off = 1; off < S; off <<= 1) rank += __shfl_xor(rank, off, 64);
    int32_t nact, nlong;
    block_excl_scan_1024((e < E && c > 0) ? 1 : 0, tmp, nact);
    block_excl_scan_1024((e < E && c >= WGRAD_SHORT_ROWS && c > 0) ? 1 : 0, tmp, nlong);
    if (er < E && part == 0) {
        int32_t p = rank;
        const int32_t ns = nact - nlong;
        if (WGRAD_SHORT_ROWS > 0 && nlong > 0 && ns > 0 && rank < nact) {
            if (rank < nlong) {
                const int32_t sb = (int32_t)(((int64_t)rank * ns) / nlong);  // short ones before
                p = rank + (sb < ns ? sb : ns);
            } else {
                const int32_t j = rank - nlong;
                p = (int32_t)(((int64_t)(j + 1) * nlong + ns - 1) / ns) + j;
            }
        }
        order[p] = er;
    }
    if (e == 0) order[E] = nact;
}

hipError_t launch_schedule(int32_t E, const int32_t *counts, const Sched &sc, hipStream_t s)
{
    k_schedule<<<1, 1024, 0, s>>>(E, counts, sc.mt_off256, sc.mt_off128, sc.order, sc.mt_a,
                                  sc.mt_b);
    return hipGetLastError();
}

}  // namespace moe
