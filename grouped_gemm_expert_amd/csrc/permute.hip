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

// chunk_hist[e * nchunks + c] = slots of chunk c routed to expert e
__global__ __launch_bounds__(PM_THREADS) void k_hist(int64_t M, int32_t E, const int32_t *idx,
                                                      int32_t *chunk_hist, int64_t nchunks)
{
    __shared__ int32_t hist[PM_EMAX];
    for (int e = threadIdx.x; e < E; e += PM_THREADS) hist[e] = 0;
    __syncthreads();
    const int64_t base = (int64_t)blockIdx.x * PM_CHUNK;
#pragma unroll
    for (int i = 0; i < PM_CHUNK / PM_THREADS; ++i) {
        int64_t f = base + threadIdx.x + i * PM_THREADS;
        if (f < M) atomicAdd(&hist[idx[f]], 1);
    }
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += PM_THREADS)
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

// One block of 1024 threads: thread e turns its row of chunk_hist into
// exclusive chunk bases (in place) and its count; then offsets = exclusive
// scan of counts.
__global__ __launch_bounds__(1024) void k_scan(int32_t E, int64_t M, int32_t *chunk_hist,
                                               int64_t nchunks, int32_t *counts,
                                               int32_t *offsets)
{
    __shared__ int32_t tmp[16];
    const int e = threadIdx.x;
    int32_t run = 0;
    if (e < E) {
        int32_t *row = chunk_hist + (int64_t)e * nchunks;
        for (int64_t c = 0; c < nchunks; ++c) {
            int32_t v = row[c];
            row[c] = run;
            run += v;
        }
        counts[e] = run;
    }
    int32_t total;
    int32_t off = block_excl_scan_1024(e < E ? run : 0, tmp, total);
    if (e < E) offsets[e] = off;
    if (e == 0) offsets[E] = (int32_t)M;
}

// Stable scatter.  Wave w of block c handles flat slots
// [c*1024 + w*256, +256) in 4 rounds of 64 lanes; ranks inside a round come
// from a match mask built with one ballot per key bit, ranks across rounds
// from per-wave running counters in LDS, ranks across waves from a prefix
// over those counters, and ranks across chunks from the scanned histogram.
__global__ __launch_bounds__(PM_THREADS) void k_scatter(int64_t M, int32_t E,
                                                         const int32_t *idx,
                                                         const int32_t *chunk_base,
                                                         int64_t nchunks,
                                                         const int32_t *offsets,
                                                         int32_t *row_map, int32_t *pos)
{
    __shared__ int32_t cnt[4][PM_EMAX];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    for (int e = threadIdx.x; e < E; e += PM_THREADS)
#pragma unroll
        for (int w = 0; w < 4; ++w) cnt[w][e] = 0;
    __syncthreads();

    const int64_t base = (int64_t)blockIdx.x * PM_CHUNK + wave * 256;
    const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    int32_t key[4], rank[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        int64_t f = base + r * 64 + lane;
        int32_t kv = (f < M) ? idx[f] : PM_EMAX;  // 11-bit key; PM_EMAX = no slot
        uint64_t match = ~0ull;
#pragma unroll
        for (int b = 0; b < 11; ++b) {
            uint64_t bb = __ballot((kv >> b) & 1);
            match &= ((kv >> b) & 1) ? bb : ~bb;
        }
        int32_t before = __popcll(match & lt_mask);
        int32_t run = (kv < PM_EMAX) ? cnt[wave][kv] : 0;
        __builtin_amdgcn_wave_barrier();
        // the lowest lane of each key group advances the wave's counter
        if (kv < PM_EMAX && before == 0) cnt[wave][kv] = run + __popcll(match);
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        key[r] = kv;
        rank[r] = run + before;
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        int32_t kv = key[r];
        if (kv >= PM_EMAX) continue;
        int32_t wb = 0;
        for (int w = 0; w < wave; ++w) wb += cnt[w][kv];
        int64_t f = base + r * 64 + lane;
        int32_t dst = offsets[kv] + chunk_base[(int64_t)kv * nchunks + blockIdx.x] + wb + rank[r];
        row_map[dst] = (int32_t)f;
        pos[f] = dst;
    }
}

hipError_t launch_permute(int64_t M, int32_t E, const int32_t *idx, int32_t *counts,
                          int32_t *offsets, int32_t *row_map, int32_t *pos,
                          int32_t *chunk_hist, hipStream_t s)
{
    int64_t nch = permute_chunks(M);
    if (nch > 0) {
        k_hist<<<(unsigned)nch, PM_THREADS, 0, s>>>(M, E, idx, chunk_hist, nch);
        hipError_t err = hipGetLastError();
        if (err != hipSuccess) return err;
    }
    k_scan<<<1, 1024, 0, s>>>(E, M, chunk_hist, nch, counts, offsets);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess || nch == 0) return err;
    k_scatter<<<(unsigned)nch, PM_THREADS, 0, s>>>(M, E, idx, chunk_hist, nch, offsets, row_map,
                                                    pos);
    return hipGetLastError();
}

// ------------------------------------------------------------- schedule ----
// mt_off*[e] = sum_{e' < e} ceil(counts[e'] / BM) for BM = 256 and 128,
// order[] = experts by count descending (ties -> lower expert index), so the
// weight-gradient GEMMs start the longest K loops first, and order[E] = the
// number of experts with at least one row (they come first in order[]).
__global__ __launch_bounds__(1024) void k_schedule(int32_t E, const int32_t *counts,
                                                   int32_t *mt256, int32_t *mt128,
                                                   int32_t *order)
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
    __syncthreads();
    if (e < E) {
        int32_t rank = 0;
        for (int j = 0; j < E; ++j) {
            int32_t cj = sc[j];
            rank += (cj > c) || (cj == c && j < e);
        }
        order[rank] = e;
    }
    int32_t nact;
    block_excl_scan_1024((e < E && c > 0) ? 1 : 0, tmp, nact);
    if (e == 0) order[E] = nact;
}

hipError_t launch_schedule(int32_t E, const int32_t *counts, const Sched &sc, hipStream_t s)
{
    k_schedule<<<1, 1024, 0, s>>>(E, counts, sc.mt_off256, sc.mt_off128, sc.order);
    return hipGetLastError();
}

}  // namespace moe
