// Per-expert (or per-batch) transposes of row-major operands, 128 rows x 64
// columns a block: which rows a block takes, and their load into LDS.  Shared
// by the MXFP8 column quantiser (mx.hip) and the bf16 weight-gradient operand
// transposer (gemm.hip); both then read a column per thread out of the tile.
#pragma once

#include "common.h"

namespace moe {

constexpr int SEG_ROWS = 128;  // rows of a segment chunk: one 128-deep k group

// Chunk L of the transposes that q describes (see ColQuant):
//   seg   the segment (batch, or expert with rows)
//   j     the 128-row chunk inside it; r0 its first source row index (sorted
//         row, or batch row), len <= 128 the rows it has
//   Kp    the segment's rows rounded up to 128 (the transposed matrix's k)
//   chunk0  chunks before this segment's (its data starts C * 128 * chunk0
//         elements into the destination in expert mode)
struct SegPos {
    int64_t seg, j, r0, len, Kp, chunk0;
};

// The chunk prefix sums (expert mode) into LDS: one cooperative load, so
// that locating a chunk costs no chain of dependent global loads.  Every
// thread calls it; the caller synchronises before seg_locate.
constexpr int SEG_MAX_E = 1024;
MOE_DEV void seg_stage_table(const ColQuant &q, int32_t *mt_s)
{
    if (!q.offsets) return;
    for (int i = threadIdx.x; i <= q.nseg; i += blockDim.x) mt_s[i] = q.mt128[i];
}

// False when L is past the last chunk (the whole block exits).  mt_s: the
// table seg_stage_table staged.
MOE_DEV bool seg_locate(const ColQuant &q, const int32_t *mt_s, int64_t L, SegPos &p)
{
    if (!q.offsets) {
        p.Kp = ceil_div(q.R, SEG_ROWS) * SEG_ROWS;
        const int64_t per = p.Kp / SEG_ROWS;
        if (L >= (int64_t)q.nseg * per) return false;
        p.seg = L / per;
        p.j = L % per;
        p.r0 = p.seg * q.R + p.j * SEG_ROWS;
        const int64_t rem = q.R - p.j * SEG_ROWS;
        p.len = rem < SEG_ROWS ? rem : SEG_ROWS;
        p.chunk0 = p.seg * per;
        return true;
    }
    if (L >= mt_s[q.nseg]) return false;
    int lo = 0, hi = q.nseg;  // largest e with mt128[e] <= L: an expert with rows
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (mt_s[mid] <= L) lo = mid; else hi = mid;
    }
    p.seg = lo;
    p.j = L - mt_s[lo];
    p.r0 = q.offsets[lo] + p.j * SEG_ROWS;
    const int64_t rem = q.offsets[lo + 1] - p.r0;
    p.len = rem < SEG_ROWS ? rem : SEG_ROWS;
    p.Kp = (int64_t)SEG_ROWS * (mt_s[lo + 1] - mt_s[lo]);
    p.chunk0 = mt_s[lo];
    return true;
}

// Rows r0 .. r0+len-1, columns 64 ct .. 64 ct + 63 of the source into
// tile[128][W] (rows gathered through q.gather / q.gk and scaled by q.rw,
// rounded to bf16, when given); rows past len are zero.  All 256 threads
// take part, 4 chunks of 16 bytes each: the row indices and weights of all
// four are loaded first, then the four data loads issued together, so a
// thread waits for two memory round trips, not eight.  The caller
// synchronises before reading the tile.  W = 64: 16-byte LDS writes; a
// padded W (66) takes 4-byte ones.
// SPLIT (bf16 transposer): the values are formed in fp32 as
// (src + src_lo) * rw and stored as bf16(v), or with q.lo_part as the
// remainder bf16(v - bf16(v)).
template <int W, int NCT = 1, bool SPLIT = false>
MOE_DEV void seg_load_tile(const ColQuant &q, const SegPos &p, int ct, uint16_t (*tile)[W])
{
    // NCT adjacent column tiles (ct .. ct+NCT-1) into tile[NCT*128][W]: one
    // source row then yields NCT*128 contiguous bytes, all loads issued together
    constexpr int NU = SEG_ROWS * 8 / 256 * NCT;
    // row indices: the branches are uniform and outside the unrolled loops,
    // so each batch of loads issues back to back; rows past len read row 0
    // of the chunk and are zeroed below
    int64_t rr[NU], sr[NU];
    float wr[NU];
#pragma unroll
    for (int u = 0; u < NU; ++u) {
        const int r = ((threadIdx.x + 256 * u) >> 3) % SEG_ROWS;
        rr[u] = p.r0 + (r < p.len ? r : 0);
        sr[u] = rr[u];
        wr[u] = 1.f;
    }
    if (q.gather) {
        int32_t gi[NU];
#pragma unroll
        for (int u = 0; u < NU; ++u) gi[u] = q.gather[rr[u]];
#pragma unroll
        for (int u = 0; u < NU; ++u) sr[u] = gi[u] / q.gk;
    }
    if (q.rw) {
#pragma unroll
        for (int u = 0; u < NU; ++u) wr[u] = q.rw[rr[u]];
    }
    u32x4_t v[NU], vl[SPLIT ? NU : 1];
#pragma unroll
    for (int u = 0; u < NU; ++u) {
        const int qd = (threadIdx.x + 256 * u) & 7, t = (threadIdx.x + 256 * u) / (SEG_ROWS * 8);
        v[u] = *(const u32x4_t *)(q.src + sr[u] * q.C + (ct + t) * 64 + qd * 8);
        if constexpr (SPLIT)
            vl[u] = q.src_lo ? *(const u32x4_t *)(q.src_lo + sr[u] * q.C + (ct + t) * 64 + qd * 8)
                             : u32x4_t{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < NU; ++u)
        if ((((threadIdx.x + 256 * u) >> 3) % SEG_ROWS) >= p.len) v[u] = u32x4_t{0u, 0u, 0u, 0u};
#pragma unroll
    for (int u = 0; u < NU; ++u) {
        // tile row r of column tile t lands in row t*128 + r
        const int i = threadIdx.x + 256 * u, r = i >> 3, qd = i & 7;
        u32x4_t x = v[u];
        if constexpr (SPLIT) {
            // v = (src + src_lo) * rw in fp32, then its bf16 part or remainder
            const bool pad = ((i >> 3) % SEG_ROWS) >= p.len;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                float f0 = bf2f((uint16_t)(x[e] & 0xffffu)), f1 = bf2f((uint16_t)(x[e] >> 16));
                if (q.src_lo && !pad) {
                    f0 += bf2f((uint16_t)(vl[u][e] & 0xffffu));
                    f1 += bf2f((uint16_t)(vl[u][e] >> 16));
                }
                if (q.rw) {
                    f0 *= wr[u];
                    f1 *= wr[u];
                }
                if (q.lo_part) {
                    f0 -= bf2f(f2bf(f0));
                    f1 -= bf2f(f2bf(f1));
                }
                x[e] = pack_bf2(f0, f1);
            }
        } else if (q.rw) {
#pragma unroll
            for (int e = 0; e < 4; ++e)
                x[e] = pack_bf2(wr[u] * bf2f((uint16_t)(x[e] & 0xffffu)), wr[u] * bf2f((uint16_t)(x[e] >> 16)));
        }
        if constexpr (W % 8 == 0) {
            *(u32x4_t *)&tile[r][qd * 8] = x;
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) *(uint32_t *)&tile[r][qd * 8 + 2 * e] = x[e];
        }
    }
}

}  // namespace moe
