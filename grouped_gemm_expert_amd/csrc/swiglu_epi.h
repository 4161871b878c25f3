// SwiGLU epilogue of the GEMM1 tiles (bf16 and MXFP8 kernels): a = silu(g) * u
// from the fp32 accumulators, out through LDS to h (gate | up, bf16) and a
// (bf16), and in the MXFP8 kernels also to a's MX form (the input of GEMM2).
#pragma once

#include "mxfmt.h"
#include "tile.h"

namespace moe {

// B tile rows: wave column wn covers gate columns i0 + wn*WN/2 + [0, WN/2) and
// the matching up columns, so each lane holds g and u of the same (r, i).
// Staging row r holds the tile's 128 gate | 128 up | 128 a values of that row
// as bf16 (48 chunks of 16 bytes, XOR-swizzled by row), and lane l < 48 writes
// chunk l of a row to h (gate, up) or a with one 16-byte store.  With MX,
// lanes 32..47 (the a chunks; 4 lanes a 32-column block, the tile's 128
// columns one scale group) also quantise the bf16 a values of the row and
// write 8 codes each and the group's scale word; columns at or past I are
// quantised as zeros, so the padding of a's MX rows holds zero codes.
// SPLIT: each value v also leaves as the bf16 rounding of its remainder,
// bf16(v - bf16(v)), into h_lo and a_lo (a second pass through the staging
// tile), so that hi + lo carries v to about 16 significant bits.
template <class C, bool MX, bool SPLIT = false>
MOE_DEV void swiglu_epilogue(const Acc<C> &acc, lds_t *lds, const MTile &t, int64_t i0, int I,
                             uint16_t *h, uint16_t *a, uint8_t *aq, uint8_t *as_, int64_t Ip,
                             uint16_t *h_lo = nullptr, uint16_t *a_lo = nullptr)
{
    static_assert(!(MX && SPLIT), "the split intermediates are a bf16-path form");
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave / C::WAVES_N, wn = wave % C::WAVES_N;
    constexpr int HF = C::FN / 2;
    constexpr int GCOLS = C::BN / 2;  // gate columns of the tile
    static_assert(3 * GCOLS == 48 * 8, "staging row = 48 chunks");
    static_assert(!MX || GCOLS == MX_GROUP, "one MX scale group per tile row");
    auto soff = [](int r, int chunk) { return r * (3 * GCOLS * 2) + ((chunk ^ (r & 15)) << 4); };
#pragma unroll
    for (int half = 0; half < C::NHALF; ++half) {
        if (t.m0 + half * EPI_ROWS >= t.seg_end) break;
#pragma unroll
      for (int part = 0; part < (SPLIT ? 2 : 1); ++part) {
#pragma unroll
        for (int i = 0; i < C::FM; ++i) {
            if ((wm * C::WM + i * 32) / EPI_ROWS != half) continue;
            const int r = acc_row<C>(wm, i, lane) - half * EPI_ROWS;
#pragma unroll
            for (int j = 0; j < HF; ++j)
#pragma unroll
                for (int rg = 0; rg < 4; ++rg) {
                    // gate column (tile-local) of wave column wn starts at wn*WN/2
                    const int gc = wn * (C::WN / 2) + j * 32 + rg * 8 + (lane >> 5) * 4;
                    float gv[4], uv[4], av[4];
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        gv[q] = acc.v[i][j][rg * 4 + q];
                        uv[q] = acc.v[i][j + HF][rg * 4 + q];
                        av[q] = gv[q] * sigmoidf_(gv[q]) * uv[q];
                        if (SPLIT && part == 1) {  // the remainders below bf16
                            gv[q] -= bf2f(f2bf(gv[q]));
                            uv[q] -= bf2f(f2bf(uv[q]));
                            av[q] -= bf2f(f2bf(av[q]));
                        }
                    }
                    const int sub = (lane >> 5) << 3;  // byte offset inside the 16-byte chunk
                    *(lds_u64 *)(lds + soff(r, gc >> 3) + sub) = pack_bf4(gv[0], gv[1], gv[2], gv[3]);
                    *(lds_u64 *)(lds + soff(r, 16 + (gc >> 3)) + sub) = pack_bf4(uv[0], uv[1], uv[2], uv[3]);
                    *(lds_u64 *)(lds + soff(r, 32 + (gc >> 3)) + sub) = pack_bf4(av[0], av[1], av[2], av[3]);
                }
        }
        __syncthreads();
        const int seg = lane >> 4;                     // 0 gate, 1 up, 2 a
        const int64_t col = i0 + 8 * (lane & 15);      // column within I
        uint16_t *hd = part ? h_lo : h, *ad = part ? a_lo : a;
        const bool live = lane < 48 && col < I && (seg == 2 || hd != nullptr);
        // RB rows a wave per pass: their LDS reads issued together, then the
        // stores.  The MX form of a: lane l encodes a-chunk l % 16 of the
        // batch's row l / 16, so the four rows take one pass of the encoder
        // (every lane runs it; rows past the segment are masked at the store)
        constexpr int NW = C::NT / 64, RB = 4;
        static_assert(EPI_ROWS % (NW * RB) == 0, "row batches tile the half");
        static_assert(!MX || RB == 4, "the MX encoding takes four rows a pass");
        for (int r0 = wave; r0 < EPI_ROWS; r0 += NW * RB) {
            if (t.m0 + half * EPI_ROWS + r0 >= t.seg_end) break;  // wave-uniform
            u32x4_t v[RB];
#pragma unroll
            for (int b = 0; b < RB; ++b) v[b] = *(const lds_u32x4 *)(lds + soff(r0 + b * NW, lane));
            u32x4_t va;
            if constexpr (MX) va = *(const lds_u32x4 *)(lds + soff(r0 + (lane >> 4) * NW, 32 + (lane & 15)));
#pragma unroll
            for (int b = 0; b < RB; ++b) {
                const int64_t m = t.m0 + half * EPI_ROWS + r0 + b * NW;
                if (live && m < t.seg_end) {
                    uint16_t *dst = seg == 2 ? ad + m * I + col : hd + m * 2 * I + (seg ? I : 0) + col;
                    *(u32x4_t *)dst = v[b];
                }
            }
            if constexpr (MX) {
                const int64_t m = t.m0 + half * EPI_ROWS + r0 + (lane >> 4) * NW;
                float f[8];
                const u32x4_t z = {0u, 0u, 0u, 0u};
                if (col >= I) va = z;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    f[2 * q] = bf2f((uint16_t)(va[q] & 0xffffu));
                    f[2 * q + 1] = bf2f((uint16_t)(va[q] >> 16));
                }
                uint32_t sc;
                const uint64_t c = mx_quant8(f, sc);
                const uint32_t w = mx_group_word(sc, lane);
                if (m < t.seg_end) {
                    *(uint64_t *)(aq + m * Ip + col) = c;
                    if ((lane & 15) == 0)
                        *(uint32_t *)(as_ + mx_scale_off(m, i0 / MX_GROUP, Ip / MX_GROUP)) = w;
                }
            }
        }
        __syncthreads();
      }
    }
}

}  // namespace moe
