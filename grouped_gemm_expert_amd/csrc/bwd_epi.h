// Epilogues of the backward GEMM tiles, shared by the bf16 and the MXFP8
// kernels: the fused SwiGLU backward and routing-weight row-dot of GEMM2's
// dgrad, and the read-modify-write store of the weight gradients.
#pragma once

#include "tile.h"

namespace moe {

// Sums over groups of LANES lanes (64: the wave; 32: each half) of RB row
// partials at once: p[b] is this lane's part of row b.  log2(RB) halving
// exchanges (lane ^ LANES/2, ^ LANES/4, ...: after the one with mask m,
// lanes with bit m set keep the upper half of the rows, adding their
// partner's copies), then the LANES/RB lanes that share a row add up over the
// remaining low lane bits by DPP (quad swaps, half-row and row mirrors) and
// at most one shuffle.  Every lane returns the total of row `row` of its
// group.
// One halving level, N rows still held (compile-time, so p stays in registers).
template <int RB, int N, int LANES>
MOE_DEV void rows_halve(float (&p)[RB], int lane, int &row)
{
    if constexpr (N > 1) {
        constexpr int m = LANES / 2 * N / RB;
        const bool up = (lane & m) != 0;
#pragma unroll
        for (int i = 0; i < N / 2; ++i) {
            const float send = up ? p[i] : p[N / 2 + i];
            const float keep = up ? p[N / 2 + i] : p[i];
            p[i] = keep + __shfl_xor(send, m, 64);
        }
        if (up) row += N / 2;
        rows_halve<RB, N / 2, LANES>(p, lane, row);
    }
}

template <int CTRL>
MOE_DEV float dpp_add(float v)
{
    return v + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

template <int RB, int LANES = 64>
MOE_DEV float rows_sum(float (&p)[RB], int lane, int &row)
{
    static_assert(RB == 2 || RB == 4 || RB == 8, "two, four or eight rows");
    static_assert(LANES == 32 || LANES == 64, "a half wave or the wave");
    constexpr int G = LANES / RB;  // lanes sharing a row after the halvings
    row = 0;
    rows_halve<RB, RB, LANES>(p, lane, row);
    float v = p[0];
    if constexpr (G >= 2) v = dpp_add<0xB1>(v);    // quad_perm(1, 0, 3, 2)
    if constexpr (G >= 4) v = dpp_add<0x4E>(v);    // quad_perm(2, 3, 0, 1)
    if constexpr (G >= 8) v = dpp_add<0x141>(v);   // row_half_mirror: 8 lanes
    if constexpr (G >= 16) v = dpp_add<0x140>(v);  // row_mirror: 16
    if constexpr (G >= 32) v += __shfl_xor(v, 16, 64);
    return v;
}

// dgrad of GEMM2, for the tile of sorted rows [t.m0, t.seg_end) and columns
// n0 .. n0+BN-1 of I (column tile t.nt of nN):
//   dw_part[m, t.nt] = sum over the tile's columns of dA'[m, i] a[m, i]
//   dA = wrow[m] dA';  dh[m, i] = dA u sig(g)(1 + g(1 - sig(g))),
//   dh[m, I + i] = dA silu(g)   (g, u from h; bf16 out)
// dA' leaves through the LDS staging tile; lane l then owns columns
// n0 + 8 (l % 32) .. + 7 of one of two rows (l / 32), so every load and store
// of h, a and dh is 16 bytes: it loads h (gate, up) and a there, applies the
// routing weight and the SwiGLU backward, stores dh, and each half wave sums
// dA'.a over the tile's columns of its row (dw_part[m, nt]; the RB rows a
// lane holds in one rows_sum).  A wave takes 2 RB rows of a 128-row half at a
// time; the loads of a batch are issued together (addresses clamped to
// valid rows), the first batch's before the half is staged, so their latency
// overlaps the staging.  I is a multiple of 64 (moe_check_config).
// SPLIT: g, u and a are read as hi + lo pairs (h + h_lo, a + a_lo) and dh
// leaves as one too: dh = bf16(v), dh_lo = bf16(v - bf16(v)).
template <class C, int RB = 4, bool SPLIT = false>
MOE_DEV void dgrad2_epilogue(const Acc<C> &acc, lds_t *lds, const MTile &t, int64_t n0, int nN,
                             int I, const uint16_t *h, const uint16_t *a, const float *wrow,
                             uint16_t *dh, float *dw_part, const uint16_t *h_lo = nullptr,
                             const uint16_t *a_lo = nullptr, uint16_t *dh_lo = nullptr)
{
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave / C::WAVES_N, wn = wave % C::WAVES_N;
    const int c = lane & 31;
    const int64_t col = n0 + 8 * c;
    const bool cok = col < I;
    const int64_t colc = cok ? col : 0;
    constexpr int NW = C::NT / 64;
    constexpr int RS = 2 * NW;  // row stride of a lane's rows in a batch
    static_assert(EPI_ROWS % (RS * RB) == 0, "row batches tile the half");
    constexpr int NL = SPLIT ? RB : 1;
    struct Batch {
        u32x4_t hg[RB], hu[RB], hv[RB];
        u32x4_t lg[NL], lu[NL], lv[NL];
        float wgt[RB];
    };
    auto unpack8 = [](const u32x4_t &v, float (&o)[8]) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            o[2 * q] = bf2f((uint16_t)(v[q] & 0xffffu));
            o[2 * q + 1] = bf2f((uint16_t)(v[q] >> 16));
        }
    };
    auto pack8 = [](const float (&o)[8]) {
        return u32x4_t{pack_bf2(o[0], o[1]), pack_bf2(o[2], o[3]), pack_bf2(o[4], o[5]),
                       pack_bf2(o[6], o[7])};
    };
    // r0: this lane's first row of the batch within the half
    auto load = [&](int half, int r0, Batch &bt) {
#pragma unroll
        for (int b = 0; b < RB; ++b) {
            int64_t m = t.m0 + half * EPI_ROWS + r0 + b * RS;
            if (m >= t.seg_end) m = t.seg_end - 1;
            bt.hg[b] = *(const u32x4_t *)(h + m * 2 * I + colc);
            bt.hu[b] = *(const u32x4_t *)(h + m * 2 * I + I + colc);
            bt.hv[b] = *(const u32x4_t *)(a + m * I + colc);
            if constexpr (SPLIT) {
                bt.lg[b] = *(const u32x4_t *)(h_lo + m * 2 * I + colc);
                bt.lu[b] = *(const u32x4_t *)(h_lo + m * 2 * I + I + colc);
                bt.lv[b] = *(const u32x4_t *)(a_lo + m * I + colc);
            }
            bt.wgt[b] = wrow[m];
        }
    };
    auto process = [&](int half, int r0, const Batch &bt) {
        float part[RB];
#pragma unroll
        for (int b = 0; b < RB; ++b) part[b] = 0.f;
#pragma unroll
        for (int b = 0; b < RB; ++b) {
            const int64_t m = t.m0 + half * EPI_ROWS + r0 + b * RS;
            if (m >= t.seg_end) break;
            const f32x4_t d0 = *(const lds_f32x4 *)(lds + epi_off(r0 + b * RS, 2 * c));
            const f32x4_t d1 = *(const lds_f32x4 *)(lds + epi_off(r0 + b * RS, 2 * c + 1));
            const float dap[8] = {d0[0], d0[1], d0[2], d0[3], d1[0], d1[1], d1[2], d1[3]};
            float gv[8], uv[8], av[8], dg[8], du[8];
            unpack8(bt.hg[b], gv);
            unpack8(bt.hu[b], uv);
            unpack8(bt.hv[b], av);
            if constexpr (SPLIT) {
                float gl[8], ul[8], al[8];
                unpack8(bt.lg[b], gl);
                unpack8(bt.lu[b], ul);
                unpack8(bt.lv[b], al);
#pragma unroll
                for (int q = 0; q < 8; ++q) {
                    gv[q] += gl[q];
                    uv[q] += ul[q];
                    av[q] += al[q];
                }
            }
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                part[b] += dap[q] * av[q];
                const float da = bt.wgt[b] * dap[q];
                const float sg = sigmoidf_(gv[q]);
                dg[q] = da * uv[q] * sg * (1.0f + gv[q] * (1.0f - sg));
                du[q] = da * gv[q] * sg;
            }
            if (cok) {
                *(u32x4_t *)(dh + m * 2 * I + col) = pack8(dg);
                *(u32x4_t *)(dh + m * 2 * I + I + col) = pack8(du);
                if constexpr (SPLIT) {
#pragma unroll
                    for (int q = 0; q < 8; ++q) {
                        dg[q] -= bf2f(f2bf(dg[q]));
                        du[q] -= bf2f(f2bf(du[q]));
                    }
                    *(u32x4_t *)(dh_lo + m * 2 * I + col) = pack8(dg);
                    *(u32x4_t *)(dh_lo + m * 2 * I + I + col) = pack8(du);
                }
            }
            if (!cok) part[b] = 0.f;
        }
        // one lane per row of each half wave writes its total (rows past the
        // segment: none)
        int row;
        const float tot = rows_sum<RB, 32>(part, lane, row);
        const int64_t m = t.m0 + half * EPI_ROWS + r0 + row * RS;
        if ((lane & (32 / RB - 1)) == 0 && m < t.seg_end) dw_part[m * nN + t.nt] = tot;
    };
#pragma unroll
    for (int half = 0; half < C::NHALF; ++half) {
        if (t.m0 + half * EPI_ROWS >= t.seg_end) break;
        const int rb = 2 * wave + (lane >> 5);
        Batch bt;
        load(half, rb, bt);  // first batch, in flight while the half is staged
        epi_stage_f32<C>(acc, lds, half, wm, wn, lane);
        __syncthreads();
        process(half, rb, bt);
        for (int r0 = rb + RS * RB; r0 < EPI_ROWS; r0 += RS * RB) {
            load(half, r0, bt);
            process(half, r0, bt);
        }
        __syncthreads();
    }
}

// Weight-gradient tile rows r0 .. r0+BM-1 (of R) and columns c0 .. c0+BN-1
// (of Cc) of the expert whose gradient starts at dW_off elements: dW (+)= the
// tile, fp32 or bf16, accumulating when acc_mode.  Each wave takes RB rows of
// a 128-row half at a time.  In accumulate mode the old values of a wave's
// first RB rows are loaded before that half's accumulators go through LDS,
// so that memory round trip overlaps the staging; the later batches load
// and store in turn.  The fp32 gradient is read and written non-temporally:
// nothing reads it again during the pass, and keeping it out of the caches
// leaves them to the operand panels: the weight gradients are 2-8% faster
// where this read-modify-write bounds them (many experts with few rows),
// unchanged where the MFMAs do.
template <class C, int RB = EPI_ROWS / (C::NT / 64)>
MOE_DEV void wgrad_epilogue(const Acc<C> &acc, lds_t *lds, int64_t r0, int64_t c0, int R, int Cc,
                            int64_t dW_off, void *dWv, int32_t acc_mode, int32_t bf16)
{
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave / C::WAVES_N, wn = wave % C::WAVES_N;
    const int64_t cc = c0 + 4 * lane;
    const bool cok = cc < Cc;
    const int64_t ccc = cok ? cc : 0;
    constexpr int NW = C::NT / 64;
    static_assert(EPI_ROWS % (NW * RB) == 0, "row batches tile the half");
    auto load = [&](int half, int rb, f32x4_t (&old)[RB]) {
#pragma unroll
        for (int b = 0; b < RB; ++b) {
            int64_t rr = r0 + half * EPI_ROWS + rb + b * NW;
            if (rr >= R) rr = R - 1;
            const int64_t o = dW_off + rr * Cc + ccc;
            old[b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
            if (acc_mode) {
                if (bf16) {
                    float t4[4];
                    unpack_bf4(*(const uint64_t *)((const uint16_t *)dWv + o), t4);
                    old[b] = f32x4_t{t4[0], t4[1], t4[2], t4[3]};
                } else {
                    old[b] = __builtin_nontemporal_load((const f32x4_t *)((const float *)dWv + o));
                }
            }
        }
    };
    auto store = [&](int half, int rb, const f32x4_t (&old)[RB]) {
        if (!cok) return;
#pragma unroll
        for (int b = 0; b < RB; ++b) {
            const int64_t rr = r0 + half * EPI_ROWS + rb + b * NW;
            if (rr >= R) break;
            const int64_t o = dW_off + rr * Cc + cc;
            const f32x4_t w = epi_read_f32(lds, rb + b * NW, lane) + old[b];
            if (bf16)
                *(uint64_t *)((uint16_t *)dWv + o) = pack_bf4(w[0], w[1], w[2], w[3]);
            else
                __builtin_nontemporal_store(w, (f32x4_t *)((float *)dWv + o));
        }
    };
#pragma unroll
    for (int half = 0; half < C::NHALF; ++half) {
        if (r0 + half * EPI_ROWS >= R) break;
        f32x4_t old[RB];
        load(half, wave, old);  // first batch, in flight while the half is staged
        epi_stage_f32<C>(acc, lds, half, wm, wn, lane);
        __syncthreads();
        store(half, wave, old);
        for (int rb = wave + RB * NW; rb < EPI_ROWS; rb += RB * NW) {
            load(half, rb, old);
            store(half, rb, old);
        }
        __syncthreads();
    }
}

}  // namespace moe
