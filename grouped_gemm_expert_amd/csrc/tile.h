// Building blocks of the bf16 MFMA GEMM tiles (gfx950): LDS tile layouts,
// direct global->LDS loaders, the MFMA stage and the two-buffer software
// pipeline, the accumulator fragment layout and the XCD-aware block remap.
// Shared by the grouped expert GEMMs (gemm.hip) and the dense router GEMMs
// (dense.hip).
#pragma once

#include <type_traits>
#include <utility>

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

// BM x BN output tile computed by waves of WM x WN.  The A operand (rows)
// has two LDS stage buffers of 64 k, the B operand (columns) NBB of them:
// the copies of a B stage get NBB-1 stages to land, which matters when B
// streams from HBM (the expert weights of the forward and dgrad ops).  The
// LDS also holds the epilogue's 128 KB staging tile.
template <int BM_, int BN_, int WM_, int WN_, int NBB_ = 2>
struct TileCfg {
    static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_, NBB = NBB_;
    static constexpr int WAVES_M = BM / WM, WAVES_N = BN / WN;
    static constexpr int NT = WAVES_M * WAVES_N * 64;
    static constexpr int FM = WM / 32, FN = WN / 32;
    static constexpr int A_BYTES = BM * 128, B_BYTES = BN * 128;
    static constexpr int RING_BYTES = 2 * A_BYTES + NBB * B_BYTES;
    static constexpr int LDS_BYTES = RING_BYTES > 131072 ? RING_BYTES : 131072;
    static_assert(NBB == 2 || NBB == 3, "two or three B stage buffers");
    static_assert(LDS_BYTES <= 163840, "LDS of one CU");
    static_assert(WM % 32 == 0 && WN % 32 == 0, "wave tile is a multiple of 32x32");
    static_assert(BM == 256 || BM == 128 || BM == 320, "m-tile schedules exist for 128, 256, 320 rows");
    // five or more row fragments a wave: A fragments refilled in place (one
    // register set), which frees the registers the taller wave tile needs
    static constexpr bool INPLACE = FM >= 5;
    static constexpr int NHALF = (BM + 127) / 128;  // 128-row epilogue passes
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
// The global address is a wave-uniform base (SGPR pair, advanced once per
// stage) plus a per-lane 32-bit byte offset, so issuing a copy costs no
// vector address arithmetic.
MOE_DEV void copy16_to_lds(const char *base, uint32_t off, lds_t *dst_block)
{
    const uint32_t m0v = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)dst_block);
    const uint64_t b = (uint64_t)(uintptr_t)base;
    // readfirstlane yields a signed int: widen through uint32_t so that a low
    // word with bit 31 set is not sign-extended into the high word
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(b >> 32));
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)b);
    const uint64_t sb = ((uint64_t)hi << 32) | (uint64_t)lo;
    asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1"
                 :
                 : "v"(off), "s"(sb), "s"(m0v)
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
    MOE_DEV void issue_one(int i, lds_t *tile, int64_t k0, int, const char *b) const
    {
        copy16_to_lds(b + k0 * 2, off[i], tile + (q0 + i) * 1024);
    }
    MOE_DEV void issue(lds_t *tile, int64_t k0, int kvalid, const char *b) const
    {
#pragma unroll
        for (int i = 0; i < NI; ++i) issue_one(i, tile, k0, kvalid, b);
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
    MOE_DEV void issue_one(int i, lds_t *tile, int64_t k0, int kvalid, const char *b) const
    {
        int k = krow(i);
        if (k >= kvalid) k = kvalid - 1;
        copy16_to_lds(b + k0 * (int64_t)ldb, (uint32_t)k * ldb + ncol[i], tile + (q0 + i) * 1024);
    }
    MOE_DEV void issue(lds_t *tile, int64_t k0, int kvalid, const char *b) const
    {
#pragma unroll
        for (int i = 0; i < NI; ++i) issue_one(i, tile, k0, kvalid, b);
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

// MFMA operand fragments of one 16-deep k-step for a wave's tile.
template <class C>
struct Frags {
    bf16x8_t a[C::FM], b[C::FN];
};

// PARTIAL: only the wave's first na row fragments hold rows of the tile; the
// others are neither read nor multiplied (na is wave-uniform).
template <class C, bool A_NMAJ, bool B_NMAJ, bool PARTIAL = false>
MOE_DEV void read_frags(const lds_t *As, const lds_t *Bs, int kk, Frags<C> &f, int wm, int wn,
                        int lane, int na = C::FM)
{
#pragma unroll
    for (int i = 0; i < C::FM; ++i)
        if (!PARTIAL || i < na)
            f.a[i] = A_NMAJ ? frag_nmaj<C::BM>(As, wm * C::WM + i * 32, kk, lane)
                            : frag_kmaj(As, wm * C::WM + i * 32, kk, lane);
#pragma unroll
    for (int j = 0; j < C::FN; ++j)
        f.b[j] = B_NMAJ ? frag_nmaj<C::BN>(Bs, wn * C::WN + j * 32, kk, lane)
                        : frag_kmaj(Bs, wn * C::WN + j * 32, kk, lane);
}

template <class C>
MOE_DEV void mfma_step(const Frags<C> &f, Acc<C> &acc)
{
#pragma unroll
    for (int i = 0; i < C::FM; ++i)
#pragma unroll
        for (int j = 0; j < C::FN; ++j)
            acc.v[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.b[j], f.a[i], acc.v[i][j], 0, 0, 0);
}

// s_waitcnt vmcnt(n) with the other counters at their maxima (gfx9 encoding:
// vmcnt bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8).
template <int N>
MOE_DEV void wait_copies_le()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Read number r of a k-step's fragments, in the order a0, b0 .. b(FN-1),
// a1 .. a(FM-1): the order in which the (i, j)-ordered MFMAs first need them.
template <class C, bool A_NMAJ, bool B_NMAJ, bool PARTIAL>
MOE_DEV void read_one(int r, const lds_t *As, const lds_t *Bs, int kk, Frags<C> &f, int wm, int wn,
                      int lane, int na)
{
    if (r == 0 || r > C::FN) {
        const int i = r == 0 ? 0 : r - C::FN;
        if (!PARTIAL || i < na)
            f.a[i] = A_NMAJ ? frag_nmaj<C::BM>(As, wm * C::WM + i * 32, kk, lane)
                            : frag_kmaj(As, wm * C::WM + i * 32, kk, lane);
    } else {
        const int j = r - 1;
        f.b[j] = B_NMAJ ? frag_nmaj<C::BN>(Bs, wn * C::WN + j * 32, kk, lane)
                        : frag_kmaj(Bs, wn * C::WN + j * 32, kk, lane);
    }
}

// The MFMAs of one k-step (fragments `cur`) in (i, j) order.  Before MFMA n
// the wave issues fragment read n of the next k-step into `nxt` (n < FM+FN)
// and the copies i (of NC) with i*NMF/NC == n, so LDS reads and
// global->LDS copies are spread evenly over the MFMAs instead of arriving in
// bursts; sched_barrier pins that order.  PARTIAL: row fragments i >= na
// are skipped, reads and MFMAs alike.
template <class C, bool A_NMAJ, bool B_NMAJ, bool PARTIAL, int NC, class Copy>
MOE_DEV void kstep(const Frags<C> &cur, Frags<C> &nxt, const lds_t *As, const lds_t *Bs, int kk_next,
                   Copy &&copy, Acc<C> &acc, int wm, int wn, int lane, int na)
{
    constexpr int NMF = C::FM * C::FN, NR = C::FM + C::FN;
    static_assert(NR <= NMF, "one read per MFMA at most");
#pragma unroll
    for (int n = 0; n < NMF; ++n) {
        if (n < NR) read_one<C, A_NMAJ, B_NMAJ, PARTIAL>(n, As, Bs, kk_next, nxt, wm, wn, lane, na);
        if constexpr (NC > 0) {
#pragma unroll
            for (int i = 0; i < NC; ++i)
                if (i * NMF / NC == n) copy(i);
        }
        __builtin_amdgcn_sched_barrier(0);
        const int i = n / C::FN, j = n % C::FN;
        if (!PARTIAL || i < na)
            acc.v[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cur.b[j], cur.a[i], acc.v[i][j], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
    }
}

// In-place form (INPLACE_A): the wave holds one set of A fragments and two
// of B.  Before MFMA n < FN the wave reads B fragment n of the next k-step
// into the other B set; right after the last MFMA that reads A fragment i
// (n = i*FN + FN-1) it reads the next k-step's A fragment i into the same
// registers, which the next k-step first needs NMF-FN MFMAs later.  A
// fragments take FM*16 bytes a lane instead of twice that (used by the
// configurations whose registers need it: it costs ~1% where the two-set
// form fits, the refilled fragment having less time to arrive).
template <class C, bool A_NMAJ, bool B_NMAJ, bool PARTIAL, int NC, class Copy>
MOE_DEV void kstep_ip(bf16x8_t (&fa)[C::FM], const bf16x8_t (&bc)[C::FN], bf16x8_t (&bn)[C::FN],
                      const lds_t *As, const lds_t *Bs, int kk_next, Copy &&copy, Acc<C> &acc,
                      int wm, int wn, int lane, int na)
{
    constexpr int NMF = C::FM * C::FN;
#pragma unroll
    for (int n = 0; n < NMF; ++n) {
        const int i = n / C::FN, j = n % C::FN;
        if (n < C::FN)
            bn[n] = B_NMAJ ? frag_nmaj<C::BN>(Bs, wn * C::WN + n * 32, kk_next, lane)
                           : frag_kmaj(Bs, wn * C::WN + n * 32, kk_next, lane);
        if constexpr (NC > 0) {
#pragma unroll
            for (int q = 0; q < NC; ++q)
                if (q * NMF / NC == n) copy(q);
        }
        __builtin_amdgcn_sched_barrier(0);
        if (!PARTIAL || i < na)
            acc.v[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bc[j], fa[i], acc.v[i][j], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
        if (j == C::FN - 1 && (!PARTIAL || i < na)) {
            fa[i] = A_NMAJ ? frag_nmaj<C::BM>(As, wm * C::WM + i * 32, kk_next, lane)
                           : frag_kmaj(As, wm * C::WM + i * 32, kk_next, lane);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
}

template <int S>
struct SetTag {
    static constexpr int value = S;
};

// f(SetTag<I>(), v + I) for I = 0 .. P-1, stopping at v1.
template <class F, int... I>
MOE_DEV void stage_run(F &&f, int v, int v1, std::integer_sequence<int, I...>)
{
    ((v + I < v1 ? f(SetTag<I>(), v + I) : void()), ...);
}

// Software pipeline over stages v0 .. v1-1 (64 k each): two LDS buffers for
// A, NBB for B, two fragment register sets.  Stage v computes k-steps 0..3
// from A buffer v%2 and B buffer v%NBB, reading the fragments of step kk+1
// while the MFMAs of step kk run.  Once the fragments of step 3 are in
// registers the wave no longer needs those buffers, so the barrier comes
// before step 3's MFMAs: each wave first waits for its own copies of stage
// v+1 (and lets `tail` fix that stage up), then the barrier publishes stage
// v+1 and frees the stage-v buffers; after it the wave reads step 0 of stage
// v+1 while step 3's MFMAs execute, and no wave idles on LDS latency right
// after the barrier.
// The copies into the freed buffers are spread so that the CU's vector
// memory path (64 bytes a clock; one copy is 1 KB) never gets them in a
// burst: the A copies of stage v+2 go into step 3 of stage v; with three B
// buffers the B copies of stage v+3 are split into four slots, one in step 3
// of stage v and one in each of steps 0..2 of stage v+1 (they still have a
// stage to land); with two B buffers they all go into step 3 of stage v.
// copy_a(q, v, As) / copy_b(q, v, Bs) issue copy q (of NCA / NCB per wave)
// of stage v's A / B tile; tail(v, As, Bs) runs after stage v landed.
// PARTIAL / na: the wave multiplies only its first na row fragments
// (read_frags); its copies are the callers' business.
template <class C, bool A_NMAJ, bool B_NMAJ, int NCA, int NCB, bool PARTIAL = false, class CopyA,
          class CopyB, class Tail>
MOE_DEV void pipeline(lds_t *lds, int v0, int v1, CopyA &&copy_a, CopyB &&copy_b, Tail &&tail,
                      Acc<C> &acc, int na = C::FM)
{
    constexpr int NB = C::NBB;
    constexpr bool SPREAD = NB == 3;
    constexpr int SB = SPREAD ? (NCB + 3) / 4 : NCB;  // B copies per slot (slot 0: after the barrier)
    static_assert(!SPREAD || NCB % 4 == 0, "B copies split into four equal slots");
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = wave / C::WAVES_N, wn = wave % C::WAVES_N;
    lds_t *As[2] = {lds, lds + C::A_BYTES};
    lds_t *Bs[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) Bs[b] = lds + 2 * C::A_BYTES + b * C::B_BYTES;
    acc.zero();
    if (v1 <= v0) return;
    auto clampv = [&](int v) { return v < v1 ? v : v1 - 1; };
    // A and B of stages v0, v0+1, then slot 0 of stage v0+2's B copies (its
    // other slots go into stage v0's first steps); past the end the last stage
    // again, into buffers nothing reads.  Wait for stage v0 only.
#pragma unroll
    for (int s = 0; s < 2; ++s) {
#pragma unroll
        for (int q = 0; q < NCA; ++q) copy_a(q, clampv(v0 + s), As[s]);
#pragma unroll
        for (int q = 0; q < NCB; ++q) copy_b(q, clampv(v0 + s), Bs[s]);
    }
    if constexpr (SPREAD) {
#pragma unroll
        for (int q = 0; q < SB; ++q) copy_b(q, clampv(v0 + 2), Bs[2]);
    }
    wait_copies_le<NCA + NCB + (SPREAD ? SB : 0)>();
    tail(v0, As[0], Bs[0]);
    __syncthreads();
    // two fragment sets f0 / f1 (k-step s multiplies one and reads step s+1
    // into the other), or with INPLACE one A set (f0.a) and two B sets
    Frags<C> f0, f1;
    read_frags<C, A_NMAJ, B_NMAJ, PARTIAL>(As[0], Bs[0], 0, f0, wm, wn, lane, na);
    // k-step: multiply `cur`, read the step kk fragments into `nxt`
    auto kst = [&](Frags<C> &cur, Frags<C> &nxt, const lds_t *A_, const lds_t *B_, int kk,
                   auto &&copy, auto nc) {
        constexpr int NC_ = decltype(nc)::value;
        if constexpr (C::INPLACE)
            kstep_ip<C, A_NMAJ, B_NMAJ, PARTIAL, NC_>(f0.a, cur.b, nxt.b, A_, B_, kk, copy, acc, wm,
                                                      wn, lane, na);
        else
            kstep<C, A_NMAJ, B_NMAJ, PARTIAL, NC_>(cur, nxt, A_, B_, kk, copy, acc, wm, wn, lane, na);
    };
    // one stage; the buffers it uses are compile-time constants, so LDS
    // addresses fold into instruction offsets
    auto stage = [&](auto tag, int v) {
        constexpr int I = decltype(tag)::value;
        constexpr int a = I % 2, an = (I + 1) % 2, b = I % NB, bn = (I + 1) % NB;
        constexpr int bp = (I + NB - 1) % NB;  // buffer of stage v-1: gets stage v-1+NB
        const int vp = clampv(v - 1 + NB);
        auto slot = [&](int s) {  // B copies of slot s of stage v-1+NB
            return [&, s](int i) { copy_b(s * SB + i, vp, Bs[bp]); };
        };
        auto none = [](int) {};
        using SBt = std::integral_constant<int, SPREAD ? SB : 0>;
        if constexpr (SPREAD) {
            kst(f0, f1, As[a], Bs[b], 1, slot(1), SBt());
            kst(f1, f0, As[a], Bs[b], 2, slot(2), SBt());
            kst(f0, f1, As[a], Bs[b], 3, slot(3), SBt());
        } else {
            kst(f0, f1, As[a], Bs[b], 1, none, SBt());
            kst(f1, f0, As[a], Bs[b], 2, none, SBt());
            kst(f0, f1, As[a], Bs[b], 3, none, SBt());
        }
        // every stage issues the same copies, and stage v+1's were all issued
        // before the last A copies; only the B copies of stage v+2 (three B
        // buffers) may still be outstanding
        wait_copies_le<(NB - 2) * NCB>();
        if (v + 1 < v1) tail(v + 1, As[an], Bs[bn]);
        __syncthreads();
        // step 0 of stage v+1; A copies of stage v+2 and B slot 0 of stage
        // v+NB into the freed buffers.  Past the end both are harmless and
        // branch-free: the reads fetch stale fragments that are never used,
        // and the last stage is copied again into buffers nothing reads.
        const int va = clampv(v + 2), vb = clampv(v + NB);
        auto copy0 = [&](int q) {
            if (q < NCA) copy_a(q, va, As[a]);
            else copy_b(q - NCA, vb, Bs[b]);
        };
        kst(f1, f0, As[an], Bs[bn], 0, copy0, std::integral_constant<int, NCA + SB>());
    };
    constexpr int P = NB == 3 ? 6 : 2;  // buffer pattern period
    int v = v0;
    for (; v + P <= v1; v += P) stage_run(stage, v, v1, std::make_integer_sequence<int, P>());
    stage_run(stage, v, v1, std::make_integer_sequence<int, P - 1>());
    wait_copies();    // the repeated copies of the last stages
    __syncthreads();  // callers may reuse the LDS
}

// The row fragments of this wave that start below `rows` (tile rows 0 ..
// rows-1 hold data): 0 .. FM.  Wave-uniform.
template <class C>
MOE_DEV int partial_row_frags(int rows)
{
    const int rel = rows - (wave_uniform_id() / C::WAVES_N) * C::WM;
    return rel <= 0 ? 0 : (rel >= C::FM * 32 ? C::FM : (rel + 31) / 32);
}

// C = A . B^T over K with two loaders of fixed base: stages of 64 k, the last
// one partial when KTAIL (its rows past K are zeroed).  PARTIAL: the tile
// holds only `rows` < BM rows of A (a segment's last m-tile; A K-major).
// Wave w copies A rows [w*RPW, (w+1)*RPW), RPW = BM/NW (KLoad): a wave whose
// rows all lie past `rows` copies no A at all (its own pipeline
// instantiation with no A copies, so that every wait counts exactly the
// copies issued), and each wave multiplies only the row fragments that start
// below `rows`: fragment i of wave tile row wm covers rows wm*WM + 32 i ..
// + 31, copied by wave (wm*WM + 32 i) / RPW, which starts below `rows` too.
// The rows skipped feed no stored output.
template <class C, bool A_NMAJ, bool B_NMAJ, bool KTAIL, bool PARTIAL = false, class LA, class LB>
MOE_DEV void mainloop(lds_t *lds, int64_t K, const LA &la, const LB &lb, Acc<C> &acc,
                      int rows = C::BM)
{
    static_assert(!PARTIAL || !A_NMAJ, "partial tiles skip the copies of K-major A rows");
    constexpr int RPW = C::BM / (C::NT / 64);
    static_assert(RPW % 8 == 0, "a wave copies whole 1 KB blocks of A rows");
    auto kvalid = [&](int s) -> int {
        const int64_t rem = K - (int64_t)s * BK;
        return KTAIL ? (rem < BK ? (int)rem : BK) : BK;
    };
    const int nst = (int)ceil_div(K, BK);
    auto cpa = [&](int q, int s, lds_t *As) { la.issue_one(q, As, (int64_t)s * BK, kvalid(s), la.base); };
    auto cpb = [&](int q, int s, lds_t *Bs) { lb.issue_one(q, Bs, (int64_t)s * BK, kvalid(s), lb.base); };
    auto tail = [&](int s, lds_t *As, lds_t *Bs) {
        if (KTAIL && kvalid(s) < BK) {
            la.zero_tail(As, kvalid(s));
            lb.zero_tail(Bs, kvalid(s));
        }
    };
    if constexpr (!PARTIAL) {
        pipeline<C, A_NMAJ, B_NMAJ, LA::NI, LB::NI>(lds, 0, nst, cpa, cpb, tail, acc);
    } else {
        const int na = partial_row_frags<C>(rows);
        if (wave_uniform_id() * RPW < rows)
            pipeline<C, A_NMAJ, B_NMAJ, LA::NI, LB::NI, true>(lds, 0, nst, cpa, cpb, tail, acc, na);
        else
            pipeline<C, A_NMAJ, B_NMAJ, 0, LB::NI, true>(lds, 0, nst, cpa, cpb, tail, acc, na);
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

// ------------------------------------------------------------ epilogue ----
// The accumulators leave the block through LDS, one 128-row half of the
// 256-row tile at a time: the waves holding that half write their fragments
// into a [128][256] fp32 staging tile (1 KB a row, 16-byte chunks XOR-swizzled
// by row so that both the fragment writes and the row reads are free of bank
// conflicts), then every wave takes whole rows, lane l owning columns
// 4l .. 4l+3, so global loads and stores are row-contiguous 16-byte (or
// 8-byte) accesses instead of the fragment layout's scattered 8-byte pieces.
constexpr int EPI_ROWS = 128;
typedef __attribute__((address_space(3))) f32x4_t lds_f32x4;
typedef __attribute__((address_space(3))) uint64_t lds_u64;

MOE_DEV int epi_off(int r, int chunk) { return r * 1024 + ((chunk ^ (r & 15)) << 4); }

// Fragments of rows [half*128, half*128 + 128) of the tile into the staging
// tile (a 32-row fragment block is wholly inside one half).
template <class C>
MOE_DEV void epi_stage_f32(const Acc<C> &acc, lds_t *lds, int half, int wm, int wn, int lane)
{
#pragma unroll
    for (int i = 0; i < C::FM; ++i) {
        if ((wm * C::WM + i * 32) / EPI_ROWS != half) continue;
        const int r = acc_row<C>(wm, i, lane) - half * EPI_ROWS;
#pragma unroll
        for (int j = 0; j < C::FN; ++j)
#pragma unroll
            for (int rg = 0; rg < 4; ++rg) {
                const int c = acc_col<C>(wn, j, rg, lane);
                f32x4_t v = {acc.v[i][j][rg * 4], acc.v[i][j][rg * 4 + 1], acc.v[i][j][rg * 4 + 2],
                             acc.v[i][j][rg * 4 + 3]};
                *(lds_f32x4 *)(lds + epi_off(r, c >> 2)) = v;
            }
    }
}

MOE_DEV f32x4_t epi_read_f32(const lds_t *lds, int r, int lane)
{
    return *(const lds_f32x4 *)(lds + epi_off(r, lane));
}

// out[m][n0 + c] = tile[m - m0][c] for rows m0 <= m < mlim (row stride
// ncols, ncols a multiple of 4; of 8 for bf16), fp32 or (OutT = uint16_t)
// bf16 with nearest-even rounding.  Starts and ends on a barrier-free LDS.  A wave
// reads 8 of its rows from LDS at once, then stores them, so the LDS latency
// is paid once per 8 rows.
MOE_DEV void store4(float *p, f32x4_t v) { *(f32x4_t *)p = v; }
MOE_DEV void store4(uint16_t *p, f32x4_t v) { *(uint64_t *)p = pack_bf4(v[0], v[1], v[2], v[3]); }
// bf16 out (ncols a multiple of 8).  The accumulators are rounded to bf16 as
// they are staged (the one rounding the output gets either way), so the
// whole tile fits the LDS at once: row r holds its BN values in 16-byte
// chunks, chunk c at r * BN * 2 + ((c ^ (r % 32)) << 4).  Then lane l takes
// chunk l % 32 (8 columns) of one of two rows (l / 32): every store is 16
// bytes and a wave covers two rows per instruction.
template <class C>
MOE_DEV int epi16_off(int r, int chunk)
{
    return r * (C::BN * 2) + ((chunk ^ (r & 31)) << 4);
}

// A tile whose bf16 values do not fit the LDS at once (320 rows) goes in
// one pass per wave row (WM rows each).
template <class C>
MOE_DEV void store_tile_bf16(const Acc<C> &acc, lds_t *lds, uint16_t *out, int64_t m0,
                             int64_t mlim, int64_t n0, int64_t ncols)
{
    static_assert(C::BN == 256, "a staged row is 32 chunks: one per lane of a half wave");
    constexpr bool WHOLE = C::BM * C::BN * 2 <= C::LDS_BYTES;
    constexpr int NPASS = WHOLE ? 1 : C::WAVES_M, PROWS = WHOLE ? C::BM : C::WM;
    static_assert(PROWS * C::BN * 2 <= C::LDS_BYTES, "a pass's bf16 rows fit the LDS");
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = wave / C::WAVES_N, wn = wave % C::WAVES_N;
    const int c = lane & 31;
    const int64_t col = n0 + 8 * c;
    constexpr int NW = C::NT / 64, RB = 8;
    static_assert(PROWS % (2 * NW * RB) == 0 || !WHOLE, "row batches tile the tile");
#pragma unroll
    for (int pass = 0; pass < NPASS; ++pass) {
        const int64_t p0 = m0 + pass * PROWS;  // first row of the pass
        if (p0 >= mlim) break;
        if (WHOLE || wm == pass) {
#pragma unroll
            for (int i = 0; i < C::FM; ++i) {
                const int r = acc_row<C>(wm, i, lane) - pass * PROWS;
#pragma unroll
                for (int j = 0; j < C::FN; ++j)
#pragma unroll
                    for (int rg = 0; rg < 4; ++rg) {
                        const int cc = acc_col<C>(wn, j, rg, lane);
                        *(lds_u64 *)(lds + epi16_off<C>(r, cc >> 3) + (cc & 4) * 2) =
                            pack_bf4(acc.v[i][j][rg * 4], acc.v[i][j][rg * 4 + 1],
                                     acc.v[i][j][rg * 4 + 2], acc.v[i][j][rg * 4 + 3]);
                    }
            }
        }
        __syncthreads();
        if (col < ncols)
            for (int r0 = 2 * wave + (lane >> 5); r0 < PROWS; r0 += 2 * NW * RB) {
                if (p0 + r0 >= mlim) break;  // rows past the segment (no barrier in the loop)
                u32x4_t v[RB];
#pragma unroll
                for (int b = 0; b < RB; ++b)
                    if (WHOLE || r0 + b * 2 * NW < PROWS)
                        v[b] = *(const lds_u32x4 *)(lds + epi16_off<C>(r0 + b * 2 * NW, c));
#pragma unroll
                for (int b = 0; b < RB; ++b) {
                    const int64_t m = p0 + r0 + b * 2 * NW;
                    if (m >= mlim || (!WHOLE && r0 + b * 2 * NW >= PROWS)) break;
                    *(u32x4_t *)(out + m * ncols + col) = v[b];
                }
            }
        __syncthreads();
    }
}

template <class C, class OutT = float>
MOE_DEV void store_tile_f32(const Acc<C> &acc, lds_t *lds, OutT *out, int64_t m0, int64_t mlim,
                            int64_t n0, int64_t ncols)
{
    if constexpr (sizeof(OutT) == 2) {
        store_tile_bf16<C>(acc, lds, out, m0, mlim, n0, ncols);
        return;
    }
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = wave / C::WAVES_N, wn = wave % C::WAVES_N;
    const int64_t col = n0 + 4 * lane;
    constexpr int NW = C::NT / 64, RB = 8;
    static_assert(EPI_ROWS % (NW * RB) == 0, "row batches tile the half");
#pragma unroll
    for (int half = 0; half < C::NHALF; ++half) {
        if (m0 + half * EPI_ROWS >= mlim) break;
        epi_stage_f32<C>(acc, lds, half, wm, wn, lane);
        __syncthreads();
        if (col < ncols)
            for (int r0 = wave; r0 < EPI_ROWS; r0 += RB * NW) {
                f32x4_t v[RB];
#pragma unroll
                for (int b = 0; b < RB; ++b) v[b] = epi_read_f32(lds, r0 + b * NW, lane);
#pragma unroll
                for (int b = 0; b < RB; ++b) {
                    const int64_t m = m0 + half * EPI_ROWS + r0 + b * NW;
                    if (m >= mlim) break;
                    store4(out + m * ncols + col, v[b]);
                }
            }
        __syncthreads();
    }
}

// ------------------------------------------------------- tile schedules ----
// XCD-aware remap of block b over `total` tiles.  Blocks are dispatched to
// the 8 XCDs round-robin (block b runs on XCD b % 8); consecutive tiles are
// dealt to the XCDs in chunks of XCD_CHUNK (half the CUs of one XCD), so the tiles
// an XCD runs together are neighbours (they share operand panels in its L2)
// while tiles of unequal cost spread evenly over all XCDs.  The grid is a
// multiple of 8 * XCD_CHUNK and at least `total` rounded up to that.
constexpr int64_t XCD_CHUNK = 16;  // measured faster overall than 8, 32 or 64
template <int64_t CH = XCD_CHUNK>
MOE_DEV int64_t xcd_remap(int64_t b, int64_t total)
{
    const int64_t x = b & 7, j = b >> 3;
    const int64_t L = ((j / CH) * 8 + x) * CH + (j % CH);
    return L < total ? L : -1;
}

template <int64_t CH = XCD_CHUNK>
inline int64_t grid_for(int64_t total) { return ceil_div(total, 8 * CH) * 8 * CH; }

// ------------------------------------------------------------ schedule ----
// Forward and dgrad GEMMs tile the sorted rows of each expert (M-grouped):
// the per-expert m-tile prefix sums live on the device and surplus blocks of
// the host-sized grid exit.
struct MTile {
    int e;
    int64_t m0, seg_end;
    int nt;
    // the fields are block-uniform: keep them in scalar registers
    MOE_DEV void uniform()
    {
        e = __builtin_amdgcn_readfirstlane(e);
        nt = __builtin_amdgcn_readfirstlane(nt);
        m0 = rfl64(m0);
        seg_end = rfl64(seg_end);
    }
    static MOE_DEV int64_t rfl64(int64_t v)
    {
        const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(uint64_t)v);
        const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)v >> 32));
        return (int64_t)(((uint64_t)hi << 32) | lo);
    }
};

// M-grouped tile L: inside each expert, groups of GM of its m-tiles sweep
// all n-tiles before moving on; a group never spans two experts, so the
// tiles an XCD runs together share the expert's weight panels and their
// token rows in its L2 (an expert with few rows is one group).
// Tile L (0 <= L < mt_off[E] nN, after the XCD remap).
template <int BM>
MOE_DEV void decode_mtile_at(int64_t L, const int32_t *mt_off, const int32_t *offsets, int E,
                             int nN, MTile &t)
{
    constexpr int GM = 4;
    // expert e owns tiles [mt_off[e] nN, mt_off[e + 1] nN): the largest e
    // with mt_off[e] nN <= L has m-tiles (mte >= 1)
    int lo = 0, hi = E;
    while (hi - lo > 1) {
        int mid = (lo + hi) >> 1;
        if ((int64_t)mt_off[mid] * nN <= L) lo = mid; else hi = mid;
    }
    const int64_t mte = mt_off[lo + 1] - mt_off[lo];
    const int64_t in0 = L - (int64_t)mt_off[lo] * nN;
    const int64_t grp = in0 / ((int64_t)GM * nN);
    const int64_t first = grp * GM;
    const int64_t gm = mte - first < GM ? mte - first : GM;
    const int64_t in = in0 - grp * (int64_t)GM * nN;
    t.nt = (int)(in / gm);
    t.e = lo;
    t.m0 = offsets[lo] + (first + in % gm) * BM;
    t.seg_end = offsets[lo + 1];
}

// The tile of block b (false: a surplus block).
template <int BM>
MOE_DEV bool decode_mtile(int64_t b, const int32_t *mt_off, const int32_t *offsets, int E,
                          int nN, MTile &t)
{
    const int64_t L = xcd_remap(b, (int64_t)mt_off[E] * nN);
    if (L < 0) return false;
    decode_mtile_at<BM>(L, mt_off, offsets, E, nN, t);
    return true;
}

// Mixed m-tiling of the bf16 forward and dgrad GEMMs.  Each expert's rows
// are cut into 256-row tiles, except that an expert with more than 256 rows
// whose count leaves 1..64 rows past a multiple of 256 ends on one tile of
// 257..320 rows instead of a full tile and a nearly empty one: under
// balanced routing (about 256 rows an expert) half the experts would
// otherwise stream their weights a second time for a few rows.  mt_a counts
// the 256-row tiles (class 0), mt_b the 320-row ones (class 1, at most one
// an expert).  One launch holds both: the longer class-1 tiles first (so
// that they do not end the launch on a tail of their own), then class 0,
// each sweeping its expert's n-tiles as decode_mtile does.  Returns the
// class, or -1 for a surplus block.
MOE_DEV int decode_mtile_mixed(int64_t b, const int32_t *mt_a, const int32_t *mt_b,
                               const int32_t *offsets, int E, int nN, MTile &t)
{
    const int64_t ta = (int64_t)mt_a[E] * nN, tb = (int64_t)mt_b[E] * nN;
    int64_t L = xcd_remap(b, ta + tb);
    if (L < 0) return -1;
    if (L >= tb) {
        decode_mtile_at<256>(L - tb, mt_a, offsets, E, nN, t);
        // a class-0 tile ends where the expert's class-1 tile (if any) starts
        if (t.seg_end > t.m0 + 256) t.seg_end = t.m0 + 256;
        t.uniform();
        return 0;
    }
    int lo = 0, hi = E;
    while (hi - lo > 1) {
        int mid = (lo + hi) >> 1;
        if ((int64_t)mt_b[mid] * nN <= L) lo = mid; else hi = mid;
    }
    t.e = lo;
    t.nt = (int)(L - (int64_t)mt_b[lo] * nN);
    t.seg_end = offsets[lo + 1];
    t.m0 = offsets[lo] + (int64_t)((t.seg_end - offsets[lo]) / 256 - 1) * 256;
    t.uniform();
    return 1;
}

// Upper bound on the blocks an M-grouped launch needs (host side; also
// bounds the mixed tiling's 256-row tiles).
int64_t mgrid_blocks(int64_t M, int E, int BM, int nN);

}  // namespace moe
