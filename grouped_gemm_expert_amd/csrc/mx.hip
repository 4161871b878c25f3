// MXFP8 expert GEMMs on gfx950 block-scaled MFMA
// (v_mfma_scale_f32_32x32x64_f8f6f4: E4M3 operands, one E8M0 scale per
// 32-deep block of each row and column, fp32 accumulation), and the
// quantiser that produces their MX operands.  (MegaMoE page, "Expert
// precision": the mxfp8 mode runs the expert stages in MXFP8 while the
// parameters stay bf16 and their quantised copies are cached.)
//
// Forward kernels:
//   k_up_swiglu_mx   h = X . W1[e]^T from the MX forms of x (token rows,
//                    gathered through row_map) and w1; SwiGLU from the fp32
//                    accumulators; writes h and a (bf16) and a's MX form.
//   k_rows_mx<DOWN>  o = A . W2[e]^T from the MX forms of a and w2 (fp32 out).
// Backward kernels (the data gradients take the transposed weights' MX forms,
// w2[e]^T along H and w1[e]^T along 2I, which the weight cache keeps):
//   k_down_dgrad_mx  dA' = dY[tok] . W2[e] from dy's MX form (token rows) and
//                    w2^T's; the SwiGLU backward, the routing-weight row-dots
//                    and dh (bf16) in the bf16 kernel's epilogue.
//   k_rows_mx<UP_DGRAD>  dxp = dH . W1[e] from dh's MX form and w1^T's.
//   k_wgrad_mx       dW2[e] = (w dY)^T A and dW1[e] = dH^T X: both operands are
//                    the transposes of sorted-row matrices, quantised along the
//                    expert's rows (k_mx_quantize_cols: one MX matrix per
//                    expert, K = its rows padded to 128, 32-row blocks from
//                    the expert's first row).
// Every operand is K-major, so the tiles reuse the bf16 kernels' [rows][128 B]
// swizzled LDS layout and direct global->LDS copies: a 128-byte row slice is
// 128 fp8 of k here (one scale group, two MFMA k-steps) instead of 64 bf16,
// so every copy still moves whole 128-byte lines.  (Stages of 64 fp8 in a
// four-deep ring were measured too: they halve the bytes per line request,
// and a CU's copy rate is set by how many line requests it keeps in flight
// against the L2 latency, so they were slower.)
// The block scales of a stage (4 bytes per row, for 256 A rows and 256 B
// rows) travel through LDS too, as 4-byte-per-lane copies in which lanes
// 0..31 copy 32 A rows and lanes 32..63 the matching 32 B rows.
//
// MFMA operand layout (32x32x64, 32 bytes per lane): lane half g of
// row r holds, for k-step s of a stage, bytes [64 s + 16 g, +16) (block 2s)
// and [64 s + 32 + 16 g, +16) (block 2s+1) of the row's stage slice, and
// supplies the scale of block 2s + g; the instruction applies the scale given
// by half b to the bytes of block 2s + b in both halves.  With the scales of
// a group stored as blocks 0, 2, 1, 3, half g reads the 16-bit word at byte
// 2g of the row's 4 scale bytes: low byte for step 0, high byte for step 1
// (selected by the instruction's op_sel).
#include "bwd_epi.h"
#include "segtile.h"
#include "swiglu_epi.h"

namespace moe {

typedef int v8i32_t __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) uint16_t lds_u16;

// ------------------------------------------------------------ quantiser ----
// Row-wise MX quantisation of a bf16 matrix src [rows, K] (K % 32 == 0) into
// codes [rows, Kp] and the scale area (layout in mxfmt.h).  Sixteen lanes
// take one 128-column group of a row, 8 columns each.  Row-groups are
// numbered (32-row block, group, row) and a block takes 16 consecutive ones:
// 16 rows of one group, whose scale words fill half of one 128-byte line.
// The grid strides over these tiles, loading the next tile before encoding
// the current one.
__global__ __launch_bounds__(256) void k_mx_quantize(const uint16_t *src, int64_t rows, int64_t K,
                                                     int64_t Kp, uint8_t *codes, uint8_t *scales,
                                                     int64_t ntiles)
{
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const uint32_t gpr = (uint32_t)(Kp / MX_GROUP);
    const int sub = (lane & 15) * 8;
    auto locate = [&](int64_t tile, int64_t &row, int64_t &j) {
        const int64_t rg = tile * 16 + wv * 4 + (lane >> 4);
        const uint32_t t = (uint32_t)(rg >> 5);
        const uint32_t rb = t / gpr;
        j = t - rb * gpr;
        row = (int64_t)rb * 32 + (rg & 31);
    };
    auto load = [&](int64_t row, int64_t j) {
        const int64_t col = j * MX_GROUP + sub;
        u32x4_t v = {0u, 0u, 0u, 0u};
        if (row < rows && col < K) v = *(const u32x4_t *)(src + row * K + col);
        return v;
    };
    int64_t tile = blockIdx.x;
    int64_t row, j;
    locate(tile, row, j);
    u32x4_t cur = load(row, j);
    for (;;) {
        const int64_t next = tile + gridDim.x;
        int64_t nrow = 0, nj = 0;
        u32x4_t nxt = {0u, 0u, 0u, 0u};
        if (next < ntiles) {
            locate(next, nrow, nj);
            nxt = load(nrow, nj);
        }
        float v[8];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            v[2 * q] = bf2f((uint16_t)(cur[q] & 0xffffu));
            v[2 * q + 1] = bf2f((uint16_t)(cur[q] >> 16));
        }
        uint32_t sc;
        const uint64_t c = mx_quant8(v, sc);
        const uint32_t word = mx_group_word(sc, lane);
        if (row < rows) {
            *(uint64_t *)(codes + row * Kp + j * MX_GROUP + sub) = c;
            if ((lane & 15) == 0) *(uint32_t *)(scales + mx_scale_off(row, j, gpr)) = word;
        }
        if (next >= ntiles) break;
        tile = next;
        row = nrow;
        j = nj;
        cur = nxt;
    }
}

hipError_t launch_mx_quantize(const uint16_t *src, int64_t rows, int64_t K, uint8_t *dst,
                              hipStream_t s)
{
    if (rows <= 0) return hipSuccess;
    const int64_t Kp = mx_kp(K);
    // 16 row-groups a tile; row-groups numbered over ceil(rows/32)*32 rows
    const int64_t ntiles = ceil_div(rows, 32) * (Kp / MX_GROUP) * 2;
    if (ceil_div(rows, 32) * (Kp / MX_GROUP) >= ((int64_t)1 << 32)) return hipErrorInvalidValue;
    const int64_t grid = ntiles < 4096 ? ntiles : 4096;
    hipLaunchKernelGGL(k_mx_quantize, dim3((unsigned)grid), dim3(256), 0, s, src, rows, K, Kp, dst,
                       dst + rows * Kp, ntiles);
    return hipGetLastError();
}

// Column quantiser: a block takes 128 rows (one scale group of the output's
// k) by NCT*64 columns of a segment into LDS (rows gathered and scaled by a
// row weight on the way when asked; each source row gives NCT*128
// contiguous bytes), then each thread quantises one (column, 32-row block)
// per column tile: 32 codes, contiguous in the output row of that column,
// and its scale, gathered through LDS into the group's word.
template <int NCT>
__global__ __launch_bounds__(256) void k_mx_quantize_cols(ColQuant q)
{
    __shared__ __attribute__((aligned(16))) uint16_t tile[NCT * SEG_ROWS][64];
    __shared__ uint32_t sc[NCT][4][64];
    const int nct = (int)(q.C / (64 * NCT));
    const int ct = (blockIdx.x % nct) * NCT;
    __shared__ int32_t mt_s[SEG_MAX_E + 1];
    seg_stage_table(q, mt_s);
    __syncthreads();
    SegPos p;
    if (!seg_locate(q, mt_s, blockIdx.x / nct, p)) return;
    // uniform batches form one MX matrix [nseg*C, Kp]; experts one each, at
    // C * 132 bytes per 128-row chunk before them
    const int64_t rowbase = q.offsets ? 0 : p.seg * q.C;
    uint8_t *codes = q.offsets ? q.dst + q.C * 132 * p.chunk0 : q.dst;
    uint8_t *scales = codes + (q.offsets ? q.C : (int64_t)q.nseg * q.C) * p.Kp;
    const int64_t j = p.j, Kp = p.Kp;
    const int t = threadIdx.x;
    seg_load_tile<64, NCT>(q, p, ct, tile);
    __syncthreads();
    const int c = t & 63, b = t >> 6;
#pragma unroll
    for (int tt = 0; tt < NCT; ++tt) {
        float v[32];
        float amax = 0.f;
#pragma unroll
        for (int i = 0; i < 32; ++i) {
            v[i] = bf2f(tile[tt * SEG_ROWS + 32 * b + i][c]);
            amax = fmaxf(amax, fabsf(v[i]));
        }
        const int X = mx_block_exp(amax);
        uint32_t w[8];
#pragma unroll
        for (int h = 0; h < 4; ++h) {
            const float (&v8)[8] = *reinterpret_cast<const float(*)[8]>(&v[8 * h]);
            const uint64_t c8 = e4m3_codes8(v8, X);
            w[2 * h] = (uint32_t)c8;
            w[2 * h + 1] = (uint32_t)(c8 >> 32);
        }
        const int64_t orow = rowbase + (ct + tt) * 64 + c;
        uint8_t *dstc = codes + orow * Kp + j * MX_GROUP + b * 32;
        *(u32x4_t *)dstc = u32x4_t{w[0], w[1], w[2], w[3]};
        *(u32x4_t *)(dstc + 16) = u32x4_t{w[4], w[5], w[6], w[7]};
        sc[tt][b][c] = (uint32_t)(X + 127);
    }
    __syncthreads();
    if (b < NCT) {
        const int64_t orow = rowbase + (ct + b) * 64 + c;
        const uint32_t word =
            sc[b][0][c] | (sc[b][2][c] << 8) | (sc[b][1][c] << 16) | (sc[b][3][c] << 24);
        *(uint32_t *)(scales + mx_scale_off(orow, j, Kp / MX_GROUP)) = word;
    }
}

hipError_t launch_mx_quantize_cols(const ColQuant &q, int64_t max_chunks, hipStream_t s)
{
    // two column tiles a block where the columns allow it
    const bool two = (q.C / 64) % 2 == 0;
    const int64_t blocks = max_chunks * (q.C / (two ? 128 : 64));
    if (blocks <= 0) return hipSuccess;
    if (two) hipLaunchKernelGGL(k_mx_quantize_cols<2>, dim3((unsigned)blocks), dim3(256), 0, s, q);
    else hipLaunchKernelGGL(k_mx_quantize_cols<1>, dim3((unsigned)blocks), dim3(256), 0, s, q);
    return hipGetLastError();
}

// Both MX forms of a batch of matrices src [B, R, C] (bf16) from one read:
// the rows' form along C (dst_f, the MX matrix of [B*R, C]) and the
// transposes' form along R (dst_t, the MX matrix of the stacked transposes
// [B*C, R]).  A block takes a 128 x 128 tile of one batch into LDS (values
// past R or C read as zero), then
//   - along C: sixteen lanes a row, 8 values each (as k_mx_quantize), codes
//     and the row's scale word for that 128-column group;
//   - along R: one thread per (column, 32-row block) (as
//     k_mx_quantize_cols), 32 codes contiguous in the transposed row and the
//     scale bytes gathered through LDS into the group's word.
// Rows past R and columns past C are not written (they belong to the next
// batch); the codes and scales are those the two separate quantisers give.
constexpr int QB_PAD = 136;  // LDS row of the tile: 128 values + 16 bytes
__global__ __launch_bounds__(256) void k_mx_quantize_both(const uint16_t *src, int64_t B, int64_t R,
                                                          int64_t C, uint8_t *dst_f,
                                                          uint8_t *dst_t, int64_t ntiles)
{
    __shared__ __attribute__((aligned(16))) uint16_t tile[128][QB_PAD];
    __shared__ uint32_t sc[4][128];
    const int t = threadIdx.x, lane = t & 63;
    const int64_t nr = ceil_div(R, 128), nc = ceil_div(C, 128);
    const int64_t Cp = mx_kp(C), Rp = mx_kp(R);
    uint8_t *codes_f = dst_f, *scales_f = dst_f + B * R * Cp;
    uint8_t *codes_t = dst_t, *scales_t = dst_t + B * C * Rp;
    for (int64_t L = blockIdx.x; L < ntiles; L += gridDim.x) {
        const int64_t b = L / (nr * nc), rem = L % (nr * nc);
        const int64_t rj = rem / nc, cj = rem % nc;   // 128-row and 128-column group
        const int64_t r0 = rj * 128, c0 = cj * 128;
        const uint16_t *sb = src + b * R * C;
        // load: 16 lanes a row (16 bytes each), 16 rows per pass, 8 passes
        u32x4_t v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int64_t r = r0 + (t >> 4) + 16 * u, c = c0 + (t & 15) * 8;
            v[u] = (r < R && c < C) ? *(const u32x4_t *)(sb + r * C + c) : u32x4_t{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int u = 0; u < 8; ++u)
            *(u32x4_t *)&tile[(t >> 4) + 16 * u][(t & 15) * 8] = v[u];
        __syncthreads();
        // along C: row (t/16 + 16 u) of the tile, columns 8 (t%16) .. +7
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const u32x4_t x = v[u];
            float f[8];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                f[2 * q] = bf2f((uint16_t)(x[q] & 0xffffu));
                f[2 * q + 1] = bf2f((uint16_t)(x[q] >> 16));
            }
            uint32_t s8;
            const uint64_t cw = mx_quant8(f, s8);
            const uint32_t word = mx_group_word(s8, lane);
            const int64_t r = r0 + (t >> 4) + 16 * u;
            if (r < R) {
                const int64_t orow = b * R + r;
                *(uint64_t *)(codes_f + orow * Cp + c0 + (t & 15) * 8) = cw;
                if ((t & 15) == 0) *(uint32_t *)(scales_f + mx_scale_off(orow, cj, Cp / MX_GROUP)) = word;
            }
        }
        // along R: column (task % 128), 32-row block (task / 128)
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2) {
            const int task = t + 256 * k2, c = task & 127, blk = task >> 7;
            float f[32];
            float amax = 0.f;
#pragma unroll
            for (int i = 0; i < 32; ++i) {
                f[i] = bf2f(tile[32 * blk + i][c]);
                amax = fmaxf(amax, fabsf(f[i]));
            }
            const int X = mx_block_exp(amax);
            uint32_t w[8];
#pragma unroll
            for (int h = 0; h < 4; ++h) {
                const float (&f8)[8] = *reinterpret_cast<const float(*)[8]>(&f[8 * h]);
                const uint64_t c8 = e4m3_codes8(f8, X);
                w[2 * h] = (uint32_t)c8;
                w[2 * h + 1] = (uint32_t)(c8 >> 32);
            }
            if (c0 + c < C) {
                uint8_t *d = codes_t + (b * C + c0 + c) * Rp + r0 + blk * 32;
                *(u32x4_t *)d = u32x4_t{w[0], w[1], w[2], w[3]};
                *(u32x4_t *)(d + 16) = u32x4_t{w[4], w[5], w[6], w[7]};
            }
            sc[blk][c] = (uint32_t)(X + 127);
        }
        __syncthreads();
        if (t < 128 && c0 + t < C) {
            const uint32_t word = sc[0][t] | (sc[2][t] << 8) | (sc[1][t] << 16) | (sc[3][t] << 24);
            *(uint32_t *)(scales_t + mx_scale_off(b * C + c0 + t, rj, Rp / MX_GROUP)) = word;
        }
        __syncthreads();  // the tile and sc are reused by the next iteration
    }
}

hipError_t launch_mx_quantize_both(const uint16_t *src, int64_t B, int64_t R, int64_t C,
                                   uint8_t *dst_f, uint8_t *dst_t, hipStream_t s)
{
    const int64_t ntiles = B * ceil_div(R, 128) * ceil_div(C, 128);
    if (ntiles <= 0) return hipSuccess;
    const int64_t grid = ntiles < 65536 ? ntiles : 65536;
    hipLaunchKernelGGL(k_mx_quantize_both, dim3((unsigned)grid), dim3(256), 0, s, src, B, R, C,
                       dst_f, dst_t, ntiles);
    return hipGetLastError();
}

// ---------------------------------------------------------------- tiles ----
// BM x BN output tile of waves WM x WN; per stage 128 fp8 of k: A and B tiles
// of 128 bytes a row (as the bf16 tiles) plus the stage's scales, a 256-byte
// block per 32 rows (A rows 32q .. 32q+31 in its first half, the same B rows
// in its second).  Two stage buffers of each.
template <int BM_, int BN_, int WM_, int WN_>
struct MxCfg {
    static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_;
    static constexpr int WAVES_M = BM / WM, WAVES_N = BN / WN;
    static constexpr int NT = WAVES_M * WAVES_N * 64;
    static constexpr int FM = WM / 32, FN = WN / 32;
    static constexpr int A_BYTES = BM * 128, B_BYTES = BN * 128, S_BYTES = BM / 32 * 256;
    static constexpr int NS = BM / 32 / (NT / 64);  // scale blocks each wave copies
    static constexpr int RING_BYTES = 2 * (A_BYTES + B_BYTES + S_BYTES);
    static constexpr int LDS_BYTES = RING_BYTES > 131072 ? RING_BYTES : 131072;
    static_assert(BM == BN && NS * (NT / 64) * 32 == BM, "scale blocks split evenly over the waves");
    static_assert(LDS_BYTES <= 163840, "LDS of one CU");
    static constexpr int NHALF = BM / 128;  // 128-row epilogue passes
};
// Eight waves of 128 x 64 (two a SIMD, 256 registers each): 128 accumulator
// registers and one in-place set of six 32-byte fragments.
using MxTile = MxCfg<256, 256, 128, 64>;
// Four waves of 128 x 128 (one a SIMD; 256 accumulators in AGPRs, eight
// fragments): a third fewer fragment bytes read from LDS per MFMA.  Faster
// for the kernels whose epilogue is a plain fp32 store (GEMM2, dgrad1:
// +10% / +6%) and for the weight gradients, whose read-modify-write takes 16
// rows a wave per batch in the registers the AGPR accumulators leave free
// (dW1 -6%, dW2 -3% against eight waves at 8 rows); slower where the
// epilogue does per-row work that eight waves share (GEMM1's SwiGLU and MX
// quantisation, dgrad2).
using MxTile4 = MxCfg<256, 256, 128, 128>;

// 4 bytes per lane from a per-lane global address into LDS: lane l writes
// bytes [4 l, 4 l + 4) of the 256-byte block at dst (address in M0).  Issued
// from inline assembly for the same reason as copy16_to_lds.
MOE_DEV void copy4_to_lds(const void *src, lds_t *dst)
{
    const uint32_t m0v = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)dst);
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dword %0, off"
                 :
                 : "v"(src), "s"(m0v)
                 : "memory", "m0");
}

// The fragments of one k-step: one register set, refilled in place.
template <class C>
struct MxFrags {
    v8i32_t a[C::FM], b[C::FN];
    int32_t sa[C::FM], sb[C::FN];
};

// Operand fragment of rows rbase + lane%32 for k-step kk (0 or 1) of a stage.
MOE_DEV v8i32_t frag_mx(const lds_t *T, int rbase, int kk, int lane)
{
    const int r = rbase + (lane & 31), g = lane >> 5;
    const u32x4_t lo = *(const lds_u32x4 *)(T + lds_off(r, 4 * kk + g));
    const u32x4_t hi = *(const lds_u32x4 *)(T + lds_off(r, 4 * kk + 2 + g));
    const v8i32_t v = {(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                       (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
    return v;
}

// Scale word of rows rbase + lane%32 for this lane's half (side 0: A, 1: B).
MOE_DEV int32_t scale_mx(const lds_t *S, int rbase, int side, int lane)
{
    const int r = rbase + (lane & 31);
    return (int32_t) * (const lds_u16 *)(S + (r >> 5) * 256 + side * 128 + (r & 31) * 4 +
                                         (lane >> 5) * 2);
}

// Refill A fragment i / B fragment j with k-step kk of the given buffers; the
// scales change once per stage, so only step 0 reads them.
template <class C>
MOE_DEV void read_a_mx(int i, const lds_t *As, const lds_t *Ss, int kk, MxFrags<C> &f, int wm,
                       int lane)
{
    const int rb = wm * C::WM + i * 32;
    f.a[i] = frag_mx(As, rb, kk, lane);
    if (kk == 0) f.sa[i] = scale_mx(Ss, rb, 0, lane);
}
template <class C>
MOE_DEV void read_b_mx(int j, const lds_t *Bs, const lds_t *Ss, int kk, MxFrags<C> &f, int wn,
                       int lane)
{
    const int rb = wn * C::WN + j * 32;
    f.b[j] = frag_mx(Bs, rb, kk, lane);
    if (kk == 0) f.sb[j] = scale_mx(Ss, rb, 1, lane);
}

// The MFMAs of one k-step (scale byte OPSEL) in j-major order: MFMA n is
// (i, j) = (n % FM, n / FM).  Right after the last MFMA that uses a fragment
// the wave refills its registers with k-step kk_next from the given buffers
// (B fragment j after MFMA FM*j + FM-1, A fragment i after the last column's
// MFMA), so one register set serves both steps and every refill still has
// at least FM-1 MFMAs before its first use.  The NC copies are spread evenly
// over the MFMAs; sched_barrier pins the order.
template <class C, int OPSEL, int NC, class Copy>
MOE_DEV void kstep_mx(MxFrags<C> &f, const lds_t *As, const lds_t *Bs, const lds_t *Ss, int kk_next,
                      Copy &&copy, Acc<C> &acc, int wm, int wn, int lane)
{
    constexpr int NMF = C::FM * C::FN;
#pragma unroll
    for (int n = 0; n < NMF; ++n) {
        if constexpr (NC > 0) {
#pragma unroll
            for (int q = 0; q < NC; ++q)
                if (q * NMF / NC == n) copy(q);
        }
        __builtin_amdgcn_sched_barrier(0);
        const int i = n % C::FM, j = n / C::FM;
        acc.v[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
            f.b[j], f.a[i], acc.v[i][j], 0, 0, OPSEL, f.sb[j], OPSEL, f.sa[i]);
        __builtin_amdgcn_sched_barrier(0);
        if (i == C::FM - 1) read_b_mx<C>(j, Bs, Ss, kk_next, f, wn, lane);
        if (j == C::FN - 1) read_a_mx<C>(i, As, Ss, kk_next, f, wm, lane);
    }
}

// Software pipeline over stages 0 .. nst-1 (128 k each), two buffers per
// operand.  Stage v: step 0's MFMAs run while step 1's fragments are read
// (all of them before the step ends); then each wave waits for its copies of
// stage v+1, the barrier publishes them and frees stage v's buffers, and step
// 1's MFMAs run while step 0 of stage v+1 is read and stage v+2 is copied
// into the freed buffers (past the
// end the last stage again, into buffers nothing reads).  copy_a(q, v, As) /
// copy_b(q, v, Bs) issue data copy q of stage v, copy_s(q, v, Ss) scale copy q.
template <class C, int NCA, int NCB, class CopyA, class CopyB, class CopyS>
MOE_DEV void mx_pipeline(lds_t *lds, int nst, CopyA &&copy_a, CopyB &&copy_b, CopyS &&copy_s,
                         Acc<C> &acc)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = wave / C::WAVES_N, wn = wave % C::WAVES_N;
    lds_t *As[2] = {lds, lds + C::A_BYTES};
    lds_t *Bs[2] = {lds + 2 * C::A_BYTES, lds + 2 * C::A_BYTES + C::B_BYTES};
    lds_t *Ss[2] = {lds + 2 * (C::A_BYTES + C::B_BYTES),
                    lds + 2 * (C::A_BYTES + C::B_BYTES) + C::S_BYTES};
    acc.zero();
    if (nst <= 0) return;
    constexpr int NC = NCA + NCB + C::NS;
    auto clampv = [&](int v) { return v < nst ? v : nst - 1; };
    auto issue = [&](int q, int v, int b) {
        if (q < NCA) copy_a(q, v, As[b]);
        else if (q < NCA + NCB) copy_b(q - NCA, v, Bs[b]);
        else copy_s(q - NCA - NCB, v, Ss[b]);
    };
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int q = 0; q < NC; ++q) issue(q, clampv(s), s);
    wait_copies_le<NC>();
    __syncthreads();
    MxFrags<C> f;
#pragma unroll
    for (int j = 0; j < C::FN; ++j) read_b_mx<C>(j, Bs[0], Ss[0], 0, f, wn, lane);
#pragma unroll
    for (int i = 0; i < C::FM; ++i) read_a_mx<C>(i, As[0], Ss[0], 0, f, wm, lane);
    auto stage = [&](auto tag, int v) {
        constexpr int I = decltype(tag)::value;
        constexpr int b = I % 2, bn = (I + 1) % 2;
        kstep_mx<C, 0, 0>(f, As[b], Bs[b], Ss[b], 1, [](int) {}, acc, wm, wn, lane);
        wait_copies();  // stage v+1 (the only copies in flight)
        __syncthreads();
        const int vc = clampv(v + 2);
        kstep_mx<C, 1, NC>(f, As[bn], Bs[bn], Ss[bn], 0, [&](int q) { issue(q, vc, b); }, acc,
                           wm, wn, lane);
    };
    int v = 0;
    for (; v + 2 <= nst; v += 2) stage_run(stage, v, nst, std::make_integer_sequence<int, 2>());
    stage_run(stage, v, nst, std::make_integer_sequence<int, 1>());
    wait_copies();
    __syncthreads();
}

// Tile-local row of scale copy q of a wave: block wave*NS + q, lanes 0..31
// copy its A rows, lanes 32..63 its B rows.
template <class C>
MOE_DEV int scale_row(int wave, int q, int lane) { return (wave * C::NS + q) * 32 + (lane & 31); }

// =========================================================================
// GEMM1 (MXFP8) + SwiGLU
// =========================================================================
template <class C>
__global__ __launch_bounds__(C::NT) void k_up_swiglu_mx(GemmArgs g)
{
    __shared__ __attribute__((aligned(16))) char lds_raw[C::LDS_BYTES];
    lds_t *lds = (lds_t *)lds_raw;
    const int I = g.I;
    const int64_t Hp = g.Hp;
    const int nN = (int)ceil_div(I, C::BN / 2);
    MTile t;
    if (!decode_mtile<C::BM>(blockIdx.x, g.sched.mt_off256, g.offsets, g.E, nN, t)) return;
    const int lane0 = threadIdx.x & 63, wave0 = wave_uniform_id();
    KLoad<C::BM, C::NT> la;
    KLoad<C::BN, C::NT> lb;
    la.init(g.xq, wave0);
    lb.init(g.w1q + (int64_t)t.e * 2 * I * Hp, wave0);
    const int64_t i0 = (int64_t)t.nt * (C::BN / 2);
    auto tok_of = [&](int rr) {
        int64_t m = t.m0 + rr;
        if (m >= t.seg_end) m = t.seg_end - 1;
        return (int64_t)(g.row_map[m] / g.k);
    };
    // B tile row -> w1 row: wave column wn takes gate rows i0 + wn*WN/2 + [0, WN/2)
    // then the matching up rows
    auto w1_row = [&](int rr) {
        const int wn = rr / C::WN, qq = rr % C::WN, half = C::WN / 2;
        int64_t i = i0 + wn * half + (qq < half ? qq : qq - half);
        if (i >= I) i = I - 1;
        return qq < half ? i : I + i;
    };
#pragma unroll
    for (int q = 0; q < la.NI; ++q) la.set(q, lane0, (uint32_t)(tok_of(la.row(q, lane0)) * Hp));
#pragma unroll
    for (int q = 0; q < lb.NI; ++q) lb.set(q, lane0, (uint32_t)(w1_row(lb.row(q, lane0)) * Hp));
    const uint8_t *sp[C::NS];
#pragma unroll
    for (int q = 0; q < C::NS; ++q) {
        const int sr = scale_row<C>(wave0, q, lane0);
        sp[q] = lane0 < 32 ? g.xs + mx_scale_off(tok_of(sr), 0, Hp / MX_GROUP)
                           : g.w1s + mx_scale_off((int64_t)t.e * 2 * I + w1_row(sr), 0, Hp / MX_GROUP);
    }
    Acc<C> acc;
    mx_pipeline<C, KLoad<C::BM, C::NT>::NI, KLoad<C::BN, C::NT>::NI>(
        lds, (int)(Hp / MX_GROUP),
        [&](int q, int s, lds_t *As) { la.issue_one(q, As, (int64_t)s * 64, 0, la.base); },
        [&](int q, int s, lds_t *Bs) { lb.issue_one(q, Bs, (int64_t)s * 64, 0, lb.base); },
        [&](int q, int s, lds_t *Ss) {
            copy4_to_lds(sp[q] + s * 128, Ss + (wave0 * C::NS + q) * 256);
        },
        acc);
    swiglu_epilogue<C, true>(acc, lds, t, i0, I, g.h, g.a, g.aq, g.as_, g.Ip);
}

// The main loop of an MX tile: stages of 128 k from the two loaders, the
// scale copies from the per-lane scale rows sp (one per scale block the wave
// copies; the stage adds its group's 128-byte line).
template <class C>
MOE_DEV void mx_mainloop(lds_t *lds, int nst, const KLoad<C::BM, C::NT> &la,
                         const KLoad<C::BN, C::NT> &lb, const uint8_t *const (&sp)[C::NS],
                         int wave0, Acc<C> &acc)
{
    mx_pipeline<C, KLoad<C::BM, C::NT>::NI, KLoad<C::BN, C::NT>::NI>(
        lds, nst, [&](int q, int s, lds_t *As) { la.issue_one(q, As, (int64_t)s * 64, 0, la.base); },
        [&](int q, int s, lds_t *Bs) { lb.issue_one(q, Bs, (int64_t)s * 64, 0, lb.base); },
        [&](int q, int s, lds_t *Ss) {
            copy4_to_lds(sp[q] + s * 128, Ss + (wave0 * C::NS + q) * 256);
        },
        acc);
}

// =========================================================================
// Sorted rows against per-expert weight rows, fp32 out:
//   DOWN       o[r, c]   = A[r] . W2[e, c, :]       (A: a's MX matrix, K = I)
//   UP_DGRAD   dxp[r, c] = DH[r] . W1[e, :, c]      (DH: dh's MX matrix, B:
//              w1[e]^T's rows e*H + c, K = 2I)
// =========================================================================
template <class C, int OP>
__global__ __launch_bounds__(C::NT) void k_rows_mx(GemmArgs g)
{
    __shared__ __attribute__((aligned(16))) char lds_raw[C::LDS_BYTES];
    lds_t *lds = (lds_t *)lds_raw;
    constexpr bool DN = OP == MOE_GEMM_DOWN;
    const int N = g.H;
    const int64_t Kp = DN ? g.Ip : mx_kp(2 * (int64_t)g.I);
    const uint8_t *aq = DN ? g.aq : g.dhq, *as_ = DN ? g.as_ : g.dhs;
    const uint8_t *bq = DN ? g.w2q : g.w1cq, *bs = DN ? g.w2s : g.w1cs;
    float *out = DN ? g.o : g.dxp;
    const int nN = (int)ceil_div(N, C::BN);
    MTile t;
    if (!decode_mtile<C::BM>(blockIdx.x, g.sched.mt_off256, g.offsets, g.E, nN, t)) return;
    const int lane0 = threadIdx.x & 63, wave0 = wave_uniform_id();
    KLoad<C::BM, C::NT> la;
    KLoad<C::BN, C::NT> lb;
    la.init(aq, wave0);
    lb.init(bq + (int64_t)t.e * N * Kp, wave0);
    const int64_t n0 = (int64_t)t.nt * C::BN;
    auto a_row = [&](int rr) {
        int64_t m = t.m0 + rr;
        return m < t.seg_end ? m : t.seg_end - 1;
    };
    auto b_row = [&](int rr) {
        int64_t n = n0 + rr;
        return n < N ? n : (int64_t)N - 1;
    };
#pragma unroll
    for (int q = 0; q < la.NI; ++q) la.set(q, lane0, (uint32_t)(a_row(la.row(q, lane0)) * Kp));
#pragma unroll
    for (int q = 0; q < lb.NI; ++q) lb.set(q, lane0, (uint32_t)(b_row(lb.row(q, lane0)) * Kp));
    const uint8_t *sp[C::NS];
#pragma unroll
    for (int q = 0; q < C::NS; ++q) {
        const int sr = scale_row<C>(wave0, q, lane0);
        sp[q] = lane0 < 32 ? as_ + mx_scale_off(a_row(sr), 0, Kp / MX_GROUP)
                           : bs + mx_scale_off((int64_t)t.e * N + b_row(sr), 0, Kp / MX_GROUP);
    }
    Acc<C> acc;
    mx_mainloop<C>(lds, (int)(Kp / MX_GROUP), la, lb, sp, wave0, acc);
    if (DN && g.o_bf16) store_tile_f32<C>(acc, lds, g.o_bf16, t.m0, t.seg_end, n0, N);
    else if (!DN && g.dxp_bf16) store_tile_f32<C>(acc, lds, g.dxp_bf16, t.m0, t.seg_end, n0, N);
    else store_tile_f32<C>(acc, lds, out, t.m0, t.seg_end, n0, N);
}

// =========================================================================
// dgrad of GEMM2 (MXFP8) + row-dot + SwiGLU backward:
//   dA'[r, i] = DY[tok(r)] . W2[e, :, i]   (DY: dy's MX matrix along H,
//   B: w2[e]^T's rows e*I + i, K = H); epilogue as the bf16 kernel's
// =========================================================================
template <class C>
__global__ __launch_bounds__(C::NT) void k_down_dgrad_mx(GemmArgs g)
{
    __shared__ __attribute__((aligned(16))) char lds_raw[C::LDS_BYTES];
    lds_t *lds = (lds_t *)lds_raw;
    const int I = g.I;
    const int64_t Hp = g.Hp;
    const int nN = (int)ceil_div(I, C::BN);
    MTile t;
    if (!decode_mtile<C::BM>(blockIdx.x, g.sched.mt_off256, g.offsets, g.E, nN, t)) return;
    const int lane0 = threadIdx.x & 63, wave0 = wave_uniform_id();
    KLoad<C::BM, C::NT> la;
    KLoad<C::BN, C::NT> lb;
    la.init(g.dyq, wave0);
    lb.init(g.w2cq + (int64_t)t.e * I * Hp, wave0);
    const int64_t n0 = (int64_t)t.nt * C::BN;
    auto tok_of = [&](int rr) {
        int64_t m = t.m0 + rr;
        if (m >= t.seg_end) m = t.seg_end - 1;
        return (int64_t)(g.row_map[m] / g.k);
    };
    auto b_row = [&](int rr) {
        int64_t n = n0 + rr;
        return n < I ? n : (int64_t)I - 1;
    };
#pragma unroll
    for (int q = 0; q < la.NI; ++q) la.set(q, lane0, (uint32_t)(tok_of(la.row(q, lane0)) * Hp));
#pragma unroll
    for (int q = 0; q < lb.NI; ++q) lb.set(q, lane0, (uint32_t)(b_row(lb.row(q, lane0)) * Hp));
    const uint8_t *sp[C::NS];
#pragma unroll
    for (int q = 0; q < C::NS; ++q) {
        const int sr = scale_row<C>(wave0, q, lane0);
        sp[q] = lane0 < 32 ? g.dys + mx_scale_off(tok_of(sr), 0, Hp / MX_GROUP)
                           : g.w2cs + mx_scale_off((int64_t)t.e * I + b_row(sr), 0, Hp / MX_GROUP);
    }
    Acc<C> acc;
    mx_mainloop<C>(lds, (int)(Hp / MX_GROUP), la, lb, sp, wave0, acc);
    dgrad2_epilogue<C, 4>(acc, lds, t, n0, nN, I, g.h, g.a, g.wrow, g.dh, g.dw_part);
}

// =========================================================================
// Weight gradients (MXFP8), K-grouped over each expert's routed rows:
//   DOWN:  dW2[e, hh, i] (+)= sum_r DYW[r, hh] A[r, i]
//   UP:    dW1[e, n, hh] (+)= sum_r DH[r, n] XG[r, hh]
// Both operands are the per-expert MX matrices of their transposes (rows =
// the output's rows / columns, K = the expert's rows padded to 128), so the
// tile is K-major on both sides like the forward ones.
// =========================================================================
template <class C, bool UP>
__global__ __launch_bounds__(C::NT) void k_wgrad_mx(GemmArgs g)
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
    constexpr int GR = 4;  // groups of GR row tiles sweep all column tiles
    const int64_t rest = L % tpe;
    const int64_t grp = rest / ((int64_t)GR * nC);
    const int64_t first = grp * GR;
    const int64_t gr = nR - first < GR ? nR - first : GR;
    const int64_t in = rest - grp * (int64_t)GR * nC;
    const int rt = (int)(first + in % gr), ct = (int)(in / gr);
    const int64_t r0 = (int64_t)rt * C::BM, c0 = (int64_t)ct * C::BN;
    const int32_t *mt = g.sched.mt_off128;
    const int64_t Kp = (int64_t)MX_GROUP * (mt[e + 1] - mt[e]);
    const uint8_t *Aq = g.segA + (int64_t)R * 132 * mt[e], *As_ = Aq + (int64_t)R * Kp;
    const uint8_t *Bq = g.segB + (int64_t)Cc * 132 * mt[e], *Bs_ = Bq + (int64_t)Cc * Kp;
    const int lane0 = threadIdx.x & 63, wave0 = wave_uniform_id();
    KLoad<C::BM, C::NT> la;
    KLoad<C::BN, C::NT> lb;
    la.init(Aq, wave0);
    lb.init(Bq, wave0);
    auto a_row = [&](int rr) { return r0 + rr < R ? r0 + rr : (int64_t)R - 1; };
    auto b_row = [&](int rr) { return c0 + rr < Cc ? c0 + rr : (int64_t)Cc - 1; };
#pragma unroll
    for (int q = 0; q < la.NI; ++q) la.set(q, lane0, (uint32_t)(a_row(la.row(q, lane0)) * Kp));
#pragma unroll
    for (int q = 0; q < lb.NI; ++q) lb.set(q, lane0, (uint32_t)(b_row(lb.row(q, lane0)) * Kp));
    const uint8_t *sp[C::NS];
#pragma unroll
    for (int q = 0; q < C::NS; ++q) {
        const int sr = scale_row<C>(wave0, q, lane0);
        sp[q] = lane0 < 32 ? As_ + mx_scale_off(a_row(sr), 0, Kp / MX_GROUP)
                           : Bs_ + mx_scale_off(b_row(sr), 0, Kp / MX_GROUP);
    }
    Acc<C> acc;
    mx_mainloop<C>(lds, (int)(Kp / MX_GROUP), la, lb, sp, wave0, acc);
    wgrad_epilogue<C, 4096 / C::NT>(acc, lds, r0, c0, R, Cc, (int64_t)e * R * Cc, UP ? g.dW1 : g.dW2,
                         g.dw_acc, g.dw_bf16);
}

hipError_t launch_mx_gemm(int32_t op, const GemmArgs &g, hipStream_t s)
{
    using C = MxTile;
    auto mgrid = [&](int64_t ncols, int per) {
        return dim3((unsigned)mgrid_blocks(g.M, g.E, C::BM, (int)ceil_div(ncols, per)));
    };
    auto wgrid = [&](int64_t R, int64_t Cc) {
        const int64_t tiles = ceil_div(R, MxTile4::BM) * ceil_div(Cc, MxTile4::BN);
        return dim3((unsigned)grid_for(tiles * g.E));
    };
    switch (op) {
    case MOE_GEMM_UP_SWIGLU:
        hipLaunchKernelGGL(k_up_swiglu_mx<C>, mgrid(g.I, C::BN / 2), dim3(C::NT), 0, s, g);
        break;
    case MOE_GEMM_DOWN:
        hipLaunchKernelGGL((k_rows_mx<MxTile4, MOE_GEMM_DOWN>), mgrid(g.H, MxTile4::BN),
                           dim3(MxTile4::NT), 0, s, g);
        break;
    case MOE_GEMM_DOWN_DGRAD:
        // the router backward reads dgrad2_cols(I) row-dot partials per row
        if (ceil_div(g.I, C::BN) != dgrad2_cols(g.I)) return hipErrorInvalidValue;
        hipLaunchKernelGGL(k_down_dgrad_mx<C>, mgrid(g.I, C::BN), dim3(C::NT), 0, s, g);
        break;
    case MOE_GEMM_UP_DGRAD:
        hipLaunchKernelGGL((k_rows_mx<MxTile4, MOE_GEMM_UP_DGRAD>), mgrid(g.H, MxTile4::BN),
                           dim3(MxTile4::NT), 0, s, g);
        break;
    case MOE_GEMM_DOWN_WGRAD:
        hipLaunchKernelGGL((k_wgrad_mx<MxTile4, false>), wgrid(g.H, g.I), dim3(MxTile4::NT), 0, s,
                           g);
        break;
    case MOE_GEMM_UP_WGRAD:
        hipLaunchKernelGGL((k_wgrad_mx<MxTile4, true>), wgrid(2 * (int64_t)g.I, g.H),
                           dim3(MxTile4::NT), 0, s, g);
        break;
    default:
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace moe
