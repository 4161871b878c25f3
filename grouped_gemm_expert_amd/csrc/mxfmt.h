// MXFP8 element and scale encoding on the device: OCP Microscaling blocks of
// 32 values along the contraction dimension, one E8M0 scale 2^X per block with
// X = floor(log2(amax)) - 8 (8 = exponent of E4M3's largest normal, 448),
// clamped below at -127, and E4M3 elements rounded to nearest-even from
// v / 2^X with saturation to +-448.  (MegaMoE page, "Expert precision": the
// mxfp8 mode of the expert stages.)
//
// MX matrix layout used by the library: a bf16 matrix [rows, K] quantised
// along K becomes codes [rows, Kp] (Kp = K rounded up to 128, padding codes 0)
// followed by the scales.  A row has one 4-byte scale word per 128-column
// group, holding the group's four block scales in the order of blocks 0, 2,
// 1, 3: one 16-bit read then yields, for one half of a wave, the scales of
// both 64-deep MFMA steps of that group (low byte: first step, high byte:
// second).  The words are stored in 32-row blocks, [ceil(rows/32)][Kp/128]
// [32][4 bytes], so that the words of 32 consecutive rows for one group are
// one contiguous 128-byte line (one line per copy instead of 32).
#pragma once

#include "common.h"

namespace moe {

constexpr int MX_GROUP = 128;  // columns per scale word

__host__ __device__ inline int64_t mx_kp(int64_t K) { return (K + MX_GROUP - 1) / MX_GROUP * MX_GROUP; }

// Byte offset of the scale word of (row, group) in the scale area, gpr =
// Kp / 128 groups per row.
__host__ __device__ inline int64_t mx_scale_off(int64_t row, int64_t group, int64_t gpr)
{
    return ((row >> 5) * gpr + group) * 128 + (row & 31) * 4;
}

// Bytes of the scale area of an MX matrix with `rows` rows.
inline int64_t mx_scale_bytes(int64_t rows, int64_t K) { return (rows + 31) / 32 * 32 * (mx_kp(K) / 32); }

// X of a block with largest magnitude amax (finite, >= 0).
MOE_DEV int mx_block_exp(float amax)
{
    const uint32_t u = __float_as_uint(amax);
    const int ev = (int)(u >> 23);
    int e;
    if (ev) {
        e = ev - 127;
    } else {
        const uint32_t m = u & 0x7FFFFFu;
        if (!m) return -127;
        e = -149 + (31 - __builtin_clz(m));
    }
    const int X = e - 8;
    return X < -127 ? -127 : X;
}

// E4M3 code of v / 2^X, nearest-even, saturating; exact integer arithmetic on
// the fp32 bits.  |v| / 2^X = sig * 2^E0; the E4M3 grid around it has spacing
// 2^kq, kq = max(floor(log2 |v / 2^X|), -6) - 3 (the -6 floor is the subnormal
// range), so the code's magnitude is sig / 2^(kq - E0) rounded to an integer n
// and placed into the exponent / mantissa fields.
MOE_DEV uint32_t e4m3_code(float v, int X)
{
    const uint32_t u = __float_as_uint(v);
    const uint32_t sign = (u >> 24) & 0x80u;
    const int ev = (int)((u >> 23) & 255u);
    uint32_t sig = u & 0x7FFFFFu;
    if (ev) sig |= 0x800000u;
    if (!sig) return sign;
    const int E0 = (ev ? ev : 1) - 150 - X;
    const int eq = E0 + (31 - __builtin_clz(sig));
    const int kq = (eq > -6 ? eq : -6) - 3;
    const int sh = kq - E0;
    uint32_t n;
    if (sh <= 0) {
        n = sig << (-sh);  // only tiny subnormal inputs: exact
    } else if (sh > 25) {
        n = 0;
    } else {
        n = sig >> sh;
        const uint32_t rem = sig & ((1u << sh) - 1u), half = 1u << (sh - 1);
        n += (rem > half || (rem == half && (n & 1u))) ? 1u : 0u;
    }
    // normal: n in [8, 16] at exponent eq = kq + 3 (n = 16 carries into the
    // next exponent); subnormal: n in [0, 8], which is the code itself
    uint32_t c = eq >= -6 ? ((uint32_t)(kq + 10) << 3) + n - 8u : n;
    c = c < 0x7Eu ? c : 0x7Eu;
    return sign | c;
}

// Lanes 4b .. 4b+3 of a wave hold the 32 values of one block, 8 each (in
// column order).  Returns this lane's 8 codes (byte q = value q) and the
// block's scale code X + 127.  Every lane of the wave must call it.
MOE_DEV uint64_t mx_quant8(const float (&v)[8], uint32_t &scale)
{
    float amax = 0.f;
#pragma unroll
    for (int q = 0; q < 8; ++q) amax = fmaxf(amax, fabsf(v[q]));
    amax = fmaxf(amax, __shfl_xor(amax, 1, 64));
    amax = fmaxf(amax, __shfl_xor(amax, 2, 64));
    const int X = mx_block_exp(amax);
    uint64_t c = 0;
#pragma unroll
    for (int q = 0; q < 8; ++q) c |= (uint64_t)e4m3_code(v[q], X) << (8 * q);
    scale = (uint32_t)(X + 127);
    return c;
}

// Lanes 16g .. 16g+15 hold one 128-column group (blocks b = lane/4 % 4): the
// group's scale word with block b at byte 2*(b%2) + b/2.  Every lane of the
// wave must call it; all 16 lanes of a group receive the word.
MOE_DEV uint32_t mx_group_word(uint32_t scale, int lane)
{
    const int b = (lane >> 2) & 3;
    uint32_t w = scale << (8 * ((b & 1) * 2 + (b >> 1)));
    w |= __shfl_xor(w, 4, 64);
    w |= __shfl_xor(w, 8, 64);
    return w;
}

}  // namespace moe
