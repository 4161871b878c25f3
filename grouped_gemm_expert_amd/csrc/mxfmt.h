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

// E4M3 codes of v[0..7] / 2^X (byte q: v[q]).  Dividing by 2^X is an exact
// multiplication by a power of two (the inputs are bf16 values, and a result
// below fp32's normal range lies far below half of E4M3's smallest subnormal,
// so it becomes zero either way); the clamp to +-448 is the format's
// saturation; v_cvt_pk_fp8_f32 then rounds to nearest even onto the OCP E4M3
// grid, subnormals included.
MOE_DEV uint64_t e4m3_codes8(const float (&v)[8], int X)
{
    const float f = __uint_as_float((uint32_t)(127 - X) << 23);
    uint32_t w[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        float s[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) s[q] = fminf(fmaxf(v[4 * h + q] * f, -448.f), 448.f);
        int p = __builtin_amdgcn_cvt_pk_fp8_f32(s[0], s[1], 0, false);
        p = __builtin_amdgcn_cvt_pk_fp8_f32(s[2], s[3], p, true);
        w[h] = (uint32_t)p;
    }
    return (uint64_t)w[0] | ((uint64_t)w[1] << 32);
}

// Largest of a over each group of 4 lanes (4b .. 4b+3), by DPP quad
// permutations (lanes 1,0,3,2 then 2,3,0,1).
MOE_DEV float quad_max(float a)
{
    a = fmaxf(a, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(a), 0xB1, 0xF, 0xF, false)));
    a = fmaxf(a, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(a), 0x4E, 0xF, 0xF, false)));
    return a;
}

// Lanes 4b .. 4b+3 of a wave hold the 32 values of one block, 8 each (in
// column order).  Returns this lane's 8 codes (byte q = value q) and the
// block's scale code X + 127.  Every lane of the wave must call it.
MOE_DEV uint64_t mx_quant8(const float (&v)[8], uint32_t &scale)
{
    float amax = 0.f;
#pragma unroll
    for (int q = 0; q < 8; ++q) amax = fmaxf(amax, fabsf(v[q]));
    const int X = mx_block_exp(quad_max(amax));
    scale = (uint32_t)(X + 127);
    return e4m3_codes8(v, X);
}

// Lanes 16g .. 16g+15 hold one 128-column group (blocks b = lane/4 % 4): the
// group's scale word with block b at byte 2*(b%2) + b/2.  Every lane of the
// wave must call it; all 16 lanes of a group receive the word.  (ds_swizzle
// in bit-mask mode: lane l reads lane l ^ 4, then l ^ 8.)
MOE_DEV uint32_t mx_group_word(uint32_t scale, int lane)
{
    const int b = (lane >> 2) & 3;
    uint32_t w = scale << (8 * ((b & 1) * 2 + (b >> 1)));
    w |= (uint32_t)__builtin_amdgcn_ds_swizzle((int)w, 0x101F);
    w |= (uint32_t)__builtin_amdgcn_ds_swizzle((int)w, 0x201F);
    return w;
}

}  // namespace moe
