// Router kernels: selection + routing weights + counts + aux partials, aux
// finalize.  (The router projection and its gradients are in dense.hip.)
//
// Follows the MegaMoE page (Primus technical guide), intro: the fused router
// is a score function, a group-limited top-k and an aux score.
#include "common.h"

namespace moe {

// ---------------------------------------------------------------- fills ----
__global__ void k_fill_i32(int32_t *p, int64_t n, int32_t v)
{
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * blockDim.x)
        p[i] = v;
}
__global__ void k_fill_f32(float *p, int64_t n, float v)
{
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * blockDim.x)
        p[i] = v;
}
hipError_t launch_fill_i32(int32_t *p, int64_t n, int32_t v, hipStream_t s)
{
    if (n <= 0) return hipSuccess;
    int64_t blocks = ceil_div(n, 256);
    if (blocks > 4096) blocks = 4096;
    k_fill_i32<<<(unsigned)blocks, 256, 0, s>>>(p, n, v);
    return hipGetLastError();
}
hipError_t launch_fill_f32(float *p, int64_t n, float v, hipStream_t s)
{
    if (n <= 0) return hipSuccess;
    int64_t blocks = ceil_div(n, 256);
    if (blocks > 4096) blocks = 4096;
    k_fill_f32<<<(unsigned)blocks, 256, 0, s>>>(p, n, v);
    return hipGetLastError();
}

// -------------------------------------------------------------- router ----
// One wavefront per token; a block holds 4 waves and walks TOK_PER_BLOCK
// tokens, accumulating the aux column sums of its tokens in registers and
// their expert counts in LDS (no global atomics: a skewed router would
// serialise them on a few addresses); both go out as per-block partials.
// Expert e lives in lane e % 64, register slot e / 64.
constexpr int RT_WAVES = 4;
constexpr int RT_TOK_PER_WAVE = 1;  // a token is a serial chain: keep many waves
constexpr int RT_TOK_PER_BLOCK = RT_WAVES * RT_TOK_PER_WAVE;

int64_t router_blocks(int64_t T) { return ceil_div(T, RT_TOK_PER_BLOCK); }

template <int EPL>
__global__ __launch_bounds__(256) void k_router_select(RouterArgs p)
{
    __shared__ float sS[RT_WAVES][64 * EPL];
    __shared__ float red[RT_WAVES][64 * EPL];
    __shared__ int32_t bcnt[64 * EPL];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int E = p.E, k = p.k;
    for (int e = threadIdx.x; e < 64 * EPL; e += blockDim.x) bcnt[e] = 0;
    __syncthreads();
    float colsum[EPL];
#pragma unroll
    for (int q = 0; q < EPL; ++q) colsum[q] = 0.f;

    for (int it = 0; it < RT_TOK_PER_WAVE; ++it) {
        const int64_t t = (int64_t)blockIdx.x * RT_TOK_PER_BLOCK + wave * RT_TOK_PER_WAVE + it;
        if (t >= p.T) break;  // wave-uniform
        float l[EPL], S[EPL], sc[EPL];
        bool ok[EPL];
#pragma unroll
        for (int q = 0; q < EPL; ++q) {
            int e = lane + 64 * q;
            ok[q] = e < E;
            l[q] = ok[q] ? p.logits[t * E + e] : 0.f;
            if (p.score == MOE_SOFTMAX) {
                S[q] = l[q];
            } else {
                // fp32(sigmoid(l)) evaluated in double, then rounded once
                float s = (float)(1.0 / (1.0 + exp(-(double)l[q])));
                sc[q] = s;
                S[q] = s + ((p.bias && ok[q]) ? p.bias[e] : 0.f);
            }
            S[q] = sel_key(S[q]);  // a NaN score ranks as -inf
            if (p.sel && ok[q]) p.sel[t * E + e] = S[q];
        }
        // softmax probabilities (fp32) of all experts
        if (p.score == MOE_SOFTMAX) {
            float m = -INFINITY;
#pragma unroll
            for (int q = 0; q < EPL; ++q)
                if (ok[q]) m = fmaxf(m, l[q]);
            m = wave_max(m);
            float z = 0.f;
#pragma unroll
            for (int q = 0; q < EPL; ++q) {
                sc[q] = ok[q] ? expf(l[q] - m) : 0.f;
                z += sc[q];
            }
            z = wave_sum(z);
            float rz = 1.0f / z;
#pragma unroll
            for (int q = 0; q < EPL; ++q) sc[q] *= rz;
        }
        // eligibility under the group limit
        bool elig[EPL];
#pragma unroll
        for (int q = 0; q < EPL; ++q) elig[q] = ok[q];
        if (p.G > 1 && !p.even) {
            const int gsz = E / p.G;
#pragma unroll
            for (int q = 0; q < EPL; ++q)
                if (ok[q]) sS[wave][lane + 64 * q] = S[q];
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            float gsv = 0.f;
            int gid = -1;
            if (lane < p.G) {
                float b1 = 0.f, b2 = 0.f;
                int i1 = -1, i2 = -1;
                for (int e = lane * gsz; e < (lane + 1) * gsz; ++e) {
                    float v = sS[wave][e];
                    if (ranks_before(v, e, b1, i1)) {
                        b2 = b1; i2 = i1; b1 = v; i1 = e;
                    } else if (ranks_before(v, e, b2, i2)) {
                        b2 = v; i2 = e;
                    }
                }
                gsv = sel_key((i2 >= 0) ? b1 + b2 : b1);  // inf - inf ranks as -inf
                gid = lane;
            }
            uint64_t kept = 0;
            for (int r = 0; r < p.kg; ++r) {
                float v = gsv;
                int i = gid;
                wave_argmax(v, i);
                kept |= 1ull << i;
                if (lane == i) gid = -1;
            }
#pragma unroll
            for (int q = 0; q < EPL; ++q) {
                int e = lane + 64 * q;
                elig[q] = ok[q] && ((kept >> (e / gsz)) & 1ull);
            }
            __builtin_amdgcn_wave_barrier();
        }
        // top-k by repeated wave arg-max, or the `even` forced experts
        int my_idx = -1;
        float my_val = 0.f;
        float zsel = 0.f;
        for (int j = 0; j < k; ++j) {
            float bv = 0.f;
            int bi = -1;
            if (p.even) {
                bi = (int)((t * k + j) % E);
            } else {
#pragma unroll
                for (int q = 0; q < EPL; ++q) {
                    int e = lane + 64 * q;
                    if (elig[q] && ranks_before(S[q], e, bv, bi)) { bv = S[q]; bi = e; }
                }
                wave_argmax(bv, bi);
            }
            // owner lane removes the winner and publishes its prob / sigmoid
            float pv = 0.f;
            if ((bi & 63) == lane) {
#pragma unroll
                for (int q = 0; q < EPL; ++q)
                    if (lane + 64 * q == bi) { elig[q] = false; pv = sc[q]; }
            }
            pv = __shfl(pv, bi & 63, 64);
            zsel += pv;
            if (lane == j) { my_idx = bi; my_val = pv; }
        }
        if (lane < k) {
            float w;
            if (p.score == MOE_SOFTMAX) w = p.renorm ? my_val / zsel : my_val;
            else w = p.scale * my_val / zsel;
            p.topk_idx[t * k + lane] = my_idx;
            p.topk_w[t * k + lane] = w;
            if (my_idx >= 0) atomicAdd(&bcnt[my_idx], 1);
        }
        // aux probabilities: softmax p, or s / sum_e s for the sigmoid router
        if (p.score == MOE_SOFTMAX) {
#pragma unroll
            for (int q = 0; q < EPL; ++q) colsum[q] += sc[q];
        } else {
            float z = 0.f;
#pragma unroll
            for (int q = 0; q < EPL; ++q) z += ok[q] ? sc[q] : 0.f;
            z = wave_sum(z);
            float rz = 1.0f / z;
#pragma unroll
            for (int q = 0; q < EPL; ++q) colsum[q] += ok[q] ? sc[q] * rz : 0.f;
        }
    }
    // block partial of the column sums: fixed order over the waves
#pragma unroll
    for (int q = 0; q < EPL; ++q) red[wave][lane + 64 * q] = colsum[q];
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += blockDim.x) {
        float v = 0.f;
#pragma unroll
        for (int w = 0; w < RT_WAVES; ++w) v += red[w][e];
        p.prob_part[(int64_t)blockIdx.x * E + e] = v;
        p.cnt_part[(int64_t)blockIdx.x * E + e] = bcnt[e];
    }
}

// ------------------------------------------------- router, 16 lanes a token ----
// The same selection with a token on a row of 16 lanes, four tokens a wave
// (E <= 256, G <= 16, k <= 16): expert e lives in lane e % 16 of the row,
// register slot e / 16, and every arg-max is the four DPP steps inside the
// row, with no cross-row shuffle; a wave's four tokens share each instruction.
// A row past the last token computes on the last token and writes nothing,
// so every lane takes part in the row-wide DPP steps.
constexpr int RQ_WAVES = 4;
constexpr int RQ_TOK_PER_BLOCK = RQ_WAVES * 4;

bool router_rows16(int32_t E, int32_t G, int32_t k) { return E <= 256 && G <= 16 && k <= 16; }

// Row-wide (16 lanes) arg-max under ranks_before; every lane of the row gets
// the winner.
MOE_DEV void row_argmax(float &v, int &i)
{
    argmax_dpp_step<0xB1>(v, i);   // quad_perm(1, 0, 3, 2)
    argmax_dpp_step<0x4E>(v, i);   // quad_perm(2, 3, 0, 1)
    argmax_dpp_step<0x141>(v, i);  // row_half_mirror
    argmax_dpp_step<0x140>(v, i);  // row_mirror
}

template <int CTRL>
MOE_DEV float dpp_f(float v)
{
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
MOE_DEV float row_sum16(float v)
{
    v += dpp_f<0xB1>(v);
    v += dpp_f<0x4E>(v);
    v += dpp_f<0x141>(v);
    return v + dpp_f<0x140>(v);
}
MOE_DEV float row_max16(float v)
{
    v = fmaxf(v, dpp_f<0xB1>(v));
    v = fmaxf(v, dpp_f<0x4E>(v));
    v = fmaxf(v, dpp_f<0x141>(v));
    return fmaxf(v, dpp_f<0x140>(v));
}

template <int EPL>
__global__ __launch_bounds__(256) void k_router_select16(RouterArgs p)
{
    __shared__ float sS[RQ_TOK_PER_BLOCK][16 * EPL];
    __shared__ float red[RQ_WAVES][16 * EPL];
    __shared__ int32_t bcnt[16 * EPL];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int j = lane & 15, slot = wave * 4 + (lane >> 4);
    const int rbase = lane & ~15;
    const int E = p.E, k = p.k;
    for (int e = threadIdx.x; e < 16 * EPL; e += blockDim.x) bcnt[e] = 0;
    __syncthreads();
    const int64_t t0 = (int64_t)blockIdx.x * RQ_TOK_PER_BLOCK + slot;
    const bool tok = t0 < p.T;
    const int64_t t = tok ? t0 : p.T - 1;
    float l[EPL], S[EPL], sc[EPL];
    bool ok[EPL];
#pragma unroll
    for (int q = 0; q < EPL; ++q) {
        const int e = j + 16 * q;
        ok[q] = e < E;
        l[q] = ok[q] ? p.logits[t * E + e] : 0.f;
        if (p.score == MOE_SOFTMAX) {
            S[q] = l[q];
        } else {
            // fp32(sigmoid(l)) evaluated in double, then rounded once
            const float sg = (float)(1.0 / (1.0 + exp(-(double)l[q])));
            sc[q] = sg;
            S[q] = sg + ((p.bias && ok[q]) ? p.bias[e] : 0.f);
        }
        S[q] = sel_key(S[q]);  // a NaN score ranks as -inf
        if (p.sel && ok[q] && tok) p.sel[t * E + e] = S[q];
    }
    if (p.score == MOE_SOFTMAX) {
        float m = -INFINITY;
#pragma unroll
        for (int q = 0; q < EPL; ++q)
            if (ok[q]) m = fmaxf(m, l[q]);
        m = row_max16(m);
        float z = 0.f;
#pragma unroll
        for (int q = 0; q < EPL; ++q) {
            sc[q] = ok[q] ? expf(l[q] - m) : 0.f;
            z += sc[q];
        }
        z = row_sum16(z);
        const float rz = 1.0f / z;
#pragma unroll
        for (int q = 0; q < EPL; ++q) sc[q] *= rz;
    }
    // eligibility under the group limit: lane g < G of the row scores group g
    // (its best two selection scores, from LDS), then kg row arg-max rounds
    bool elig[EPL];
#pragma unroll
    for (int q = 0; q < EPL; ++q) elig[q] = ok[q];
    if (p.G > 1 && !p.even) {
        const int gsz = E / p.G;
#pragma unroll
        for (int q = 0; q < EPL; ++q)
            if (ok[q]) sS[slot][j + 16 * q] = S[q];
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        float gsv = 0.f;
        int gid = -1;
        if (j < p.G) {
            float b1 = 0.f, b2 = 0.f;
            int i1 = -1, i2 = -1;
            for (int e = j * gsz; e < (j + 1) * gsz; ++e) {
                const float v = sS[slot][e];
                if (ranks_before(v, e, b1, i1)) {
                    b2 = b1; i2 = i1; b1 = v; i1 = e;
                } else if (ranks_before(v, e, b2, i2)) {
                    b2 = v; i2 = e;
                }
            }
            gsv = sel_key((i2 >= 0) ? b1 + b2 : b1);  // inf - inf ranks as -inf
            gid = j;
        }
        uint32_t kept = 0;
        for (int r = 0; r < p.kg; ++r) {
            float v = gsv;
            int i = gid;
            row_argmax(v, i);
            kept |= 1u << i;
            if (j == i) gid = -1;
        }
#pragma unroll
        for (int q = 0; q < EPL; ++q) elig[q] = ok[q] && ((kept >> ((j + 16 * q) / gsz)) & 1u);
        __builtin_amdgcn_wave_barrier();
    }
    // top-k by repeated row arg-max, or the `even` forced experts; the owner
    // lane removes the winner and the row reads its probability / sigmoid
    int my_idx = -1;
    float my_val = 0.f, zsel = 0.f;
    for (int r = 0; r < k; ++r) {
        float bv = 0.f;
        int bi = -1;
        if (p.even) {
            bi = (int)((t * k + r) % E);
        } else {
#pragma unroll
            for (int q = 0; q < EPL; ++q) {
                const int e = j + 16 * q;
                if (elig[q] && ranks_before(S[q], e, bv, bi)) { bv = S[q]; bi = e; }
            }
            row_argmax(bv, bi);
        }
        float pv = 0.f;
        if ((bi & 15) == j) {
#pragma unroll
            for (int q = 0; q < EPL; ++q)
                if (j + 16 * q == bi) { elig[q] = false; pv = sc[q]; }
        }
        pv = __shfl(pv, rbase + (bi & 15), 64);
        zsel += pv;
        if (j == r) { my_idx = bi; my_val = pv; }
    }
    if (j < k && tok) {
        float w;
        if (p.score == MOE_SOFTMAX) w = p.renorm ? my_val / zsel : my_val;
        else w = p.scale * my_val / zsel;
        p.topk_idx[t * k + j] = my_idx;
        p.topk_w[t * k + j] = w;
        if (my_idx >= 0) atomicAdd(&bcnt[my_idx], 1);
    }
    // aux probabilities: softmax p, or s / sum_e s for the sigmoid router
    float colsum[EPL];
    if (p.score == MOE_SOFTMAX) {
#pragma unroll
        for (int q = 0; q < EPL; ++q) colsum[q] = tok ? sc[q] : 0.f;
    } else {
        float z = 0.f;
#pragma unroll
        for (int q = 0; q < EPL; ++q) z += ok[q] ? sc[q] : 0.f;
        z = row_sum16(z);
        const float rz = 1.0f / z;
#pragma unroll
        for (int q = 0; q < EPL; ++q) colsum[q] = (ok[q] && tok) ? sc[q] * rz : 0.f;
    }
    // the wave's four rows, then the block's waves, in a fixed order
#pragma unroll
    for (int q = 0; q < EPL; ++q) {
        colsum[q] += __shfl_xor(colsum[q], 16, 64);
        colsum[q] += __shfl_xor(colsum[q], 32, 64);
    }
    if (lane < 16) {
#pragma unroll
        for (int q = 0; q < EPL; ++q) red[wave][j + 16 * q] = colsum[q];
    }
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += blockDim.x) {
        float v = 0.f;
#pragma unroll
        for (int w = 0; w < RQ_WAVES; ++w) v += red[w][e];
        p.prob_part[(int64_t)blockIdx.x * E + e] = v;
        p.cnt_part[(int64_t)blockIdx.x * E + e] = bcnt[e];
    }
}

// The router blocks' partials are reduced in two fixed-order steps, so the
// result is deterministic and no single block walks all of them.
// Step 1 (k_aux_slices): block s sums router blocks [s*AUX_SLICE,
// (s+1)*AUX_SLICE) in ascending order, for every expert.
constexpr int AUX_SLICE = 32;

int64_t aux_slices(int64_t T) { return ceil_div(router_blocks(T), AUX_SLICE); }

__global__ __launch_bounds__(256) void k_aux_slices(RouterArgs p, int64_t nblk)
{
    const int E = p.E;
    const int64_t b0 = (int64_t)blockIdx.x * AUX_SLICE;
    const int64_t b1 = b0 + AUX_SLICE < nblk ? b0 + AUX_SLICE : nblk;
    for (int e = threadIdx.x; e < E; e += blockDim.x) {
        float P = 0.f;
        int32_t n = 0;
        for (int64_t b = b0; b < b1; ++b) {
            P += p.prob_part[b * E + e];
            n += p.cnt_part[b * E + e];
        }
        p.prob_slice[blockIdx.x * (int64_t)E + e] = P;
        p.cnt_slice[blockIdx.x * (int64_t)E + e] = n;
    }
}

// Step 2 (one block of 1024 threads): counts[e] = the sum of expert e's
// slices, P[e] likewise; expert e's slices are split into S = 1024 / E
// groups (slice s in group s % S), each summed by one thread, and the
// groups are added in group order; then aux = coeff * E / (k T^2) *
// sum_e counts[e] * P[e] by a fixed-order tree.
__global__ __launch_bounds__(1024) void k_aux_finalize(RouterArgs p, int64_t nslice)
{
    __shared__ float part[1024];
    __shared__ int32_t cpart[1024];
    __shared__ double red[1024];
    const int E = p.E, S = 1024 / E;  // E <= 1024 (moe_check_config)
    const int i = threadIdx.x;
    if (i < E * S) {
        const int e = i / S, sl = i % S;
        float P = 0.f;
        int32_t n = 0;
        for (int64_t b = sl; b < nslice; b += S) {
            P += p.prob_slice[b * E + e];
            n += p.cnt_slice[b * E + e];
        }
        part[i] = P;
        cpart[i] = n;
    }
    __syncthreads();
    double v = 0.0;
    if (i < E) {
        float P = 0.f;
        int32_t n = 0;
        for (int sl = 0; sl < S; ++sl) {
            P += part[i * S + sl];
            n += cpart[i * S + sl];
        }
        p.counts[i] = n;
        v = (double)n * (double)P;
    }
    red[i] = v;
    __syncthreads();
    for (int st = 512; st > 0; st >>= 1) {
        if (i < st) red[i] += red[i + st];
        __syncthreads();
    }
    if (i == 0) {
        double T = (double)p.T;
        p.aux[0] = (float)((double)p.aux_coeff * (double)p.E / ((double)p.k * T * T) * red[0]);
    }
}

hipError_t launch_router(const RouterArgs &a, hipStream_t s)
{
    hipError_t err;
    // router_blocks(T) (the 64-lane kernel's count) bounds both block counts,
    // which size the partials
    int64_t nblk;
    if (router_rows16(a.E, a.G, a.k)) {
        nblk = ceil_div(a.T, RQ_TOK_PER_BLOCK);
        const int epl = (int)ceil_div(a.E, 16);
        if (epl <= 2) k_router_select16<2><<<(unsigned)nblk, 256, 0, s>>>(a);
        else if (epl <= 4) k_router_select16<4><<<(unsigned)nblk, 256, 0, s>>>(a);
        else if (epl <= 8) k_router_select16<8><<<(unsigned)nblk, 256, 0, s>>>(a);
        else k_router_select16<16><<<(unsigned)nblk, 256, 0, s>>>(a);
    } else {
        nblk = router_blocks(a.T);
        const int epl = (int)ceil_div(a.E, 64);
        if (epl <= 1) k_router_select<1><<<(unsigned)nblk, 256, 0, s>>>(a);
        else if (epl <= 2) k_router_select<2><<<(unsigned)nblk, 256, 0, s>>>(a);
        else if (epl <= 4) k_router_select<4><<<(unsigned)nblk, 256, 0, s>>>(a);
        else if (epl <= 8) k_router_select<8><<<(unsigned)nblk, 256, 0, s>>>(a);
        else k_router_select<16><<<(unsigned)nblk, 256, 0, s>>>(a);
    }
    err = hipGetLastError();
    if (err != hipSuccess) return err;
    const int64_t nsl = ceil_div(nblk, AUX_SLICE);
    k_aux_slices<<<(unsigned)nsl, 256, 0, s>>>(a, nblk);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
    k_aux_finalize<<<1, 1024, 0, s>>>(a, nsl);
    return hipGetLastError();
}

}  // namespace moe
