// Memory-bound kernels of the expert path: the weighted combine (and the
// un-permute reduce of the backward, the same kernel with unit weights), the
// stand-alone SwiGLU forward/backward, and the router backward.
#include "common.h"

namespace moe {

// --------------------------------------------------------------- combine ----
// y[t, :] = sum_j w[t, j] * o[pos[t*k + j], :], j ascending, fp32.
// One block per token, float4 columns.  Deterministic (no atomics).
// Rows of o in fp32 or bf16 (InT = uint16_t: 8-byte loads of 4 values).
MOE_DEV f32x4_t load4_nt(const float *p) { return __builtin_nontemporal_load((const f32x4_t *)p); }
MOE_DEV f32x4_t load4_nt(const uint16_t *p)
{
    const uint64_t v = __builtin_nontemporal_load((const uint64_t *)p);
    return f32x4_t{bf2f((uint16_t)(v & 0xffffu)), bf2f((uint16_t)((v >> 16) & 0xffffu)),
                   bf2f((uint16_t)((v >> 32) & 0xffffu)), bf2f((uint16_t)(v >> 48))};
}

template <class InT>
__global__ __launch_bounds__(256) void k_combine(int64_t T, int32_t k, int32_t H, const InT *o,
                                                 const float *w, const int32_t *pos, float *y)
{
    __shared__ int32_t rows[32];
    __shared__ float wts[32];
    const int64_t t = blockIdx.x;
    if (threadIdx.x < k) {
        rows[threadIdx.x] = pos[t * k + threadIdx.x];
        wts[threadIdx.x] = w ? w[t * k + threadIdx.x] : 1.0f;
    }
    __syncthreads();
    // o is read once and y written once: non-temporal accesses keep them
    // from displacing cached data; two column chunks per thread keep twice
    // the loads in flight
    const int H4 = H / 4;
    f32x4_t *y4 = (f32x4_t *)(y + t * H);
    const int nt = blockDim.x;
    int c = threadIdx.x;
    for (; c + nt < H4; c += 2 * nt) {
        f32x4_t acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
        for (int j = 0; j < k; ++j) {
            const InT *src = o + (int64_t)rows[j] * H + 4 * c;
            const f32x4_t v0 = load4_nt(src);
            const f32x4_t v1 = load4_nt(src + 4 * nt);
            acc0 += wts[j] * v0;
            acc1 += wts[j] * v1;
        }
        __builtin_nontemporal_store(acc0, y4 + c);
        __builtin_nontemporal_store(acc1, y4 + c + nt);
    }
    for (; c < H4; c += nt) {
        f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
        for (int j = 0; j < k; ++j) acc += wts[j] * load4_nt(o + (int64_t)rows[j] * H + 4 * c);
        __builtin_nontemporal_store(acc, y4 + c);
    }
}

hipError_t launch_combine(int64_t T, int32_t k, int32_t H, const float *o, const float *w,
                          const int32_t *pos, float *y, hipStream_t s)
{
    if (T <= 0) return hipSuccess;
    k_combine<float><<<(unsigned)T, 256, 0, s>>>(T, k, H, o, w, pos, y);
    return hipGetLastError();
}

hipError_t launch_combine_bf16(int64_t T, int32_t k, int32_t H, const uint16_t *o, const float *w,
                               const int32_t *pos, float *y, hipStream_t s)
{
    if (T <= 0) return hipSuccess;
    k_combine<uint16_t><<<(unsigned)T, 256, 0, s>>>(T, k, H, o, w, pos, y);
    return hipGetLastError();
}

// ---------------------------------------------------------- row weights ----
// wrow[r] = topk_w[row_map[r]]: the routing weight of each sorted row.
__global__ __launch_bounds__(256) void k_row_weights(int64_t M, const int32_t *row_map,
                                                     const float *topk_w, float *wrow)
{
    const int64_t r = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (r < M) wrow[r] = topk_w[row_map[r]];
}

hipError_t launch_row_weights(int64_t M, const int32_t *row_map, const float *topk_w, float *wrow,
                              hipStream_t s)
{
    if (M <= 0) return hipSuccess;
    k_row_weights<<<(unsigned)ceil_div(M, 256), 256, 0, s>>>(M, row_map, topk_w, wrow);
    return hipGetLastError();
}

// ---------------------------------------------------------------- SwiGLU ----
__global__ void k_swiglu_fwd(int64_t M, int32_t I, const uint16_t *h, uint16_t *a)
{
    const int64_t n = M * I;
    for (int64_t q = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; q < n;
         q += (int64_t)gridDim.x * blockDim.x) {
        int64_t m = q / I, i = q % I;
        float g = bf2f(h[m * 2 * I + i]), u = bf2f(h[m * 2 * I + I + i]);
        a[q] = f2bf(g * sigmoidf_(g) * u);
    }
}

__global__ void k_swiglu_bwd(int64_t M, int32_t I, const uint16_t *h, const float *da,
                             uint16_t *dh)
{
    const int64_t n = M * I;
    for (int64_t q = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; q < n;
         q += (int64_t)gridDim.x * blockDim.x) {
        int64_t m = q / I, i = q % I;
        float g = bf2f(h[m * 2 * I + i]), u = bf2f(h[m * 2 * I + I + i]);
        float d = da[q], sg = sigmoidf_(g);
        dh[m * 2 * I + i] = f2bf(d * u * sg * (1.0f + g * (1.0f - sg)));
        dh[m * 2 * I + I + i] = f2bf(d * g * sg);
    }
}

hipError_t launch_swiglu(int32_t backward, int64_t M, int32_t I, const uint16_t *h,
                         const float *da, uint16_t *out, hipStream_t s)
{
    if (M <= 0) return hipSuccess;
    int64_t blocks = ceil_div(M * I, 256);
    if (blocks > 8192) blocks = 8192;
    if (backward) k_swiglu_bwd<<<(unsigned)blocks, 256, 0, s>>>(M, I, h, da, out);
    else k_swiglu_fwd<<<(unsigned)blocks, 256, 0, s>>>(M, I, h, out);
    return hipGetLastError();
}

// -------------------------------------------------------- router backward ----
// One wavefront per token.  dw_j = sum over column tiles of the dgrad row-dot
// partials of the token's j-th row; then the gradient of the routing weights
// and of the aux loss w.r.t. the router probabilities, through the softmax or
// sigmoid, to the logits.  Counts are constants; the selection has no
// gradient; the selection bias has none either.
template <int EPL>
__global__ __launch_bounds__(256) void k_router_bwd(RouterBwdArgs p)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t t = (int64_t)blockIdx.x * 4 + wave;
    if (t >= p.T) return;
    const int E = p.E, k = p.k;
    const float daux = p.d_aux ? p.d_aux[0] : 0.f;
    const float aux_scale =
        (float)((double)daux * (double)p.aux_coeff * (double)E / ((double)k * (double)p.T * (double)p.T));
    float l[EPL], sc[EPL], dp[EPL];
    bool ok[EPL];
#pragma unroll
    for (int q = 0; q < EPL; ++q) {
        int e = lane + 64 * q;
        ok[q] = e < E;
        l[q] = ok[q] ? p.logits[t * E + e] : 0.f;
        dp[q] = 0.f;
    }
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
    } else {
#pragma unroll
        for (int q = 0; q < EPL; ++q)
            sc[q] = ok[q] ? (float)(1.0 / (1.0 + exp(-(double)l[q]))) : 0.f;
    }
    // per-slot quantities on lanes j < k
    int ej = -1;
    float dwj = 0.f, wj = 0.f, pj = 0.f;
    if (lane < k) {
        ej = p.topk_idx[t * k + lane];
        wj = p.topk_w[t * k + lane];
        const float *dp_row = p.dw_part + (int64_t)p.pos[t * k + lane] * p.ncols;
        for (int c = 0; c < p.ncols; ++c) dwj += dp_row[c];
    }
    // probability (or sigmoid) of each selected expert, from its owner lane
    for (int j = 0; j < k; ++j) {
        int e = __shfl(ej, j, 64);
        float v = 0.f;
#pragma unroll
        for (int q = 0; q < EPL; ++q)
            if (lane + 64 * q == e) v = sc[q];
        v = __shfl(v, e & 63, 64);
        if (lane == j) pj = v;
    }
    const float zsel = wave_sum(lane < k ? pj : 0.f);
    const float sdw = wave_sum(lane < k ? dwj * wj : 0.f);
    float gsel = 0.f;  // d loss / d (p or s) of the selected expert
    if (lane < k) {
        if (p.score == MOE_SOFTMAX) gsel = p.renorm ? (dwj - sdw) / zsel : dwj;
        else gsel = p.scale / zsel * (dwj - sdw / p.scale);
    }
    for (int j = 0; j < k; ++j) {
        int e = __shfl(ej, j, 64);
        float gv = __shfl(gsel, j, 64);
#pragma unroll
        for (int q = 0; q < EPL; ++q)
            if (lane + 64 * q == e) dp[q] += gv;
    }
    if (p.score == MOE_SOFTMAX) {
#pragma unroll
        for (int q = 0; q < EPL; ++q)
            if (ok[q]) dp[q] += aux_scale * (float)p.counts[lane + 64 * q];
        float dot = 0.f;
#pragma unroll
        for (int q = 0; q < EPL; ++q) dot += ok[q] ? dp[q] * sc[q] : 0.f;
        dot = wave_sum(dot);
#pragma unroll
        for (int q = 0; q < EPL; ++q)
            if (ok[q]) p.dlogits[t * E + lane + 64 * q] = sc[q] * (dp[q] - dot);
    } else {
        float ssum = 0.f, ap = 0.f;
#pragma unroll
        for (int q = 0; q < EPL; ++q) {
            if (!ok[q]) continue;
            ssum += sc[q];
            ap += aux_scale * (float)p.counts[lane + 64 * q] * sc[q];
        }
        ssum = wave_sum(ssum);
        ap = wave_sum(ap) / ssum;
#pragma unroll
        for (int q = 0; q < EPL; ++q) {
            if (!ok[q]) continue;
            float ds = dp[q] + (aux_scale * (float)p.counts[lane + 64 * q] - ap) / ssum;
            p.dlogits[t * E + lane + 64 * q] = ds * sc[q] * (1.0f - sc[q]);
        }
    }
}

hipError_t launch_router_bwd(const RouterBwdArgs &a, hipStream_t s)
{
    if (a.T <= 0) return hipSuccess;
    unsigned blocks = (unsigned)ceil_div(a.T, 4);
    int epl = (int)ceil_div(a.E, 64);
    if (epl <= 1) k_router_bwd<1><<<blocks, 256, 0, s>>>(a);
    else if (epl <= 2) k_router_bwd<2><<<blocks, 256, 0, s>>>(a);
    else if (epl <= 4) k_router_bwd<4><<<blocks, 256, 0, s>>>(a);
    else if (epl <= 8) k_router_bwd<8><<<blocks, 256, 0, s>>>(a);
    else k_router_bwd<16><<<blocks, 256, 0, s>>>(a);
    return hipGetLastError();
}

}  // namespace moe
