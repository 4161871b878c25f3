// Host layer of libmoe: argument validation, workspace carving and the launch
// sequence of every C entry point declared in include/moe.h.  Nothing here
// allocates, frees or synchronises; every call only enqueues on the stream.
#include <string.h>

#include <mutex>

#include "common.h"
#include "mxfmt.h"

using namespace moe;

namespace {

constexpr size_t kAlign = 256;

size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

// Bump allocator over the caller's workspace.
struct Carver {
    char *base;
    size_t used = 0;
    explicit Carver(void *b) : base((char *)b) {}
    template <class T>
    T *take(int64_t n)
    {
        T *p = base ? (T *)(base + used) : nullptr;
        used += align_up(sizeof(T) * (size_t)(n > 0 ? n : 0));
        return p;
    }
};

// Bytes of an MX matrix [rows, K]: codes [rows, Kp] then the scale area.
int64_t mx_bytes(int64_t rows, int64_t K) { return rows * mx_kp(K) + mx_scale_bytes(rows, K); }

struct FwdWs {
    float *prob_part;
    int32_t *cnt_part;
    float *prob_slice;
    int32_t *cnt_slice;
    int32_t *chunk_hist;
    Sched sched;
    float *wrow;
    float *o;   // [M,H] fp32; the single-op weight gradients reuse it (see carve_fwd)
    void *router;  // router GEMM scratch (router_ws_bytes_fwd)
    uint8_t *xmx;  // MXFP8 forward: MX matrix of x [T, Hp]
    uint8_t *amx;  // MXFP8 forward: MX matrix of a [M, Ip]
};

struct BwdWs {
    Sched sched;
    uint16_t *dh;
    float *dw_part;
    float *dxp;
    float *wrow;
    void *router;  // router GEMM scratch (router_ws_bytes_bwd)
    uint8_t *dymx;  // MXFP8 backward: MX matrix of dy [T, H]
    uint8_t *dhmx;  // MXFP8 backward: MX matrix of dh [M, 2I]
    // the weight gradients' operands, each expert's rows transposed: bf16
    // (tA: w*dy or dh; tB: a or x), or in MX form in the same memory
    uint16_t *tA, *tB;
    uint8_t *segA, *segB;
    uint16_t *dh_lo, *tA_lo, *tB_lo;  // split intermediates only
};

// Elements of the two transposed weight-gradient operand areas: rows R times
// the 128-row chunks of all experts (at most M/128 + E).
static int64_t seg_chunks(const moe_config &c) { return c.T * c.k / 128 + c.E; }
static int64_t seg_rows_a(const moe_config &c) { return c.H > 2 * (int64_t)c.I ? c.H : 2 * (int64_t)c.I; }
static int64_t seg_rows_b(const moe_config &c) { return c.H > c.I ? c.H : c.I; }

// Each expert's rows of a sorted-row operand [M, C] (rows gathered through
// `gather` / k and scaled by `rw` when given), transposed for the weight
// gradients: bf16 into dst (uint16_t), or as MX matrices (mx).
static hipError_t prepare_segments(const moe_config &c, const Sched &sc, const int32_t *offsets,
                                   const uint16_t *src, int64_t C, const int32_t *gather,
                                   const float *rw, bool mx, void *dst, hipStream_t s,
                                   const uint16_t *src_lo = nullptr, int32_t lo_part = 0)
{
    ColQuant q = {};
    q.src_lo = src_lo;
    q.lo_part = lo_part;
    q.src = src;
    q.C = C;
    q.gather = gather;
    q.gk = c.k;
    q.rw = rw;
    q.nseg = c.E;
    q.R = 0;
    q.offsets = offsets;
    q.mt128 = sc.mt_off128;
    q.dst = (uint8_t *)dst;
    return mx ? launch_mx_quantize_cols(q, seg_chunks(c), s)
              : launch_transpose_segments(q, seg_chunks(c), (uint16_t *)dst, s);
}

// The forward workspace.  The bf16 forward and its parts (router, permute,
// the forward GEMMs, combine) use only its first `bf16_bytes`; the rest holds
// the single-op weight-gradient GEMMs' transposed operands (an extension of
// o's area, from o's start) and the MXFP8 forward's MX matrices.
FwdWs carve_fwd(const moe_config &c, void *ws, size_t *bytes, size_t *bf16_bytes = nullptr)
{
    Carver cv(ws);
    const int64_t M = c.T * c.k;
    FwdWs w;
    w.prob_part = cv.take<float>(router_blocks(c.T) * c.E);
    w.cnt_part = cv.take<int32_t>(router_blocks(c.T) * c.E);
    w.prob_slice = cv.take<float>(aux_slices(c.T) * c.E);
    w.cnt_slice = cv.take<int32_t>(aux_slices(c.T) * c.E);
    w.chunk_hist = cv.take<int32_t>(permute_chunks(M) * (c.E + 1));
    w.sched.mt_off256 = cv.take<int32_t>(c.E + 1);
    w.sched.mt_off128 = cv.take<int32_t>(c.E + 1);
    w.sched.order = cv.take<int32_t>(c.E + 1);
    w.sched.mt_a = cv.take<int32_t>(c.E + 1);
    w.sched.mt_b = cv.take<int32_t>(c.E + 1);
    w.wrow = cv.take<float>(M);
    w.router = cv.take<char>((int64_t)router_ws_bytes_fwd(c.T, c.E, c.H));
    w.o = cv.take<float>(M * c.H);   // [M,H] fp32 expert outputs
    if (bf16_bytes) *bf16_bytes = cv.used;
    // the single-op weight-gradient GEMMs put their transposed operands where
    // o starts, extended here to their size
    const int64_t t_elems = (seg_rows_a(c) + seg_rows_b(c)) * 128 * seg_chunks(c);
    if ((t_elems + 1) / 2 > M * c.H) cv.take<float>((t_elems + 1) / 2 - M * c.H);
    w.xmx = cv.take<uint8_t>(mx_bytes(c.T, c.H));
    w.amx = cv.take<uint8_t>(mx_bytes(M, c.I));
    if (bytes) *bytes = cv.used;
    return w;
}

// The forward workspace bytes an entry point needs: the bf16 forward's part,
// or all of it (the MXFP8 forward, the single-op GEMMs).
size_t fwd_need(const moe_config &c, bool full)
{
    size_t all = 0, part = 0;
    carve_fwd(c, nullptr, &all, &part);
    return full ? all : part;
}

BwdWs carve_bwd(const moe_config &c, void *ws, size_t *bytes)
{
    Carver cv(ws);
    const int64_t M = c.T * c.k;
    BwdWs w;
    w.sched.mt_off256 = cv.take<int32_t>(c.E + 1);
    w.sched.mt_off128 = cv.take<int32_t>(c.E + 1);
    w.sched.order = cv.take<int32_t>(c.E + 1);
    w.sched.mt_a = cv.take<int32_t>(c.E + 1);
    w.sched.mt_b = cv.take<int32_t>(c.E + 1);
    w.dh = cv.take<uint16_t>(M * 2 * c.I);
    w.dw_part = cv.take<float>(M * dgrad2_cols(c.I));
    w.dxp = cv.take<float>(M * c.H);
    w.wrow = cv.take<float>(M);
    w.router = cv.take<char>((int64_t)router_ws_bytes_bwd(c.T, c.E, c.H));
    w.dymx = cv.take<uint8_t>(mx_bytes(c.T, c.H));
    w.dhmx = cv.take<uint8_t>(mx_bytes(M, 2 * (int64_t)c.I));
    // per-expert transposes of the weight-gradient operands: rows R, K = the
    // expert's rows padded to 128, <= (M/128 + E) 128-row chunks in all; the
    // MX forms (132 bytes per 128 elements) fit in the bf16 ones
    w.tA = cv.take<uint16_t>(seg_rows_a(c) * 128 * seg_chunks(c));
    w.tB = cv.take<uint16_t>(seg_rows_b(c) * 128 * seg_chunks(c));
    w.segA = (uint8_t *)w.tA;
    w.segB = (uint8_t *)w.tB;
    // split intermediates: dh's remainder and the remainder halves of the
    // weight gradients' split operands
    const bool split = c.precision == MOE_PRECISION_SPLIT;
    w.dh_lo = split ? cv.take<uint16_t>(M * 2 * c.I) : nullptr;
    w.tA_lo = split ? cv.take<uint16_t>(seg_rows_a(c) * 128 * seg_chunks(c)) : nullptr;
    w.tB_lo = split ? cv.take<uint16_t>(seg_rows_b(c) * 128 * seg_chunks(c)) : nullptr;
    if (bytes) *bytes = cv.used;
    return w;
}

// Stage event registry (see moe_set_stage_events).
hipEvent_t g_stage_start[MOE_STAGE_COUNT];
hipEvent_t g_stage_stop[MOE_STAGE_COUNT];

// Records the stage's registered events around a scope of launches.
struct StageMark {
    int id;
    hipStream_t s;
    StageMark(int stage, hipStream_t stream) : id(stage), s(stream)
    {
        if (g_stage_start[id]) (void)hipEventRecord(g_stage_start[id], s);
    }
    ~StageMark()
    {
        if (g_stage_stop[id]) (void)hipEventRecord(g_stage_stop[id], s);
    }
};

hipError_t run_gemm(int32_t op, const GemmArgs &g, hipStream_t s)
{
    StageMark mark(op, s);
    if (!g.dw_acc && (op == MOE_GEMM_DOWN_WGRAD || op == MOE_GEMM_UP_WGRAD)) {
        // experts without rows get exact zeros; the GEMM only visits the others
        const bool up = op == MOE_GEMM_UP_WGRAD;
        hipError_t e = launch_zero_empty(g.E, (int64_t)2 * g.I * g.H / (up ? 1 : 2), g.counts,
                                         up ? g.dW1 : g.dW2, g.dw_bf16, s);
        if (e != hipSuccess) return e;
    }
    return launch_grouped_gemm(op, g, s);
}

#define MOE_TRY(expr)                                  \
    do {                                               \
        hipError_t e_ = (expr);                        \
        if (e_ != hipSuccess) return MOE_EHIP;         \
    } while (0)

#define MOE_CHECK(expr)                                \
    do {                                               \
        moe_status s_ = (expr);                        \
        if (s_ != MOE_OK) return s_;                   \
    } while (0)

moe_status check_ptrs(std::initializer_list<const void *> ps)
{
    for (const void *p : ps)
        if (!p || !aligned16(p)) return MOE_EINVAL;
    return MOE_OK;
}

moe_status check_opt_ptr(const void *p) { return (!p || aligned16(p)) ? MOE_OK : MOE_EINVAL; }

GemmArgs gemm_args(const moe_config &c, const moe_gemm_args &a, const Sched &sc)
{
    GemmArgs g;
    memset(&g, 0, sizeof g);
    g.T = c.T;
    g.M = c.T * c.k;
    g.E = c.E;
    g.k = c.k;
    g.H = c.H;
    g.I = c.I;
    g.counts = a.counts;
    g.offsets = a.offsets;
    g.row_map = a.row_map;
    g.topk_w = a.topk_w;
    g.x = a.x;
    g.dy = a.dy;
    g.w1 = a.w1;
    g.w2 = a.w2;
    g.h = a.h;
    g.a = a.a;
    g.o = a.o;
    g.dh = a.dh;
    g.dw_part = a.dw_part;
    g.dxp = a.dxp;
    g.dW1 = a.dW1;
    g.dW2 = a.dW2;
    g.dw_bf16 = a.dw_dtype == MOE_BF16;
    g.dw_acc = a.dw_accumulate != 0;
    g.sched = sc;
    return g;
}

}  // namespace

extern "C" {

const char *moe_status_string(moe_status s)
{
    switch (s) {
    case MOE_OK: return "ok";
    case MOE_EINVAL: return "invalid argument (null or misaligned pointer, bad enum or size)";
    case MOE_EUNSUPPORTED: return "unsupported shape or option";
    case MOE_EWORKSPACE: return "workspace too small";
    case MOE_EHIP: return "HIP kernel launch failed";
    }
    return "unknown status";
}

const char *moe_version(void) { return "libmoe 0.1 gfx950"; }

moe_status moe_set_stage_events(int32_t stage, hipEvent_t start, hipEvent_t stop)
{
    if (stage < 0 || stage >= MOE_STAGE_COUNT) return MOE_EINVAL;
    if ((start == nullptr) != (stop == nullptr)) return MOE_EINVAL;
    g_stage_start[stage] = start;
    g_stage_stop[stage] = stop;
    return MOE_OK;
}

moe_status moe_check_config(const moe_config *cfg)
{
    if (!cfg) return MOE_EINVAL;
    const moe_config &c = *cfg;
    if (c.T < 0 || c.H <= 0 || c.I <= 0 || c.E <= 0 || c.k <= 0) return MOE_EINVAL;
    if (c.score != MOE_SOFTMAX && c.score != MOE_SIGMOID) return MOE_EINVAL;
    if (c.route_mode != MOE_ROUTE_LEARNED && c.route_mode != MOE_ROUTE_EVEN) return MOE_EINVAL;
    if (c.precision != MOE_PRECISION_BF16 && c.precision != MOE_PRECISION_SPLIT) return MOE_EINVAL;
    if (c.k > c.E || c.k > 32 || c.E > 1024) return MOE_EUNSUPPORTED;
    if (c.n_groups < 1 || c.n_groups > 64 || c.E % c.n_groups != 0) return MOE_EUNSUPPORTED;
    if (c.topk_groups < 1 || c.topk_groups > c.n_groups) return MOE_EUNSUPPORTED;
    if (c.n_groups > 1 && (int64_t)c.k > (int64_t)c.topk_groups * (c.E / c.n_groups))
        return MOE_EUNSUPPORTED;
    if (c.H % 64 != 0 || c.I % 64 != 0) return MOE_EUNSUPPORTED;
    const int64_t M = c.T * (int64_t)c.k;
    const int64_t widest = c.H > 2 * c.I ? c.H : 2 * (int64_t)c.I;
    if (M >= (1ll << 31) || M * widest >= (1ll << 31)) return MOE_EUNSUPPORTED;
    // an expert's transposed weight-gradient operands: widest x (rows + pad)
    if (widest * (c.T + 128) >= (1ll << 31)) return MOE_EUNSUPPORTED;
    if ((int64_t)2 * c.I * c.H >= (1ll << 31)) return MOE_EUNSUPPORTED;
    return MOE_OK;
}

moe_status moe_workspace_size(const moe_config *cfg, size_t *fwd_bytes, size_t *bwd_bytes)
{
    MOE_CHECK(moe_check_config(cfg));
    size_t f = 0, b = 0;
    carve_fwd(*cfg, nullptr, &f);
    carve_bwd(*cfg, nullptr, &b);
    if (fwd_bytes) *fwd_bytes = f;
    if (bwd_bytes) *bwd_bytes = b;
    return MOE_OK;
}

int32_t moe_dw_part_cols(const moe_config *cfg) { return cfg ? dgrad2_cols(cfg->I) : 0; }

moe_status moe_router(const moe_config *cfg, const uint16_t *x, const float *Wr,
                      const float *bias, float *logits, float *sel_scores,
                      int32_t *topk_idx, float *topk_w, int32_t *counts, float *aux,
                      void *ws, size_t ws_bytes, hipStream_t stream)
{
    MOE_CHECK(moe_check_config(cfg));
    const moe_config &c = *cfg;
    MOE_CHECK(check_ptrs({logits, topk_idx, topk_w, counts, aux}));
    MOE_CHECK(check_opt_ptr(bias));
    MOE_CHECK(check_opt_ptr(sel_scores));
    if (Wr) MOE_CHECK(check_ptrs({x, Wr}));
    const size_t need = fwd_need(c, false);
    FwdWs w = carve_fwd(c, ws, nullptr);
    if (ws_bytes < need || (need && !ws)) return MOE_EWORKSPACE;
    if (c.T == 0) {
        MOE_TRY(launch_fill_i32(counts, c.E, 0, stream));
        MOE_TRY(launch_fill_f32(aux, 1, 0.f, stream));
        return MOE_OK;
    }
    if (Wr) {
        StageMark mark(MOE_STAGE_ROUTER_PROJ, stream);
        MOE_TRY(launch_router_logits(c.T, c.E, c.H, x, Wr, logits, w.router, stream));
    }
    RouterArgs ra;
    ra.T = c.T;
    ra.E = c.E;
    ra.k = c.k;
    ra.G = c.n_groups;
    ra.kg = c.topk_groups;
    ra.score = c.score;
    ra.renorm = c.renorm;
    ra.scale = c.scale;
    ra.aux_coeff = c.aux_coeff;
    ra.even = c.route_mode == MOE_ROUTE_EVEN;
    ra.logits = logits;
    ra.bias = bias;
    ra.sel = sel_scores;
    ra.topk_w = topk_w;
    ra.topk_idx = topk_idx;
    ra.counts = counts;
    ra.aux = aux;
    ra.prob_part = w.prob_part;
    ra.cnt_part = w.cnt_part;
    ra.prob_slice = w.prob_slice;
    ra.cnt_slice = w.cnt_slice;
    StageMark mark(MOE_STAGE_ROUTER, stream);
    MOE_TRY(launch_router(ra, stream));
    return MOE_OK;
}

moe_status moe_permute(const moe_config *cfg, const int32_t *topk_idx, int32_t *counts,
                       int32_t *offsets, int32_t *row_map, int32_t *pos, void *ws,
                       size_t ws_bytes, hipStream_t stream)
{
    MOE_CHECK(moe_check_config(cfg));
    const moe_config &c = *cfg;
    MOE_CHECK(check_ptrs({counts, offsets}));
    if (c.T > 0) MOE_CHECK(check_ptrs({topk_idx, row_map, pos}));
    const size_t need = fwd_need(c, false);
    FwdWs w = carve_fwd(c, ws, nullptr);
    if (ws_bytes < need || (need && !ws)) return MOE_EWORKSPACE;
    MOE_TRY(launch_permute(c.T * c.k, c.E, topk_idx, counts, offsets, row_map, pos, w.chunk_hist,
                           stream));
    return MOE_OK;
}

moe_status moe_permute_checked(const moe_config *cfg, const int32_t *topk_idx, int32_t *counts,
                               int32_t *offsets, int32_t *row_map, int32_t *pos, int32_t *n_bad,
                               void *ws, size_t ws_bytes, hipStream_t stream)
{
    MOE_CHECK(moe_check_config(cfg));
    const moe_config &c = *cfg;
    MOE_CHECK(check_ptrs({counts, offsets, n_bad}));
    if (c.T > 0) MOE_CHECK(check_ptrs({topk_idx, row_map, pos}));
    const size_t need = fwd_need(c, false);
    FwdWs w = carve_fwd(c, ws, nullptr);
    if (ws_bytes < need || (need && !ws)) return MOE_EWORKSPACE;
    MOE_TRY(launch_permute_checked(c.T * c.k, c.E, topk_idx, counts, offsets, row_map, pos,
                                   w.chunk_hist, n_bad, stream));
    return MOE_OK;
}

moe_status moe_saved_sizes(const moe_config *cfg, size_t sizes[MOE_SAVED_N])
{
    MOE_CHECK(moe_check_config(cfg));
    if (!sizes) return MOE_EINVAL;
    const moe_config &c = *cfg;
    const size_t T = (size_t)c.T, E = (size_t)c.E, k = (size_t)c.k, M = T * k;
    const size_t I = (size_t)c.I;
    sizes[0] = T * E * sizeof(float);        // logits
    sizes[1] = M * sizeof(int32_t);          // topk_idx
    sizes[2] = M * sizeof(float);            // topk_w
    sizes[3] = E * sizeof(int32_t);          // counts
    sizes[4] = (E + 1) * sizeof(int32_t);    // offsets
    sizes[5] = M * sizeof(int32_t);          // row_map
    sizes[6] = M * sizeof(int32_t);          // pos
    sizes[7] = M * 2 * I * sizeof(uint16_t); // h
    sizes[8] = M * I * sizeof(uint16_t);     // a
    const bool split = c.precision == MOE_PRECISION_SPLIT;
    sizes[9] = split ? sizes[7] : 0;         // h_lo
    sizes[10] = split ? sizes[8] : 0;        // a_lo
    return MOE_OK;
}

moe_status moe_grouped_gemm(int32_t op, const moe_config *cfg, const moe_gemm_args *args,
                            void *ws, size_t ws_bytes, hipStream_t stream)
{
    MOE_CHECK(moe_check_config(cfg));
    if (!args) return MOE_EINVAL;
    const moe_config &c = *cfg;
    const moe_gemm_args &a = *args;
    if (c.precision != MOE_PRECISION_BF16) return MOE_EUNSUPPORTED;
    size_t need = 0;
    FwdWs w = carve_fwd(c, ws, &need);
    if (ws_bytes < need || (need && !ws)) return MOE_EWORKSPACE;
    MOE_CHECK(check_ptrs({a.counts, a.offsets}));
    switch (op) {
    case MOE_GEMM_UP_SWIGLU:
        MOE_CHECK(check_ptrs({a.x, a.w1, a.row_map, a.a}));
        MOE_CHECK(check_opt_ptr(a.h));
        break;
    case MOE_GEMM_DOWN:
        MOE_CHECK(check_ptrs({a.a, a.w2, a.o}));
        break;
    case MOE_GEMM_DOWN_DGRAD:
        MOE_CHECK(check_ptrs({a.dy, a.w2, a.row_map, a.topk_w, a.h, a.a, a.dh, a.dw_part}));
        break;
    case MOE_GEMM_UP_DGRAD:
        MOE_CHECK(check_ptrs({a.dh, a.w1, a.dxp}));
        break;
    case MOE_GEMM_DOWN_WGRAD:
        MOE_CHECK(check_ptrs({a.dy, a.a, a.row_map, a.topk_w, a.dW2}));
        break;
    case MOE_GEMM_UP_WGRAD:
        MOE_CHECK(check_ptrs({a.dh, a.x, a.row_map, a.dW1}));
        break;
    default:
        return MOE_EINVAL;
    }
    if (a.dw_dtype != MOE_F32 && a.dw_dtype != MOE_BF16) return MOE_EINVAL;
    const bool wgrad = op == MOE_GEMM_DOWN_WGRAD || op == MOE_GEMM_UP_WGRAD;
    if (c.T == 0 && !wgrad) return MOE_OK;
    MOE_TRY(launch_schedule(c.E, a.counts, w.sched, stream));
    GemmArgs g = gemm_args(c, a, w.sched);
    const int64_t M = c.T * c.k;
    // the routing weight per sorted row (dgrad2, and w*dy for dW2)
    if (op == MOE_GEMM_DOWN_DGRAD || op == MOE_GEMM_DOWN_WGRAD)
        MOE_TRY(launch_row_weights(M, a.row_map, a.topk_w, w.wrow, stream));
    // the weight gradients' operands, transposed per expert (in the area of o)
    uint16_t *tA = (uint16_t *)w.o, *tB = tA + seg_rows_a(c) * 128 * seg_chunks(c);
    if (op == MOE_GEMM_DOWN_WGRAD && c.T > 0) {
        MOE_TRY(prepare_segments(c, w.sched, a.offsets, a.dy, c.H, a.row_map, w.wrow, false, tA,
                                 stream));
        MOE_TRY(prepare_segments(c, w.sched, a.offsets, a.a, c.I, nullptr, nullptr, false, tB,
                                 stream));
    }
    if (op == MOE_GEMM_UP_WGRAD && c.T > 0) {
        MOE_TRY(prepare_segments(c, w.sched, a.offsets, a.dh, 2 * (int64_t)c.I, nullptr, nullptr,
                                 false, tA, stream));
        MOE_TRY(prepare_segments(c, w.sched, a.offsets, a.x, c.H, a.row_map, nullptr, false, tB,
                                 stream));
    }
    g.wrow = w.wrow;
    g.tA = tA;
    g.tB = tB;
    MOE_TRY(run_gemm(op, g, stream));
    return MOE_OK;
}

moe_status moe_swiglu(int32_t backward, int64_t M, int32_t I, const uint16_t *h, const float *da,
                      uint16_t *out, hipStream_t stream)
{
    if (M < 0 || I <= 0) return MOE_EINVAL;
    if (M == 0) return MOE_OK;
    MOE_CHECK(check_ptrs({h, out}));
    if (backward) MOE_CHECK(check_ptrs({da}));
    MOE_TRY(launch_swiglu(backward, M, I, h, da, out, stream));
    return MOE_OK;
}

moe_status moe_combine(const moe_config *cfg, const float *o, const float *topk_w,
                       const int32_t *pos, float *y, hipStream_t stream)
{
    MOE_CHECK(moe_check_config(cfg));
    const moe_config &c = *cfg;
    if (c.T == 0) return MOE_OK;
    MOE_CHECK(check_ptrs({o, pos, y}));
    MOE_CHECK(check_opt_ptr(topk_w));
    StageMark mark(MOE_STAGE_COMBINE, stream);
    MOE_TRY(launch_combine(c.T, c.k, c.H, o, topk_w, pos, y, stream));
    return MOE_OK;
}

static moe_status check_saved(const moe_saved *s, const moe_config &c)
{
    if (!s) return MOE_EINVAL;
    MOE_CHECK(check_ptrs({s->logits, s->topk_idx, s->topk_w, s->counts, s->offsets, s->row_map,
                          s->pos, s->h, s->a}));
    if (c.precision == MOE_PRECISION_SPLIT) MOE_CHECK(check_ptrs({s->h_lo, s->a_lo}));
    return MOE_OK;
}

// The backward reads only counts and offsets of a forward over no tokens (the
// other saved tensors are empty and may be NULL).
static moe_status check_saved_bwd(const moe_saved *s, const moe_config &c)
{
    if (!s) return MOE_EINVAL;
    if (c.T == 0) return check_ptrs({s->counts, s->offsets});
    return check_saved(s, c);
}

static moe_gemm_args saved_gemm_args(const moe_saved *saved)
{
    moe_gemm_args a;
    memset(&a, 0, sizeof a);
    a.counts = saved->counts;
    a.offsets = saved->offsets;
    a.row_map = saved->row_map;
    a.topk_w = saved->topk_w;
    a.h = saved->h;
    a.a = saved->a;
    return a;
}

// The split intermediates of a config in MOE_PRECISION_SPLIT (saved h_lo,
// a_lo; the backward's dh_lo and operand remainders).
static void set_split(GemmArgs &g, const moe_config &c, const moe_saved *saved,
                      const BwdWs *bw)
{
    g.split = c.precision == MOE_PRECISION_SPLIT;
    if (!g.split) return;
    g.h_lo = saved->h_lo;
    g.a_lo = saved->a_lo;
    if (bw) {
        g.dh_lo = bw->dh_lo;
        g.tA_lo = bw->tA_lo;
        g.tB_lo = bw->tB_lo;
    }
}

// ----------------------------------------------------------- two stages ----
// The MegaMoE design section splits the layer into two stages that each own
// one weight: stage 1 (router, dispatch, GEMM1 + SwiGLU; w1) and stage 2
// (GEMM2 + combine; w2).  The backward runs stage 2 first (dW2), then stage 1
// (dW1, router).  moe_forward / moe_backward are these stages back to back.

// The forward stages in bf16 (w1 / w2) or MXFP8 (w1_mx / w2_mx: MX matrices
// of w1 as [E*2I, H] and w2 as [E*H, I]); exactly one of each pair is given.
static void set_mx(GemmArgs &g, const moe_config &c, const FwdWs &w)
{
    const int64_t M = c.T * c.k;
    g.Hp = mx_kp(c.H);
    g.Ip = mx_kp(c.I);
    g.xq = w.xmx;
    g.xs = w.xmx + c.T * g.Hp;
    g.aq = w.amx;
    g.as_ = w.amx + M * g.Ip;
}

static moe_status stage1_fwd(const moe_config *cfg, const uint16_t *x, const float *Wr,
                             const float *bias, const uint16_t *w1, const uint8_t *w1_mx,
                             float *aux, const moe_saved *saved, void *ws, size_t ws_bytes,
                             hipStream_t stream)
{
    MOE_CHECK(moe_check_config(cfg));
    const moe_config &c = *cfg;
    if (w1_mx && c.precision != MOE_PRECISION_BF16) return MOE_EUNSUPPORTED;
    if (!saved || !aux) return MOE_EINVAL;
    const size_t need = fwd_need(c, w1_mx != nullptr);
    FwdWs w = carve_fwd(c, ws, nullptr);
    if (ws_bytes < need || (need && !ws)) return MOE_EWORKSPACE;
    if (c.T == 0) {
        MOE_CHECK(check_ptrs({saved->counts, saved->offsets, aux}));
        MOE_TRY(launch_fill_i32(saved->counts, c.E, 0, stream));
        MOE_TRY(launch_fill_i32(saved->offsets, c.E + 1, 0, stream));
        MOE_TRY(launch_fill_f32(aux, 1, 0.f, stream));
        return MOE_OK;
    }
    MOE_CHECK(check_saved(saved, c));
    MOE_CHECK(check_ptrs({x, w1_mx ? (const void *)w1_mx : (const void *)w1}));
    MOE_CHECK(moe_router(cfg, x, Wr, bias, saved->logits, nullptr, saved->topk_idx,
                         saved->topk_w, saved->counts, aux, ws, ws_bytes, stream));
    {
        StageMark mark(MOE_STAGE_PERMUTE, stream);
        MOE_TRY(launch_permute(c.T * c.k, c.E, saved->topk_idx, saved->counts, saved->offsets,
                               saved->row_map, saved->pos, w.chunk_hist, stream));
        MOE_TRY(launch_schedule(c.E, saved->counts, w.sched, stream));
    }
    moe_gemm_args a = saved_gemm_args(saved);
    a.x = x;
    a.w1 = w1;
    GemmArgs g = gemm_args(c, a, w.sched);
    set_split(g, c, saved, nullptr);
    if (!w1_mx) {
        MOE_TRY(run_gemm(MOE_GEMM_UP_SWIGLU, g, stream));
        return MOE_OK;
    }
    set_mx(g, c, w);
    g.w1q = w1_mx;
    g.w1s = w1_mx + (int64_t)c.E * 2 * c.I * g.Hp;
    {
        StageMark mark(MOE_STAGE_MX_QUANT, stream);
        MOE_TRY(launch_mx_quantize(x, c.T, c.H, w.xmx, stream));
    }
    StageMark mark(MOE_GEMM_UP_SWIGLU, stream);
    MOE_TRY(launch_mx_gemm(MOE_GEMM_UP_SWIGLU, g, stream));
    return MOE_OK;
}

// sched_ready: the schedule in `ws` is already this call's (the one-call
// forward runs stage 1, which computes it, on the same workspace just before)
static moe_status stage2_fwd(const moe_config *cfg, const uint16_t *w2, const uint8_t *w2_mx,
                             const moe_saved *saved, float *y, void *ws, size_t ws_bytes,
                             hipStream_t stream, bool sched_ready = false)
{
    MOE_CHECK(moe_check_config(cfg));
    const moe_config &c = *cfg;
    if (w2_mx && c.precision != MOE_PRECISION_BF16) return MOE_EUNSUPPORTED;
    if (!saved) return MOE_EINVAL;
    const size_t need = fwd_need(c, w2_mx != nullptr);
    FwdWs w = carve_fwd(c, ws, nullptr);
    if (ws_bytes < need || (need && !ws)) return MOE_EWORKSPACE;
    if (c.T == 0) return MOE_OK;
    MOE_CHECK(check_saved(saved, c));
    MOE_CHECK(check_ptrs({w2_mx ? (const void *)w2_mx : (const void *)w2, y}));
    if (!sched_ready) MOE_TRY(launch_schedule(c.E, saved->counts, w.sched, stream));
    moe_gemm_args a = saved_gemm_args(saved);
    a.w2 = w2;
    a.o = w.o;
    GemmArgs g = gemm_args(c, a, w.sched);
    set_split(g, c, saved, nullptr);
    // with bf16 intermediates (and on the MXFP8 path, which has no other
    // form) the expert outputs between GEMM2 and the combine are bf16 too
    // (the combine sums them in fp32); split keeps fp32
    const bool o16 = c.precision == MOE_PRECISION_BF16;
    if (o16) g.o_bf16 = (uint16_t *)w.o;
    if (!w2_mx) {
        MOE_TRY(run_gemm(MOE_GEMM_DOWN, g, stream));
    } else {
        set_mx(g, c, w);
        g.w2q = w2_mx;
        g.w2s = w2_mx + (int64_t)c.E * c.H * g.Ip;
        StageMark mark(MOE_GEMM_DOWN, stream);
        MOE_TRY(launch_mx_gemm(MOE_GEMM_DOWN, g, stream));
    }
    StageMark mark(MOE_STAGE_COMBINE, stream);
    if (o16)
        MOE_TRY(launch_combine_bf16(c.T, c.k, c.H, (const uint16_t *)w.o, saved->topk_w, saved->pos,
                                    y, stream));
    else
        MOE_TRY(launch_combine(c.T, c.k, c.H, w.o, saved->topk_w, saved->pos, y, stream));
    return MOE_OK;
}

moe_status moe_stage1_forward(const moe_config *cfg, const uint16_t *x, const float *Wr,
                              const float *bias, const uint16_t *w1, float *aux,
                              const moe_saved *saved, void *ws, size_t ws_bytes,
                              hipStream_t stream)
{
    return stage1_fwd(cfg, x, Wr, bias, w1, nullptr, aux, saved, ws, ws_bytes, stream);
}

moe_status moe_stage2_forward(const moe_config *cfg, const uint16_t *w2, const moe_saved *saved,
                              float *y, void *ws, size_t ws_bytes, hipStream_t stream)
{
    return stage2_fwd(cfg, w2, nullptr, saved, y, ws, ws_bytes, stream);
}

moe_status moe_forward(const moe_config *cfg, const uint16_t *x, const float *Wr,
                       const float *bias, const uint16_t *w1, const uint16_t *w2, float *y,
                       float *aux, const moe_saved *saved, void *ws, size_t ws_bytes,
                       hipStream_t stream)
{
    MOE_CHECK(moe_check_config(cfg));
    if (cfg->T > 0) MOE_CHECK(check_ptrs({w2, y}));
    MOE_CHECK(moe_stage1_forward(cfg, x, Wr, bias, w1, aux, saved, ws, ws_bytes, stream));
    return stage2_fwd(cfg, w2, nullptr, saved, y, ws, ws_bytes, stream, true);
}

// ---------------------------------------------------------------- MXFP8 ----

moe_status moe_mx_size(int64_t rows, int64_t K, size_t *bytes)
{
    if (!bytes || rows < 0 || K <= 0 || K % 32 != 0) return MOE_EINVAL;
    *bytes = (size_t)mx_bytes(rows, K);
    return MOE_OK;
}

moe_status moe_mx_quantize(const uint16_t *src, int64_t rows, int64_t K, void *dst,
                           size_t dst_bytes, hipStream_t stream)
{
    size_t need = 0;
    MOE_CHECK(moe_mx_size(rows, K, &need));
    if (rows == 0) return MOE_OK;
    MOE_CHECK(check_ptrs({src, dst}));
    if (dst_bytes < need) return MOE_EINVAL;
    StageMark mark(MOE_STAGE_MX_QUANT, stream);
    MOE_TRY(launch_mx_quantize(src, rows, K, (uint8_t *)dst, stream));
    return MOE_OK;
}

moe_status moe_grouped_gemm_mx(int32_t op, const moe_config *cfg, const moe_gemm_mx_args *args,
                               void *ws, size_t ws_bytes, hipStream_t stream)
{
    MOE_CHECK(moe_check_config(cfg));
    if (!args) return MOE_EINVAL;
    const moe_config &c = *cfg;
    const moe_gemm_mx_args &a = *args;
    if (c.precision != MOE_PRECISION_BF16) return MOE_EUNSUPPORTED;
    size_t need = 0;
    FwdWs w = carve_fwd(c, ws, &need);
    if (ws_bytes < need || (need && !ws)) return MOE_EWORKSPACE;
    MOE_CHECK(check_ptrs({a.counts, a.offsets}));
    if (op == MOE_GEMM_UP_SWIGLU) {
        MOE_CHECK(check_ptrs({a.x_mx, a.w1_mx, a.a_mx, a.row_map, a.a}));
        MOE_CHECK(check_opt_ptr(a.h));
    } else if (op == MOE_GEMM_DOWN) {
        MOE_CHECK(check_ptrs({a.a_mx, a.w2_mx, a.o}));
    } else {
        return MOE_EINVAL;
    }
    if (c.T == 0) return MOE_OK;
    MOE_TRY(launch_schedule(c.E, a.counts, w.sched, stream));
    moe_gemm_args b;
    memset(&b, 0, sizeof b);
    b.counts = a.counts;
    b.offsets = a.offsets;
    b.row_map = a.row_map;
    b.h = a.h;
    b.a = a.a;
    b.o = a.o;
    GemmArgs g = gemm_args(c, b, w.sched);
    const int64_t M = c.T * c.k;
    g.Hp = mx_kp(c.H);
    g.Ip = mx_kp(c.I);
    g.xq = (const uint8_t *)a.x_mx;
    g.xs = g.xq ? g.xq + c.T * g.Hp : nullptr;
    g.w1q = (const uint8_t *)a.w1_mx;
    g.w1s = g.w1q ? g.w1q + (int64_t)c.E * 2 * c.I * g.Hp : nullptr;
    g.w2q = (const uint8_t *)a.w2_mx;
    g.w2s = g.w2q ? g.w2q + (int64_t)c.E * c.H * g.Ip : nullptr;
    g.aq = (uint8_t *)a.a_mx;
    g.as_ = g.aq + M * g.Ip;
    StageMark mark(op, stream);
    MOE_TRY(launch_mx_gemm(op, g, stream));
    return MOE_OK;
}

moe_status moe_stage1_forward_mx(const moe_config *cfg, const uint16_t *x, const float *Wr,
                                 const float *bias, const void *w1_mx, float *aux,
                                 const moe_saved *saved, void *ws, size_t ws_bytes,
                                 hipStream_t stream)
{
    if (!w1_mx) return MOE_EINVAL;
    return stage1_fwd(cfg, x, Wr, bias, nullptr, (const uint8_t *)w1_mx, aux, saved, ws, ws_bytes,
                      stream);
}

moe_status moe_stage2_forward_mx(const moe_config *cfg, const void *w2_mx, const moe_saved *saved,
                                 float *y, void *ws, size_t ws_bytes, hipStream_t stream)
{
    if (!w2_mx) return MOE_EINVAL;
    return stage2_fwd(cfg, nullptr, (const uint8_t *)w2_mx, saved, y, ws, ws_bytes, stream);
}

moe_status moe_forward_mx(const moe_config *cfg, const uint16_t *x, const float *Wr,
                          const float *bias, const void *w1_mx, const void *w2_mx, float *y,
                          float *aux, const moe_saved *saved, void *ws, size_t ws_bytes,
                          hipStream_t stream)
{
    MOE_CHECK(moe_check_config(cfg));
    if (cfg->T > 0) MOE_CHECK(check_ptrs({w2_mx, y}));
    MOE_CHECK(moe_stage1_forward_mx(cfg, x, Wr, bias, w1_mx, aux, saved, ws, ws_bytes, stream));
    return stage2_fwd(cfg, nullptr, (const uint8_t *)w2_mx, saved, y, ws, ws_bytes, stream, true);
}

static moe_status stage2_bwd(const moe_config *cfg, const moe_saved *saved, const uint16_t *w2,
                             const uint8_t *w2t_mx, const uint16_t *dy, void *dW2,
                             int32_t dw_dtype, int32_t dw_accumulate, void *ws, size_t ws_bytes,
                             hipStream_t stream);
// sched_ready: the schedule in `ws` is already this call's (the one-call
// backward runs stage 2, which computes it, on the same workspace just before)
static moe_status stage1_bwd(const moe_config *cfg, const moe_saved *saved, const uint16_t *x,
                             const float *Wr, const uint16_t *w1, const uint8_t *w1t_mx,
                             const float *d_aux, float *dx, float *dlogits, float *dWr, void *dW1,
                             int32_t dw_dtype, int32_t dw_accumulate, void *ws, size_t ws_bytes,
                             hipStream_t stream, bool sched_ready = false);

moe_status moe_mx_quantize_t(const uint16_t *src, int64_t batches, int64_t R, int64_t C, void *dst,
                             size_t dst_bytes, hipStream_t stream)
{
    if (batches < 0 || C <= 0 || C % 64 != 0) return MOE_EINVAL;
    size_t need = 0;
    MOE_CHECK(moe_mx_size(batches * C, R, &need));
    if (batches == 0) return MOE_OK;
    MOE_CHECK(check_ptrs({src, dst}));
    if (dst_bytes < need) return MOE_EINVAL;
    ColQuant q = {};
    q.src = src;
    q.C = C;
    q.gather = nullptr;
    q.gk = 1;
    q.rw = nullptr;
    q.nseg = (int32_t)batches;
    q.R = R;
    q.offsets = nullptr;
    q.mt128 = nullptr;
    q.dst = (uint8_t *)dst;
    StageMark mark(MOE_STAGE_MX_QUANT, stream);
    MOE_TRY(launch_mx_quantize_cols(q, batches * (mx_kp(R) / MX_GROUP), stream));
    return MOE_OK;
}

moe_status moe_mx_quantize_both(const uint16_t *src, int64_t batches, int64_t R, int64_t C,
                                void *dst, size_t dst_bytes, void *dst_t, size_t dst_t_bytes,
                                hipStream_t stream)
{
    if (batches < 0 || R <= 0 || C <= 0 || R % 32 != 0 || C % 32 != 0) return MOE_EINVAL;
    size_t need_f = 0, need_t = 0;
    MOE_CHECK(moe_mx_size(batches * R, C, &need_f));
    MOE_CHECK(moe_mx_size(batches * C, R, &need_t));
    if (batches == 0) return MOE_OK;
    MOE_CHECK(check_ptrs({src, dst, dst_t}));
    if (dst_bytes < need_f || dst_t_bytes < need_t) return MOE_EINVAL;
    StageMark mark(MOE_STAGE_MX_QUANT, stream);
    MOE_TRY(launch_mx_quantize_both(src, batches, R, C, (uint8_t *)dst, (uint8_t *)dst_t, stream));
    return MOE_OK;
}

moe_status moe_stage2_backward_mx(const moe_config *cfg, const moe_saved *saved,
                                  const void *w2t_mx, const uint16_t *dy, void *dW2,
                                  int32_t dw_dtype, int32_t dw_accumulate, void *ws,
                                  size_t ws_bytes, hipStream_t stream)
{
    if (!w2t_mx) return MOE_EINVAL;
    return stage2_bwd(cfg, saved, nullptr, (const uint8_t *)w2t_mx, dy, dW2, dw_dtype,
                      dw_accumulate, ws, ws_bytes, stream);
}

moe_status moe_stage1_backward_mx(const moe_config *cfg, const moe_saved *saved,
                                  const uint16_t *x, const float *Wr, const void *w1t_mx,
                                  const float *d_aux, float *dx, float *dlogits, float *dWr,
                                  void *dW1, int32_t dw_dtype, int32_t dw_accumulate, void *ws,
                                  size_t ws_bytes, hipStream_t stream)
{
    if (!w1t_mx) return MOE_EINVAL;
    return stage1_bwd(cfg, saved, x, Wr, nullptr, (const uint8_t *)w1t_mx, d_aux, dx, dlogits,
                      dWr, dW1, dw_dtype, dw_accumulate, ws, ws_bytes, stream);
}

moe_status moe_backward_mx(const moe_config *cfg, const moe_saved *saved, const uint16_t *x,
                           const float *Wr, const void *w1t_mx, const void *w2t_mx,
                           const uint16_t *dy, const float *d_aux, float *dx, float *dlogits,
                           float *dWr, void *dW1, void *dW2, int32_t dw_dtype,
                           int32_t dw_accumulate, void *ws, size_t ws_bytes, hipStream_t stream)
{
    MOE_CHECK(moe_check_config(cfg));
    // everything stage 1 validates, checked before stage 2 launches anything
    MOE_CHECK(check_ptrs({w1t_mx, dW1}));
    if (cfg->T > 0) MOE_CHECK(check_ptrs({x, dx, dlogits}));
    MOE_CHECK(check_opt_ptr(Wr));
    MOE_CHECK(check_opt_ptr(dWr));
    MOE_CHECK(check_opt_ptr(d_aux));
    MOE_CHECK(moe_stage2_backward_mx(cfg, saved, w2t_mx, dy, dW2, dw_dtype, dw_accumulate, ws,
                                     ws_bytes, stream));
    return stage1_bwd(cfg, saved, x, Wr, nullptr, (const uint8_t *)w1t_mx, d_aux, dx, dlogits,
                      dWr, dW1, dw_dtype, dw_accumulate, ws, ws_bytes, stream, true);
}

// The backward stages in bf16 (w2 / w1) or MXFP8 (w2t_mx / w1t_mx: MX
// matrices of w2[e]^T as [E*I, H] and w1[e]^T as [E*H, 2I]).
static void set_mx_bwd(GemmArgs &g, const moe_config &c, const BwdWs &w)
{
    const int64_t M = c.T * c.k;
    g.Hp = mx_kp(c.H);
    g.Ip = mx_kp(c.I);
    g.dyq = w.dymx;
    g.dys = w.dymx + c.T * g.Hp;
    g.dhq = w.dhmx;
    g.dhs = w.dhmx + M * mx_kp(2 * (int64_t)c.I);
    g.segA = w.segA;
    g.segB = w.segB;
}

static hipError_t run_mx_gemm(int32_t op, const GemmArgs &g, hipStream_t s)
{
    StageMark mark(op, s);
    if (!g.dw_acc && (op == MOE_GEMM_DOWN_WGRAD || op == MOE_GEMM_UP_WGRAD)) {
        const bool up = op == MOE_GEMM_UP_WGRAD;
        hipError_t e = launch_zero_empty(g.E, (int64_t)2 * g.I * g.H / (up ? 1 : 2), g.counts,
                                         up ? g.dW1 : g.dW2, g.dw_bf16, s);
        if (e != hipSuccess) return e;
    }
    if (g.T == 0) return hipSuccess;
    return launch_mx_gemm(op, g, s);
}



static moe_status stage2_bwd(const moe_config *cfg, const moe_saved *saved, const uint16_t *w2,
                             const uint8_t *w2t_mx, const uint16_t *dy, void *dW2,
                             int32_t dw_dtype, int32_t dw_accumulate, void *ws, size_t ws_bytes,
                             hipStream_t stream)
{
    MOE_CHECK(moe_check_config(cfg));
    const moe_config &c = *cfg;
    if (dw_dtype != MOE_F32 && dw_dtype != MOE_BF16) return MOE_EINVAL;
    if (w2t_mx && c.precision != MOE_PRECISION_BF16) return MOE_EUNSUPPORTED;
    MOE_CHECK(check_saved_bwd(saved, c));
    MOE_CHECK(check_ptrs({w2t_mx ? (const void *)w2t_mx : (const void *)w2, dW2}));
    if (c.T > 0) MOE_CHECK(check_ptrs({dy}));
    size_t need = 0;
    BwdWs w = carve_bwd(c, ws, &need);
    if (ws_bytes < need || (need && !ws)) return MOE_EWORKSPACE;
    MOE_TRY(launch_schedule(c.E, saved->counts, w.sched, stream));
    moe_gemm_args a = saved_gemm_args(saved);
    a.dy = dy;
    a.w2 = w2;
    a.dh = w.dh;
    a.dw_part = w.dw_part;
    a.dW2 = dW2;
    a.dw_dtype = dw_dtype;
    a.dw_accumulate = dw_accumulate;
    GemmArgs g = gemm_args(c, a, w.sched);
    g.wrow = w.wrow;
    g.tA = w.tA;
    g.tB = w.tB;
    set_split(g, c, saved, &w);
    const bool mx = w2t_mx != nullptr;
    if (mx) {
        set_mx_bwd(g, c, w);
        g.w2cq = w2t_mx;
        g.w2cs = w2t_mx + (int64_t)c.E * c.I * g.Hp;
    }
    MOE_TRY(launch_row_weights(c.T * c.k, saved->row_map, saved->topk_w, w.wrow, stream));
    if (c.T > 0) {
        // dW2's operands, w*dy (dy gathered, times the routing weight) and a,
        // along each expert's rows; with MX also dy along H for the dgrad
        StageMark mark(MOE_STAGE_OPERANDS_BWD2, stream);
        if (mx) MOE_TRY(launch_mx_quantize(dy, c.T, c.H, w.dymx, stream));
        if (g.split) {
            // dy exact (gathered); w * (a + a_lo) in fp32, as a hi + lo pair
            MOE_TRY(prepare_segments(c, w.sched, saved->offsets, dy, c.H, saved->row_map, nullptr,
                                     false, w.tA, stream));
            MOE_TRY(prepare_segments(c, w.sched, saved->offsets, saved->a, c.I, nullptr, w.wrow,
                                     false, w.tB, stream, saved->a_lo, 0));
            MOE_TRY(prepare_segments(c, w.sched, saved->offsets, saved->a, c.I, nullptr, w.wrow,
                                     false, w.tB_lo, stream, saved->a_lo, 1));
        } else {
            MOE_TRY(prepare_segments(c, w.sched, saved->offsets, dy, c.H, saved->row_map, w.wrow,
                                     mx, w.tA, stream));
            MOE_TRY(prepare_segments(c, w.sched, saved->offsets, saved->a, c.I, nullptr, nullptr,
                                     mx, w.tB, stream));
        }
    }
    // dgrad (+ SwiGLU backward, routing-weight row-dots), then dW2
    if (mx) {
        if (c.T > 0) MOE_TRY(run_mx_gemm(MOE_GEMM_DOWN_DGRAD, g, stream));
        MOE_TRY(run_mx_gemm(MOE_GEMM_DOWN_WGRAD, g, stream));
    } else {
        if (c.T > 0) MOE_TRY(run_gemm(MOE_GEMM_DOWN_DGRAD, g, stream));
        MOE_TRY(run_gemm(MOE_GEMM_DOWN_WGRAD, g, stream));
    }
    return MOE_OK;
}

static moe_status stage1_bwd(const moe_config *cfg, const moe_saved *saved, const uint16_t *x,
                             const float *Wr, const uint16_t *w1, const uint8_t *w1t_mx,
                             const float *d_aux, float *dx, float *dlogits, float *dWr, void *dW1,
                             int32_t dw_dtype, int32_t dw_accumulate, void *ws, size_t ws_bytes,
                             hipStream_t stream, bool sched_ready)
{
    MOE_CHECK(moe_check_config(cfg));
    const moe_config &c = *cfg;
    if (dw_dtype != MOE_F32 && dw_dtype != MOE_BF16) return MOE_EINVAL;
    if (w1t_mx && c.precision != MOE_PRECISION_BF16) return MOE_EUNSUPPORTED;
    MOE_CHECK(check_saved_bwd(saved, c));
    MOE_CHECK(check_ptrs({w1t_mx ? (const void *)w1t_mx : (const void *)w1, dW1}));
    if (c.T > 0) MOE_CHECK(check_ptrs({x, dx, dlogits}));
    MOE_CHECK(check_opt_ptr(Wr));
    MOE_CHECK(check_opt_ptr(dWr));
    MOE_CHECK(check_opt_ptr(d_aux));
    size_t need = 0;
    BwdWs w = carve_bwd(c, ws, &need);
    if (ws_bytes < need || (need && !ws)) return MOE_EWORKSPACE;
    if (!sched_ready) MOE_TRY(launch_schedule(c.E, saved->counts, w.sched, stream));
    moe_gemm_args a = saved_gemm_args(saved);
    a.x = x;
    a.w1 = w1;
    a.dh = w.dh;
    a.dw_part = w.dw_part;
    a.dxp = w.dxp;
    a.dW1 = dW1;
    a.dw_dtype = dw_dtype;
    a.dw_accumulate = dw_accumulate;
    GemmArgs g = gemm_args(c, a, w.sched);
    g.tA = w.tA;
    g.tB = w.tB;
    set_split(g, c, saved, &w);
    // dgrad1's per-row partials of dx go out in bf16 (half the bytes for the
    // GEMM's epilogue and the un-permute); dx itself is summed in fp32
    g.dxp_bf16 = (uint16_t *)w.dxp;
    const bool mx = w1t_mx != nullptr;
    if (mx) {
        set_mx_bwd(g, c, w);
        g.w1cq = w1t_mx;
        g.w1cs = w1t_mx + (int64_t)c.E * c.H * mx_kp(2 * (int64_t)c.I);
    }
    if (c.T > 0) {
        // dW1's operands, dh and x (gathered), along each expert's rows; with
        // MX also dh along 2I for the dgrad
        StageMark mark(MOE_STAGE_OPERANDS_BWD1, stream);
        if (mx) MOE_TRY(launch_mx_quantize(w.dh, c.T * c.k, 2 * (int64_t)c.I, w.dhmx, stream));
        MOE_TRY(prepare_segments(c, w.sched, saved->offsets, w.dh, 2 * (int64_t)c.I, nullptr,
                                 nullptr, mx, w.tA, stream));
        if (g.split)  // dh's remainder, for dW1's second pass
            MOE_TRY(prepare_segments(c, w.sched, saved->offsets, w.dh_lo, 2 * (int64_t)c.I,
                                     nullptr, nullptr, false, w.tA_lo, stream));
        MOE_TRY(prepare_segments(c, w.sched, saved->offsets, x, c.H, saved->row_map, nullptr, mx,
                                 w.tB, stream));
    }
    // dgrad, then dW1
    if (mx) {
        if (c.T > 0) MOE_TRY(run_mx_gemm(MOE_GEMM_UP_DGRAD, g, stream));
        MOE_TRY(run_mx_gemm(MOE_GEMM_UP_WGRAD, g, stream));
    } else {
        if (c.T > 0) MOE_TRY(run_gemm(MOE_GEMM_UP_DGRAD, g, stream));
        MOE_TRY(run_gemm(MOE_GEMM_UP_WGRAD, g, stream));
    }
    if (c.T == 0) {
        if (dWr && Wr) MOE_TRY(launch_fill_f32(dWr, (int64_t)c.E * c.H, 0.f, stream));
        return MOE_OK;
    }
    // router: d logits (from the routing-weight row-dots stage 2 left in the
    // workspace), then dx = un-permute(dxp) + dlogits . Wr, dWr = dlogits^T . x
    RouterBwdArgs rb;
    rb.T = c.T;
    rb.E = c.E;
    rb.k = c.k;
    rb.score = c.score;
    rb.renorm = c.renorm;
    rb.ncols = dgrad2_cols(c.I);
    rb.scale = c.scale;
    rb.aux_coeff = c.aux_coeff;
    rb.logits = saved->logits;
    rb.topk_w = saved->topk_w;
    rb.dw_part = w.dw_part;
    rb.d_aux = d_aux;
    rb.topk_idx = saved->topk_idx;
    rb.counts = saved->counts;
    rb.pos = saved->pos;
    rb.dlogits = dlogits;
    {
        StageMark mark(MOE_STAGE_ROUTER_BWD, stream);
        MOE_TRY(launch_router_bwd(rb, stream));
    }
    {
        StageMark mark(MOE_STAGE_UNPERMUTE, stream);
        MOE_TRY(launch_combine_bf16(c.T, c.k, c.H, g.dxp_bf16, nullptr, saved->pos, dx, stream));
    }
    if (Wr) {
        StageMark mark(MOE_STAGE_ROUTER_GRADS, stream);
        MOE_TRY(launch_router_grads(c.T, c.E, c.H, dlogits, x, Wr, dx, dWr, w.router, stream));
    }
    return MOE_OK;
}

moe_status moe_stage2_backward(const moe_config *cfg, const moe_saved *saved, const uint16_t *w2,
                               const uint16_t *dy, void *dW2, int32_t dw_dtype,
                               int32_t dw_accumulate, void *ws, size_t ws_bytes,
                               hipStream_t stream)
{
    return stage2_bwd(cfg, saved, w2, nullptr, dy, dW2, dw_dtype, dw_accumulate, ws, ws_bytes,
                      stream);
}

moe_status moe_stage1_backward(const moe_config *cfg, const moe_saved *saved, const uint16_t *x,
                               const float *Wr, const uint16_t *w1, const float *d_aux, float *dx,
                               float *dlogits, float *dWr, void *dW1, int32_t dw_dtype,
                               int32_t dw_accumulate, void *ws, size_t ws_bytes,
                               hipStream_t stream)
{
    return stage1_bwd(cfg, saved, x, Wr, w1, nullptr, d_aux, dx, dlogits, dWr, dW1, dw_dtype,
                      dw_accumulate, ws, ws_bytes, stream);
}

moe_status moe_backward(const moe_config *cfg, const moe_saved *saved, const uint16_t *x,
                        const float *Wr, const uint16_t *w1, const uint16_t *w2,
                        const uint16_t *dy, const float *d_aux, float *dx, float *dlogits,
                        float *dWr, void *dW1, void *dW2, int32_t dw_dtype,
                        int32_t dw_accumulate, void *ws, size_t ws_bytes, hipStream_t stream)
{
    MOE_CHECK(moe_check_config(cfg));
    // everything stage 1 validates, checked before stage 2 launches anything
    MOE_CHECK(check_ptrs({w1, dW1}));
    if (cfg->T > 0) MOE_CHECK(check_ptrs({x, dx, dlogits}));
    MOE_CHECK(check_opt_ptr(Wr));
    MOE_CHECK(check_opt_ptr(dWr));
    MOE_CHECK(check_opt_ptr(d_aux));
    MOE_CHECK(moe_stage2_backward(cfg, saved, w2, dy, dW2, dw_dtype, dw_accumulate, ws, ws_bytes,
                                  stream));
    return stage1_bwd(cfg, saved, x, Wr, w1, nullptr, d_aux, dx, dlogits, dWr, dW1, dw_dtype,
                      dw_accumulate, ws, ws_bytes, stream, true);
}

// ------------------------------------------------------ no allocation ----
// moe_forward on a scratch area the library owns: a file-scope device array
// (one copy per GPU, created when the code object loads and held until the
// process ends).  Host code never passes the array's name to a kernel: it
// reads the array's device address once per device with hipGetSymbolAddress
// and passes that.
static __device__ __align__(256) unsigned char scratch[MOE_NOALLOC_SCRATCH_BYTES];

static std::mutex g_scratch_mu;
static void *g_scratch_dev[MOE_NOALLOC_MAX_DEVICES];

// The current device's address of `scratch` (looked up on the first call on
// that device, with that device current).
static moe_status scratch_address(hipStream_t stream, void **out)
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return MOE_EHIP;
    if (dev < 0 || dev >= MOE_NOALLOC_MAX_DEVICES) return MOE_EUNSUPPORTED;
    if (stream) {
        hipDevice_t sdev = -1;
        if (hipStreamGetDevice(stream, &sdev) != hipSuccess) return MOE_EHIP;
        if ((int)sdev != dev) return MOE_EINVAL;  // the stream must belong to the current device
    }
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_dev[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MOE_EHIP;
        g_scratch_dev[dev] = p;
    }
    *out = g_scratch_dev[dev];
    return MOE_OK;
}

moe_status moe_forward_noalloc_bytes(const moe_config *cfg, size_t *bytes)
{
    MOE_CHECK(moe_check_config(cfg));
    if (!bytes) return MOE_EINVAL;
    *bytes = fwd_need(*cfg, false);
    return MOE_OK;
}

moe_status moe_forward_noalloc(const moe_config *cfg, const uint16_t *x, const float *Wr,
                               const float *bias, const uint16_t *w1, const uint16_t *w2,
                               float *y, float *aux, const moe_saved *saved, hipStream_t stream)
{
    MOE_CHECK(moe_check_config(cfg));
    const size_t need = fwd_need(*cfg, false);
    if (need > (size_t)MOE_NOALLOC_SCRATCH_BYTES) return MOE_EWORKSPACE;
    void *ws = nullptr;
    MOE_CHECK(scratch_address(stream, &ws));
    // every area of the forward workspace is written before it is read in one
    // call, so nothing is cleared first
    return moe_forward(cfg, x, Wr, bias, w1, w2, y, aux, saved, ws,
                       (size_t)MOE_NOALLOC_SCRATCH_BYTES, stream);
}

}  // extern "C"
