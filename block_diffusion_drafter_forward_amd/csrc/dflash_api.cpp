// Host side of the C ABI declared in include/dflash.h: argument validation (done entirely before any HIP
// call, so every error path can be exercised without a GPU), workspace planning, the launch sequence of the
// drafter pass and of KV injection, and optional per-kernel event timing.
#include <hip/hip_runtime.h>

#include <cmath>
#include <initializer_list>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <map>
#include <string>
#include <vector>

#include "dflash.h"
#include "gemm_core.h"
#include "kernels.h"

using namespace df;

// ---------------------------------------------------------------------------------------------------------
// errors
// ---------------------------------------------------------------------------------------------------------
static thread_local char g_err[512] = "";

static int fail(int code, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return code;
}

extern "C" const char* dflash_last_error(void) { return g_err; }

#define HIP_TRY(expr)                                                                          \
    do {                                                                                       \
        hipError_t e_ = (expr);                                                                \
        if (e_ != hipSuccess) return fail(DFLASH_E_HIP, "%s: %s", #expr, hipGetErrorString(e_)); \
    } while (0)

// ---------------------------------------------------------------------------------------------------------
// handle
// ---------------------------------------------------------------------------------------------------------
struct ProfEntry {
    std::string name;
    hipEvent_t start, stop;
};

// Element offsets of every packed matrix in the store of a bfloat16 drafter (layout: gemm_core.h).  Matrices
// that one GEMM stacks along N are packed as one matrix: [wq; wk; wv], [w_gate; w_up], and the [uk; uv] of the
// layers one inject GEMM covers (MAX_LAYERS_PER_KV_GEMM at a time).  The store lists the drafter pass's
// matrices in the order the pass reads them.
#define MAX_LAYERS_PER_KV_GEMM (DF_MAX_SEG / 2)
struct PackLayout {
    std::vector<size_t> qkv, o, gu, down;  // per layer
    size_t kv = 0, kv_stride = 0;          // layer l's [uk; uv] at kv + l * kv_stride
    size_t fc = 0, lm = 0, total = 0;
};

// Row segments of matrices stacked along N (each {rows pointer, row count}).
static Segs stack_rows(std::initializer_list<std::pair<const void*, int>> parts) {
    Segs s{};
    int n = 0, i = 0;
    for (const auto& p : parts) {
        s.ptr[i] = p.first;
        s.start[i] = n;
        n += p.second;
        ++i;
    }
    s.start[i] = n;
    s.n = i;
    return s;
}

static PackLayout pack_layout(const dflash_config& c) {
    PackLayout pl;
    const int H = c.hidden, F = c.ffn, qd = c.n_q_heads * c.head_dim, kvd = c.n_kv_heads * c.head_dim;
    size_t off = 0;
    auto take = [&](size_t n) { size_t o = off; off += n; return o; };
    for (int l = 0; l < c.n_layers; ++l) {
        pl.qkv.push_back(take(packed_elems(qd + 2 * kvd, H)));
        pl.o.push_back(take(packed_elems(H, qd)));
        pl.gu.push_back(take(packed_elems(2 * F, H)));
        pl.down.push_back(take(packed_elems(H, F)));
    }
    pl.kv_stride = packed_elems(2 * kvd, H);  // a group of n layers: n * kv_stride (2 kvd is a multiple of 64)
    pl.kv = take((size_t)c.n_layers * pl.kv_stride);
    pl.fc = take(packed_elems(H, c.feat_dim));
    pl.lm = take(packed_elems(c.vocab, H));
    pl.total = off;
    return pl;
}

struct dflash_handle {
    dflash_config cfg;
    dflash_weights w;
    std::vector<dflash_layer_weights> layers;
    RopeFreq rf;
    PackLayout pl;
    const bf16_t* packed = nullptr;  // packed store (bfloat16 drafters), set by dflash_pack_weights
    bool profiling = false;
    std::vector<hipEvent_t> event_pool;
    std::vector<ProfEntry> pending;
};

static bool is_bf16(const dflash_config& c) { return c.dtype == DFLASH_BF16; }
static size_t elt(const dflash_config& c) { return is_bf16(c) ? 2 : 4; }
// Transient activations: a pair of bfloat16 planes (bfloat16 drafters) or float32 -- 4 bytes per element.
static const size_t ACT = 4;

static int validate_config(const dflash_config* c) {
    if (!c) return fail(DFLASH_E_ARG, "config is NULL");
    if (c->n_layers < 1 || c->hidden < 1 || c->n_q_heads < 1 || c->n_kv_heads < 1 || c->head_dim < 2 ||
        c->ffn < 1 || c->vocab < 1 || c->feat_dim < 1)
        return fail(DFLASH_E_ARG, "config sizes must be positive");
    if (c->dtype != DFLASH_F32 && c->dtype != DFLASH_BF16) return fail(DFLASH_E_ARG, "unknown dtype %d", c->dtype);
    if (c->n_q_heads % c->n_kv_heads) return fail(DFLASH_E_SHAPE, "n_q_heads %% n_kv_heads != 0");
    {
        const int G = c->n_q_heads / c->n_kv_heads;
        if (G != 1 && G != 2 && G != 4 && G != 8)
            return fail(DFLASH_E_UNSUPPORTED, "query heads per KV head must be 1, 2, 4 or 8");
    }
    if (c->block_len < 2 || c->block_len > 16) return fail(DFLASH_E_UNSUPPORTED, "block_len must be in [2, 16]");
    if (c->page_size != 16) return fail(DFLASH_E_UNSUPPORTED, "page_size must be 16");
    if (c->hidden > 16384) return fail(DFLASH_E_UNSUPPORTED, "hidden must be <= 16384");
    if (!(c->rms_eps >= 0.f) || !(c->rope_theta >= 0.f)) return fail(DFLASH_E_ARG, "rms_eps and rope_theta must be >= 0");
    const int qd = c->n_q_heads * c->head_dim;
    if (is_bf16(*c)) {
        if (c->head_dim != 64 && c->head_dim != 128) return fail(DFLASH_E_UNSUPPORTED, "bf16 kernels need head_dim 64 or 128");
        if (c->hidden % 256 || c->ffn % 256 || c->feat_dim % 256 || qd % 256)
            return fail(DFLASH_E_UNSUPPORTED, "bf16 kernels need hidden, ffn, feat_dim, n_q*d multiples of 256");
    } else {
        if (c->head_dim % 2 || c->head_dim > 128) return fail(DFLASH_E_UNSUPPORTED, "f32 kernels need even head_dim <= 128");
        if (c->hidden % 4 || c->ffn % 4 || c->feat_dim % 4 || qd % 4)
            return fail(DFLASH_E_UNSUPPORTED, "f32 kernels need hidden, ffn, feat_dim, n_q*d multiples of 4");
    }
    return DFLASH_OK;
}

extern "C" int dflash_create(const dflash_config* cfg, const dflash_weights* w, dflash_handle** out) {
    if (!out) return fail(DFLASH_E_ARG, "out is NULL");
    *out = nullptr;
    int rc = validate_config(cfg);
    if (rc) return rc;
    if (!w || !w->layers) return fail(DFLASH_E_ARG, "weights or weights->layers is NULL");
    if (!w->fc_w || !w->embed || !w->final_norm || !w->lm_head) return fail(DFLASH_E_ARG, "a global weight is NULL");
    for (int l = 0; l < cfg->n_layers; ++l) {
        const dflash_layer_weights& L = w->layers[l];
        if (!L.attn_norm || !L.wq || !L.wk || !L.wv || !L.wo || !L.uk || !L.uv || !L.ffn_norm || !L.w_gate ||
            !L.w_up || !L.w_down)
            return fail(DFLASH_E_ARG, "a weight of layer %d is NULL", l);
    }
    dflash_handle* h = new dflash_handle();
    h->cfg = *cfg;
    h->layers.assign(w->layers, w->layers + cfg->n_layers);
    h->w = *w;
    h->w.layers = h->layers.data();
    std::memset(&h->rf, 0, sizeof(h->rf));
    h->rf.on = cfg->rope_theta > 0.f;
    for (int i = 0; i < cfg->head_dim / 2; ++i)
        h->rf.inv[i] = h->rf.on ? (float)std::pow((double)cfg->rope_theta, -2.0 * i / cfg->head_dim) : 0.f;
    if (is_bf16(*cfg)) h->pl = pack_layout(*cfg);
    *out = h;
    return DFLASH_OK;
}

extern "C" size_t dflash_packed_weight_bytes(const dflash_handle* h) {
    if (!h || !is_bf16(h->cfg)) return 0;
    return h->pl.total * 2;
}

extern "C" int dflash_pack_weights(dflash_handle* h, void* dst, size_t dst_bytes, void* stream) {
    if (!h) return fail(DFLASH_E_ARG, "handle is NULL");
    const dflash_config& c = h->cfg;
    if (!is_bf16(c)) return DFLASH_OK;  // float32 drafters stream the row-major matrices
    if (!dst) return fail(DFLASH_E_ARG, "dst is NULL");
    if (((uintptr_t)dst) & 255) return fail(DFLASH_E_ARG, "dst must be 256-byte aligned");
    if (dst_bytes < h->pl.total * 2) return fail(DFLASH_E_CAPACITY, "dst %zu < %zu bytes", dst_bytes, h->pl.total * 2);
    {
        uintptr_t a = (uintptr_t)h->w.fc_w | (uintptr_t)h->w.lm_head;
        for (const dflash_layer_weights& w : h->layers)
            a |= (uintptr_t)w.wq | (uintptr_t)w.wk | (uintptr_t)w.wv | (uintptr_t)w.wo | (uintptr_t)w.w_gate |
                 (uintptr_t)w.w_up | (uintptr_t)w.w_down | (uintptr_t)w.uk | (uintptr_t)w.uv;
        if (a & 15) return fail(DFLASH_E_ARG, "projection matrices must be 16-byte aligned");
    }
    hipStream_t st = (hipStream_t)stream;
    bf16_t* P = (bf16_t*)dst;
    const int H = c.hidden, F = c.ffn, qd = c.n_q_heads * c.head_dim, kvd = c.n_kv_heads * c.head_dim;
    const PackLayout& pl = h->pl;
    if ((2 * kvd) % 64) return fail(DFLASH_E_UNSUPPORTED, "2 * n_kv_heads * head_dim must be a multiple of 64");
    for (int l = 0; l < c.n_layers; ++l) {
        const dflash_layer_weights& w = h->layers[l];
        HIP_TRY(launch_pack(stack_rows({{w.wq, qd}, {w.wk, kvd}, {w.wv, kvd}}), qd + 2 * kvd, H, P + pl.qkv[l], st));
        HIP_TRY(launch_pack(stack_rows({{w.wo, H}}), H, qd, P + pl.o[l], st));
        HIP_TRY(launch_pack(stack_rows({{w.w_gate, F}, {w.w_up, F}}), 2 * F, H, P + pl.gu[l], st));
        HIP_TRY(launch_pack(stack_rows({{w.w_down, H}}), H, F, P + pl.down[l], st));
    }
    for (int l0 = 0; l0 < c.n_layers; l0 += MAX_LAYERS_PER_KV_GEMM) {  // the groups dflash_inject_ctx multiplies
        const int nl = std::min(MAX_LAYERS_PER_KV_GEMM, c.n_layers - l0);
        Segs s{};
        for (int i = 0; i < nl; ++i) {
            s.ptr[2 * i] = h->layers[l0 + i].uk;
            s.ptr[2 * i + 1] = h->layers[l0 + i].uv;
            s.start[2 * i] = 2 * i * kvd;
            s.start[2 * i + 1] = (2 * i + 1) * kvd;
        }
        s.start[2 * nl] = 2 * nl * kvd;
        s.n = 2 * nl;
        HIP_TRY(launch_pack(s, 2 * nl * kvd, H, P + pl.kv + l0 * pl.kv_stride, st));
    }
    HIP_TRY(launch_pack(stack_rows({{h->w.fc_w, H}}), H, c.feat_dim, P + pl.fc, st));
    HIP_TRY(launch_pack(stack_rows({{h->w.lm_head, c.vocab}}), c.vocab, H, P + pl.lm, st));
    h->packed = P;
    return DFLASH_OK;
}

extern "C" void dflash_destroy(dflash_handle* h) {
    if (!h) return;
    for (auto& p : h->pending) {
        h->event_pool.push_back(p.start);
        h->event_pool.push_back(p.stop);
    }
    for (hipEvent_t e : h->event_pool) (void)hipEventDestroy(e);
    delete h;
}

// ---------------------------------------------------------------------------------------------------------
// profiling
// ---------------------------------------------------------------------------------------------------------
thread_local LaunchTiming* df::df_launch_timing = nullptr;

static hipEvent_t take_event(dflash_handle* h) {
    if (!h->event_pool.empty()) {
        hipEvent_t e = h->event_pool.back();
        h->event_pool.pop_back();
        return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
}

// One profiled launch.  The start event is recorded before the launch; a launcher that takes the events
// (DF_LAUNCH) records both again around the kernel itself, otherwise the stop event is recorded after the
// launch.
struct Timed {
    dflash_handle* h;
    hipStream_t st;
    ProfEntry e{};
    LaunchTiming lt{};
    bool on;
    Timed(dflash_handle* h_, const char* name, hipStream_t s, int N = 0, int K = 0)
        : h(h_), st(s), on(h_ && h_->profiling) {
        if (!on) return;
        e.name = name;
        if (N > 0) e.name += " N=" + std::to_string(N) + " K=" + std::to_string(K);
        e.start = take_event(h);
        e.stop = take_event(h);
        if (e.start) (void)hipEventRecord(e.start, st);
        if (e.start && e.stop) {
            lt = LaunchTiming{e.start, e.stop, false};
            df_launch_timing = &lt;
        }
    }
    ~Timed() {
        if (!on) return;
        df_launch_timing = nullptr;
        if (e.stop && !lt.used) (void)hipEventRecord(e.stop, st);
        if (e.start && e.stop) h->pending.push_back(e);
    }
};

extern "C" int dflash_profile_enable(dflash_handle* h, int on) {
    if (!h) return fail(DFLASH_E_ARG, "handle is NULL");
    h->profiling = on != 0;
    return DFLASH_OK;
}

extern "C" int dflash_profile_collect(dflash_handle* h, dflash_kernel_stat* out, int max_entries) {
    if (!h) return fail(DFLASH_E_ARG, "handle is NULL");
    if (max_entries > 0 && !out) return fail(DFLASH_E_ARG, "out is NULL");
    std::map<std::string, std::pair<int, double>> acc;
    std::vector<std::string> order;
    for (auto& p : h->pending) {
        HIP_TRY(hipEventSynchronize(p.stop));
        float ms = 0.f;
        HIP_TRY(hipEventElapsedTime(&ms, p.start, p.stop));
        if (!acc.count(p.name)) order.push_back(p.name);
        acc[p.name].first += 1;
        acc[p.name].second += ms;
        h->event_pool.push_back(p.start);
        h->event_pool.push_back(p.stop);
    }
    h->pending.clear();
    int n = 0;
    for (auto& name : order) {
        if (n >= max_entries) break;
        std::memset(&out[n], 0, sizeof(out[n]));
        std::snprintf(out[n].name, sizeof(out[n].name), "%s", name.c_str());
        out[n].launches = acc[name].first;
        out[n].total_ms = acc[name].second;
        ++n;
    }
    return n;
}

// ---------------------------------------------------------------------------------------------------------
// workspace planning
// ---------------------------------------------------------------------------------------------------------
static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

struct Carve {
    size_t off = 0;
    size_t take(size_t bytes) {
        size_t o = off;
        off = align256(off + bytes);
        return o;
    }
};

struct DraftPlan {
    int M;
    GemmPlan qkv, oproj, gateup, down;
    AttnPlan attn;
    size_t err, h, u, q, kb, vbt, o, a, part, opart, ml, hpart, total;
};

static DraftPlan plan_draft(const dflash_config& c, int batch, int max_ctx) {
    DraftPlan p{};
    const int bf = is_bf16(c);
    const int M = batch * c.block_len;
    const int qd = c.n_q_heads * c.head_dim, kvd = c.n_kv_heads * c.head_dim;
    p.M = M;
    p.qkv = plan_gemm(bf, M, qd + 2 * kvd, c.hidden, true);
    p.oproj = plan_gemm(bf, M, c.hidden, qd, true);
    p.gateup = plan_gemm(bf, M, 2 * c.ffn, c.hidden, true);
    p.down = plan_gemm(bf, M, c.hidden, c.ffn, true);
    p.attn = plan_attention(batch, c.n_q_heads, c.n_kv_heads, max_ctx, c.n_layers);
    size_t part = (size_t)p.qkv.splits * M * (qd + 2 * kvd);
    part = std::max(part, (size_t)p.oproj.splits * M * c.hidden);
    part = std::max(part, (size_t)p.gateup.splits * M * 2 * c.ffn);
    part = std::max(part, (size_t)p.down.splits * M * c.hidden);
    Carve cv;
    p.err = cv.take(256);
    p.h = cv.take((size_t)M * c.hidden * 4);
    p.u = cv.take((size_t)M * c.hidden * ACT);
    p.q = cv.take((size_t)M * qd * ACT);
    p.kb = cv.take((size_t)batch * kvd * 16 * ACT);
    p.vbt = cv.take((size_t)batch * kvd * 16 * ACT);
    p.o = cv.take((size_t)M * qd * ACT);
    p.a = cv.take((size_t)M * c.ffn * ACT);
    p.part = cv.take(part * 4);
    const size_t C1 = (size_t)attn_slots(p.attn);
    if (bf) {
        p.opart = cv.take((size_t)batch * c.n_q_heads * C1 * 16 * c.head_dim * 4);
        p.ml = cv.take((size_t)batch * c.n_q_heads * C1 * 16 * 2 * 4);
    } else {
        p.opart = cv.take((size_t)M * qd * 4);
        p.ml = cv.take(0);
    }
    p.hpart = cv.take(head_partial_floats(bf, c.vocab, M) * 4);
    p.total = cv.off;
    return p;
}

static bool draft_shape_ok(const dflash_config& c, int batch) {
    const int M = batch * c.block_len;
    return is_bf16(c) || M <= 32;  // the float32 LM head keeps at most 32 block rows per workgroup
}

extern "C" size_t dflash_draft_workspace_bytes(const dflash_handle* h, int max_batch, int max_ctx) {
    if (!h || max_batch < 1 || max_ctx < 0) return 0;
    return plan_draft(h->cfg, max_batch, max_ctx).total;
}

#define INJECT_ROWS 4096  // rows per internal chunk of dflash_inject_ctx (bounds the workspace)

struct InjectPlan {
    int rows;
    size_t err, f, part, total;
};

// Float32 split partials one chunk of R rows writes: the fusion GEMM's and the widest KV GEMM's.  plan_gemm
// may give a short chunk more splits than a long one (fewer tiles, so K is split further), so the product is
// not monotonic in R.
static size_t inject_part_floats(const dflash_config& c, int R) {
    const int bf = is_bf16(c);
    const int kvd = c.n_kv_heads * c.head_dim;
    const GemmPlan fc = plan_gemm(bf, R, c.hidden, c.feat_dim);
    size_t need = (size_t)fc.splits * R * c.hidden;
    // every layer group's KV GEMM (the last group may be narrower, hence split further)
    for (int l0 = 0; l0 < c.n_layers; l0 += MAX_LAYERS_PER_KV_GEMM) {
        const int nl = std::min(MAX_LAYERS_PER_KV_GEMM, c.n_layers - l0);
        const GemmPlan kv = plan_gemm(bf, R, nl * 2 * kvd, c.hidden);
        need = std::max(need, (size_t)kv.splits * R * nl * 2 * kvd);
    }
    return need;
}

// Workspace of a dflash_inject_ctx call of n_rows rows: chunks of INJECT_ROWS rows and a shorter last chunk
// (exact = 1), or of any call of at most n_rows rows, i.e. any chunk length up to min(n_rows, INJECT_ROWS)
// (exact = 0, what dflash_inject_workspace_bytes reports).
static InjectPlan plan_inject(const dflash_config& c, int n_rows, bool exact) {
    InjectPlan p{};
    const int R = n_rows < INJECT_ROWS ? n_rows : INJECT_ROWS;
    p.rows = R;
    size_t part = 0;
    if (exact) {
        part = inject_part_floats(c, R);
        if (n_rows % R) part = std::max(part, inject_part_floats(c, n_rows % R));
    } else {
        for (int r = 1; r <= R; ++r) part = std::max(part, inject_part_floats(c, r));
    }
    Carve cv;
    p.err = cv.take(256);
    p.f = cv.take((size_t)R * c.hidden * ACT);
    p.part = cv.take(part * 4);
    p.total = cv.off;
    return p;
}

extern "C" size_t dflash_inject_workspace_bytes(const dflash_handle* h, int max_rows) {
    if (!h || max_rows < 1) return 0;
    return plan_inject(h->cfg, max_rows, false).total;
}

// ---------------------------------------------------------------------------------------------------------
// dflash_draft_block
// ---------------------------------------------------------------------------------------------------------
static Segs segs1(const void* p, int n) {
    Segs s{};
    s.ptr[0] = p;
    s.start[0] = 0;
    s.start[1] = n;
    s.n = 1;
    return s;
}

// One projection: bfloat16 drafters stream the packed matrix at element offset `packed_off` of the store,
// float32 drafters the row-major segments `rows`.
static hipError_t project(const dflash_handle* h, const GemmPlan& p, const void* x, int ldx, size_t xplane, int M,
                          size_t packed_off, const Segs& rows, int N, int K, float* part, hipStream_t st) {
    if (is_bf16(h->cfg)) return launch_gemm_bf16(p, x, ldx, xplane, M, h->packed + packed_off, N, K, part, st);
    return launch_gemm_f32((const float*)x, ldx, M, rows, N, K, part, st);
}

// The drafter pass; sample != 0 draws each row's token at temperature 1 (Gumbel-max, keyed by seed) instead
// of taking the argmax, and logits_out (nullable) receives the full logits.
// static_scratch: the workspace is the library's own static scratch (ws and ws_bytes unused), looked up only
// after every argument check has passed.
static int draft_impl(dflash_handle* h, int batch, const int32_t* block_tokens, const int32_t* ctx_len,
                      const int32_t* page_table, int max_pages, const dflash_kv* kv, int max_ctx, int top_k,
                      int sample, uint64_t seed, int32_t* tokens, int32_t* topk_ids, float* topk_logprobs,
                      float* logits_out, const dflash_debug* dbg, void* ws, size_t ws_bytes, bool static_scratch,
                      void* stream) {
    if (!h) return fail(DFLASH_E_ARG, "handle is NULL");
    const dflash_config& c = h->cfg;
    if (batch < 1) return fail(DFLASH_E_ARG, "batch must be >= 1");
    if (!block_tokens || !ctx_len || !tokens || (!ws && !static_scratch))
        return fail(DFLASH_E_ARG, "a required pointer is NULL");
    if (top_k < 0 || top_k > DF_TOPK) return fail(DFLASH_E_UNSUPPORTED, "top_k must be in [0, 8]");
    if (top_k > c.vocab) return fail(DFLASH_E_ARG, "top_k exceeds the vocabulary");
    if (top_k > 0 && (!topk_ids || !topk_logprobs)) return fail(DFLASH_E_ARG, "top-k outputs are NULL");
    if (max_ctx < 0) return fail(DFLASH_E_ARG, "max_ctx must be >= 0");
    if (max_ctx > 0) {
        if (!page_table || !kv || !kv->k || !kv->v) return fail(DFLASH_E_ARG, "page table or KV pool is NULL");
        if (max_pages < 1 || kv->n_pages < 1) return fail(DFLASH_E_ARG, "max_pages and n_pages must be >= 1");
        if ((long long)max_ctx > (long long)max_pages * c.page_size)
            return fail(DFLASH_E_CAPACITY, "max_ctx %d exceeds max_pages * page_size", max_ctx);
    }
    if (!draft_shape_ok(c, batch))
        return fail(DFLASH_E_UNSUPPORTED, "float32 drafters support batch * block_len <= 32 (got %d)",
                    batch * c.block_len);
    const DraftPlan p = plan_draft(c, batch, max_ctx);
    if (static_scratch) {
        if (p.total > DFLASH_NOALLOC_SCRATCH_BYTES)
            return fail(DFLASH_E_CAPACITY,
                        "batch %d with max_ctx %d needs %zu bytes of scratch; the allocation-free pass has %u "
                        "(use dflash_draft_block with a workspace)",
                        batch, max_ctx, p.total, (unsigned)DFLASH_NOALLOC_SCRATCH_BYTES);
    } else {
        if (ws_bytes < p.total) return fail(DFLASH_E_CAPACITY, "workspace %zu < %zu bytes", ws_bytes, p.total);
        if (((uintptr_t)ws) & 255) return fail(DFLASH_E_ARG, "workspace must be 256-byte aligned");
    }
    if (is_bf16(c) && !h->packed) return fail(DFLASH_E_ARG, "bfloat16 weights are not packed (dflash_pack_weights)");
    if (static_scratch) HIP_TRY(scratch_region(&ws, &ws_bytes));

    hipStream_t st = (hipStream_t)stream;
    char* W = (char*)ws;
    uint32_t* err = (uint32_t*)(W + p.err);
    float* hbuf = (float*)(W + p.h);
    void* u = W + p.u;
    void* q = W + p.q;
    void* kb = W + p.kb;
    void* vbt = W + p.vbt;
    void* o = W + p.o;
    void* a = W + p.a;
    float* part = (float*)(W + p.part);
    float* opart = (float*)(W + p.opart);
    float* ml = (float*)(W + p.ml);
    float* hpart = (float*)(W + p.hpart);
    const int bf = is_bf16(c);
    const int M = p.M, H = c.hidden, L = c.block_len;
    const int nq = c.n_q_heads, nkv = c.n_kv_heads, d = c.head_dim;
    const int qd = nq * d, kvd = nkv * d;
    const size_t tap_stride = (size_t)M * H;
    float* tap = dbg ? dbg->hidden : nullptr;
    const void* kpool = max_ctx > 0 && kv ? kv->k : nullptr;
    const void* vpool = max_ctx > 0 && kv ? kv->v : nullptr;
    // Without context the attention kernels read no page table and no pool, whatever the caller passed.
    const int n_pages = max_ctx > 0 && kv ? kv->n_pages : 0;
    if (max_ctx == 0) {
        page_table = nullptr;
        max_pages = 0;
    }

    {
        Timed t(h, "embed_norm", st);
        HIP_TRY(launch_embed_norm(bf, block_tokens, M, c.vocab, h->w.embed, h->layers[0].attn_norm, H, c.rms_eps, hbuf,
                                  u, tap, err, st));
    }
    for (int l = 0; l < c.n_layers; ++l) {
        const dflash_layer_weights& lw = h->layers[l];
        Segs sq{};
        sq.ptr[0] = lw.wq; sq.ptr[1] = lw.wk; sq.ptr[2] = lw.wv;
        sq.start[0] = 0; sq.start[1] = qd; sq.start[2] = qd + kvd; sq.start[3] = qd + 2 * kvd;
        sq.n = 3;
        {
            Timed t(h, gemm_kernel_name(p.qkv, bf), st, qd + 2 * kvd, H);
            HIP_TRY(project(h, p.qkv, u, H, bf ? (size_t)M * H : 0, M, bf ? h->pl.qkv[l] : 0, sq, qd + 2 * kvd, H,
                            part, st));
        }
        {
            Timed t(h, "qkv_epilogue", st);
            HIP_TRY(launch_qkv_epilogue(bf, part, p.qkv.splits, batch, L, nq, nkv, d, ctx_len, h->rf, q, kb, vbt, st));
        }
        {
            Timed t(h, bf ? "attn_bf16" : "attn_f32", st);
            HIP_TRY(launch_attention(bf, p.attn, batch, L, nq, nkv, d, q, kb, vbt, kpool, vpool, l, n_pages, page_table,
                                     max_pages, ctx_len, max_ctx, opart, ml, err, st));
        }
        const void* attn_out = opart;
        if (bf) {
            Timed t(h, "attn_merge", st);
            HIP_TRY(launch_attn_merge(bf, p.attn, batch, L, nq, d, opart, ml, o, st));
            attn_out = o;
        }
        {
            Timed t(h, gemm_kernel_name(p.oproj, bf), st, H, qd);
            HIP_TRY(project(h, p.oproj, attn_out, qd, bf ? (size_t)M * qd : 0, M, bf ? h->pl.o[l] : 0, segs1(lw.wo, H),
                            H, qd, part, st));
        }
        {
            Timed t(h, "resid_norm", st);
            HIP_TRY(launch_resid_norm(bf, part, p.oproj.splits, M, H, hbuf, lw.ffn_norm, c.rms_eps, u, nullptr, st));
        }
        Segs sg{};
        sg.ptr[0] = lw.w_gate; sg.ptr[1] = lw.w_up;
        sg.start[0] = 0; sg.start[1] = c.ffn; sg.start[2] = 2 * c.ffn;
        sg.n = 2;
        {
            Timed t(h, gemm_kernel_name(p.gateup, bf), st, 2 * c.ffn, H);
            HIP_TRY(project(h, p.gateup, u, H, bf ? (size_t)M * H : 0, M, bf ? h->pl.gu[l] : 0, sg, 2 * c.ffn, H,
                            part, st));
        }
        {
            Timed t(h, "swiglu", st);
            HIP_TRY(launch_swiglu(bf, part, p.gateup.splits, M, c.ffn, a, st));
        }
        {
            Timed t(h, gemm_kernel_name(p.down, bf), st, H, c.ffn);
            HIP_TRY(project(h, p.down, a, c.ffn, bf ? (size_t)M * c.ffn : 0, M, bf ? h->pl.down[l] : 0,
                            segs1(lw.w_down, H), H, c.ffn, part, st));
        }
        {
            const void* next_gain = l + 1 < c.n_layers ? h->layers[l + 1].attn_norm : h->w.final_norm;
            Timed t(h, "resid_norm", st);
            HIP_TRY(launch_resid_norm(bf, part, p.down.splits, M, H, hbuf, next_gain, c.rms_eps, u,
                                      tap ? tap + (l + 1) * tap_stride : nullptr, st));
        }
    }
    {
        Timed t(h, bf ? "lm_head_bf16" : "lm_head_f32", st);
        const void* wlm = bf ? (const void*)(h->packed + h->pl.lm) : h->w.lm_head;
        HIP_TRY(launch_lm_head(bf, u, M, wlm, c.vocab, H, hpart, logits_out, sample, seed, st));
    }
    {
        Timed t(h, "head_merge", st);
        HIP_TRY(launch_head_merge(bf, M, c.vocab, top_k, sample, hpart, block_tokens, tokens, topk_ids,
                                  topk_logprobs, err, st));
    }
    return DFLASH_OK;
}

extern "C" int dflash_draft_block(dflash_handle* h, int batch, const int32_t* block_tokens, const int32_t* ctx_len,
                                  const int32_t* page_table, int max_pages, const dflash_kv* kv, int max_ctx,
                                  int top_k, int32_t* tokens, int32_t* topk_ids, float* topk_logprobs,
                                  const dflash_debug* dbg, void* ws, size_t ws_bytes, void* stream) {
    return draft_impl(h, batch, block_tokens, ctx_len, page_table, max_pages, kv, max_ctx, top_k, 0, 0, tokens,
                      topk_ids, topk_logprobs, dbg ? dbg->logits : nullptr, dbg, ws, ws_bytes, false, stream);
}

extern "C" int dflash_draft_block_noalloc(dflash_handle* h, int batch, const int32_t* block_tokens,
                                          const int32_t* ctx_len, const int32_t* page_table, int max_pages,
                                          const dflash_kv* kv, int max_ctx, int top_k, int32_t* tokens,
                                          int32_t* topk_ids, float* topk_logprobs, const dflash_debug* dbg,
                                          void* stream) {
    return draft_impl(h, batch, block_tokens, ctx_len, page_table, max_pages, kv, max_ctx, top_k, 0, 0, tokens,
                      topk_ids, topk_logprobs, dbg ? dbg->logits : nullptr, dbg, nullptr, 0, true, stream);
}

extern "C" int dflash_draft_block_sample(dflash_handle* h, int batch, const int32_t* block_tokens,
                                         const int32_t* ctx_len, const int32_t* page_table, int max_pages,
                                         const dflash_kv* kv, int max_ctx, int top_k, uint64_t seed, int32_t* tokens,
                                         int32_t* topk_ids, float* topk_logprobs, float* logits, void* ws,
                                         size_t ws_bytes, void* stream) {
    return draft_impl(h, batch, block_tokens, ctx_len, page_table, max_pages, kv, max_ctx, top_k, 1, seed, tokens,
                      topk_ids, topk_logprobs, logits, nullptr, ws, ws_bytes, false, stream);
}

// ---------------------------------------------------------------------------------------------------------
// dflash_inject_ctx
// ---------------------------------------------------------------------------------------------------------
extern "C" int dflash_inject_ctx(dflash_handle* h, int batch, int n_rows, const void* feats, int64_t feat_row_stride,
                                 const int32_t* row_offsets, const int32_t* start_pos, const int32_t* page_table,
                                 int max_pages, const dflash_kv* kv, void* ws, size_t ws_bytes, void* stream) {
    if (!h) return fail(DFLASH_E_ARG, "handle is NULL");
    const dflash_config& c = h->cfg;
    if (batch < 1 || n_rows < 1) return fail(DFLASH_E_ARG, "batch and n_rows must be >= 1");
    if (!feats || !row_offsets || !start_pos || !page_table || !kv || !kv->k || !kv->v || !ws)
        return fail(DFLASH_E_ARG, "a required pointer is NULL");
    if (feat_row_stride < c.feat_dim) return fail(DFLASH_E_ARG, "feat_row_stride < feat_dim");
    if (is_bf16(c) ? (feat_row_stride % 8) : (feat_row_stride % 4))
        return fail(DFLASH_E_ARG, "feat_row_stride must keep rows 16-byte aligned");
    if (max_pages < 1 || kv->n_pages < 1) return fail(DFLASH_E_ARG, "max_pages and n_pages must be >= 1");
    const InjectPlan p = plan_inject(c, n_rows, true);
    if (ws_bytes < p.total) return fail(DFLASH_E_CAPACITY, "workspace %zu < %zu bytes", ws_bytes, p.total);
    if (((uintptr_t)ws) & 255) return fail(DFLASH_E_ARG, "workspace must be 256-byte aligned");
    if (is_bf16(c) && !h->packed) return fail(DFLASH_E_ARG, "bfloat16 weights are not packed (dflash_pack_weights)");

    hipStream_t st = (hipStream_t)stream;
    const int bf = is_bf16(c);
    char* W = (char*)ws;
    uint32_t* err = (uint32_t*)(W + p.err);
    void* f = W + p.f;
    float* part = (float*)(W + p.part);
    const int H = c.hidden, kvd = c.n_kv_heads * c.head_dim;
    const size_t E = elt(c);
    for (int row0 = 0; row0 < n_rows; row0 += p.rows) {
        const int R = std::min(p.rows, n_rows - row0);
        const char* x = (const char*)feats + (size_t)row0 * feat_row_stride * E;
        const GemmPlan fc = plan_gemm(bf, R, H, c.feat_dim);
        {
            Timed t(h, gemm_kernel_name(fc, false), st, H, c.feat_dim);
            HIP_TRY(project(h, fc, x, (int)feat_row_stride, 0, R, h->pl.fc, segs1(h->w.fc_w, H), H, c.feat_dim, part,
                            st));
        }
        {
            Timed t(h, "fuse_cast", st);
            // the first chunk's cast also clears the device error word (kv_scatter is the first kernel to set it)
            HIP_TRY(launch_reduce_cast(bf, part, fc.splits, R, H, h->w.fc_b, f, row0 == 0 ? err : nullptr, st));
        }
        for (int l0 = 0; l0 < c.n_layers; l0 += MAX_LAYERS_PER_KV_GEMM) {
            const int nl = std::min(MAX_LAYERS_PER_KV_GEMM, c.n_layers - l0);
            Segs s{};
            for (int i = 0; i < nl; ++i) {
                s.ptr[2 * i] = h->layers[l0 + i].uk;
                s.ptr[2 * i + 1] = h->layers[l0 + i].uv;
                s.start[2 * i] = 2 * i * kvd;
                s.start[2 * i + 1] = (2 * i + 1) * kvd;
            }
            s.start[2 * nl] = 2 * nl * kvd;
            s.n = 2 * nl;
            const GemmPlan kp = plan_gemm(bf, R, 2 * nl * kvd, H);
            {
                Timed t(h, gemm_kernel_name(kp, bf), st, 2 * nl * kvd, H);
                HIP_TRY(project(h, kp, f, H, bf ? (size_t)R * H : 0, R, h->pl.kv + l0 * h->pl.kv_stride, s,
                                2 * nl * kvd, H, part, st));
            }
            {
                Timed t(h, "kv_scatter", st);
                HIP_TRY(launch_kv_scatter(bf, part, kp.splits, R, row0, l0, nl, c.n_kv_heads, c.head_dim, batch,
                                          row_offsets, start_pos, page_table, max_pages, kv->n_pages, kv->k, kv->v,
                                          h->rf, err, st));
            }
        }
    }
    return DFLASH_OK;
}

// ---------------------------------------------------------------------------------------------------------
// dflash_accept_len, building blocks
// ---------------------------------------------------------------------------------------------------------
extern "C" int dflash_accept_len(int batch, int n_draft, const int32_t* draft, int64_t draft_stride,
                                 const int32_t* target, int64_t target_stride, int32_t* tau, void* stream) {
    if (batch < 1 || n_draft < 0) return fail(DFLASH_E_ARG, "batch must be >= 1 and n_draft >= 0");
    if (!draft || !target || !tau) return fail(DFLASH_E_ARG, "a required pointer is NULL");
    if (draft_stride < n_draft || target_stride < n_draft) return fail(DFLASH_E_ARG, "stride smaller than n_draft");
    HIP_TRY(launch_accept(batch, n_draft, draft, draft_stride, target, target_stride, tau, (hipStream_t)stream));
    return DFLASH_OK;
}

#define VERIFY_MAX_DRAFT 63  // one lane per draft position in the acceptance tests

extern "C" size_t dflash_verify_sample_workspace_bytes(int batch, int n_draft, int vocab) {
    if (batch < 1 || n_draft < 0 || n_draft > VERIFY_MAX_DRAFT || vocab < 1) return 0;
    return sv_workspace_bytes(batch, n_draft, vocab);
}

extern "C" int dflash_verify_sample(int batch, int n_draft, int vocab, const int32_t* draft, int64_t draft_stride,
                                    const float* q_logits, int64_t q_req_stride, const float* p_logits,
                                    int64_t p_req_stride, uint64_t seed, int32_t* tau, int32_t* next_token, void* ws,
                                    size_t ws_bytes, void* stream) {
    if (batch < 1 || batch > 65535) return fail(DFLASH_E_ARG, "batch must be in [1, 65535]");
    if (n_draft < 0 || n_draft > VERIFY_MAX_DRAFT) return fail(DFLASH_E_UNSUPPORTED, "n_draft must be in [0, 63]");
    if (vocab < 1) return fail(DFLASH_E_ARG, "vocab must be >= 1");
    if (!p_logits || !tau || !next_token || !ws) return fail(DFLASH_E_ARG, "a required pointer is NULL");
    if (n_draft > 0 && (!draft || !q_logits)) return fail(DFLASH_E_ARG, "drafts or drafter logits are NULL");
    if (draft_stride < n_draft) return fail(DFLASH_E_ARG, "draft_stride < n_draft");
    if (p_req_stride < (int64_t)(n_draft + 1) * vocab) return fail(DFLASH_E_ARG, "p_req_stride < (n_draft + 1) * vocab");
    if (n_draft > 0 && q_req_stride < (int64_t)n_draft * vocab) return fail(DFLASH_E_ARG, "q_req_stride < n_draft * vocab");
    const size_t need = sv_workspace_bytes(batch, n_draft, vocab);
    if (ws_bytes < need) return fail(DFLASH_E_CAPACITY, "workspace %zu < %zu bytes", ws_bytes, need);
    if (((uintptr_t)ws) & 255) return fail(DFLASH_E_ARG, "workspace must be 256-byte aligned");
    HIP_TRY(launch_verify_sample(batch, n_draft, vocab, draft, draft_stride, q_logits, q_req_stride, p_logits,
                                 p_req_stride, seed, tau, next_token, ws, (hipStream_t)stream));
    return DFLASH_OK;
}

// Shape checks of the tree attention: DFLASH_OK, or the status and *msg.
static int tree_shape_check(int batch, int max_tokens, int nq, int nkv, int d, int max_ctx, const char** msg) {
    if (batch < 1 || batch > 65535) return *msg = "batch must be in [1, 65535]", DFLASH_E_ARG;
    if (max_tokens < 1 || max_tokens > TREE_MAX_TOKENS) return *msg = "max_tokens must be in [1, 2048]", DFLASH_E_ARG;
    if (max_ctx < 0) return *msg = "max_ctx must be >= 0", DFLASH_E_ARG;
    if (nkv < 1 || nq < 1 || nq % nkv) return *msg = "n_q_heads must be a multiple of n_kv_heads", DFLASH_E_ARG;
    if (d != 128) return *msg = "head_dim must be 128", DFLASH_E_UNSUPPORTED;
    const int G = nq / nkv;
    if (G != 1 && G != 2 && G != 4 && G != 8)
        return *msg = "n_q_heads / n_kv_heads must be 1, 2, 4 or 8", DFLASH_E_UNSUPPORTED;
    // the kernels index the context's 64-key rounds of every (request, token tile) in 32-bit arithmetic
    if ((long long)batch * ((max_tokens + 15) / 16) * ((max_ctx + 63) / 64 + 64) >= (1LL << 31))
        return *msg = "batch x tree tiles x context rounds is too large", DFLASH_E_UNSUPPORTED;
    return DFLASH_OK;
}

extern "C" size_t dflash_tree_attention_workspace_bytes(int batch, int max_tokens, int n_q_heads, int n_kv_heads,
                                                        int head_dim, int max_ctx) {
    const char* msg;
    if (tree_shape_check(batch, max_tokens, n_q_heads, n_kv_heads, head_dim, max_ctx, &msg) != DFLASH_OK) return 0;
    return plan_tree(batch, max_tokens, n_q_heads, n_kv_heads, max_ctx).total;
}

extern "C" int dflash_tree_attention(int batch, int max_tokens, const int32_t* n_tokens, const int32_t* parent,
                                     int n_q_heads, int n_kv_heads, int head_dim, const void* q, const void* k,
                                     const void* v, const void* k_pages, const void* v_pages, int n_pages,
                                     const int32_t* page_table, int max_pages, const int32_t* ctx_len, int max_ctx,
                                     float rope_theta, void* out, void* ws, size_t ws_bytes, void* stream) {
    const char* msg;
    if (const int code = tree_shape_check(batch, max_tokens, n_q_heads, n_kv_heads, head_dim, max_ctx, &msg))
        return fail(code, "%s", msg);
    if (!n_tokens || !parent || !q || !k || !v || !ctx_len || !out || !ws)
        return fail(DFLASH_E_ARG, "a required pointer is NULL");
    if (max_ctx > 0) {
        if (!k_pages || !v_pages || !page_table) return fail(DFLASH_E_ARG, "page table or KV pages are NULL");
        if (max_pages < 1 || n_pages < 1) return fail(DFLASH_E_ARG, "max_pages and n_pages must be >= 1");
        if ((long long)max_ctx > (long long)max_pages * 16)
            return fail(DFLASH_E_CAPACITY, "max_ctx %d exceeds max_pages * 16", max_ctx);
        if ((((uintptr_t)k_pages) | ((uintptr_t)v_pages)) & 15) return fail(DFLASH_E_ARG, "KV pages must be 16-byte aligned");
    }
    if (!(rope_theta >= 0.f)) return fail(DFLASH_E_ARG, "rope_theta must be >= 0");
    if ((((uintptr_t)q) | ((uintptr_t)k) | ((uintptr_t)v) | ((uintptr_t)out)) & 15)
        return fail(DFLASH_E_ARG, "q, k, v and out must be 16-byte aligned");
    const TreePlan p = plan_tree(batch, max_tokens, n_q_heads, n_kv_heads, max_ctx);
    if (ws_bytes < p.total) return fail(DFLASH_E_CAPACITY, "workspace %zu < %zu bytes", ws_bytes, p.total);
    if (((uintptr_t)ws) & 255) return fail(DFLASH_E_ARG, "workspace must be 256-byte aligned");
    RopeFreq rf{};
    rf.on = rope_theta > 0.f;  // theta = 0: no rotation
    for (int i = 0; i < head_dim / 2; ++i)  // theta^(-2i/d) in double, rounded to float
        rf.inv[i] = rf.on ? (float)std::pow((double)rope_theta, -(2.0 * i) / head_dim) : 0.f;
    HIP_TRY(launch_tree_attention(p, batch, max_tokens, n_tokens, parent, n_q_heads, n_kv_heads, q, k, v, k_pages,
                                  v_pages, n_pages, page_table, max_pages, ctx_len, max_ctx, rf, out, ws,
                                  (hipStream_t)stream));
    return DFLASH_OK;
}

// Workspace of dflash_linear: the float32 split partials, then (bfloat16) the packed image of w.
static size_t linear_part_bytes(int dtype, int M, int N, int K) {
    const GemmPlan p = plan_gemm(dtype == DFLASH_BF16, M, N, K);
    return align256((size_t)p.splits * M * N * 4);
}

extern "C" size_t dflash_linear_workspace_bytes(int dtype, int M, int N, int K) {
    if ((dtype != DFLASH_F32 && dtype != DFLASH_BF16) || M < 1 || N < 1 || K < 1) return 0;
    const size_t part = linear_part_bytes(dtype, M, N, K);
    return dtype == DFLASH_BF16 ? part + align256(packed_elems(N, K) * 2) : part;
}

extern "C" int dflash_linear(int dtype, int M, int N, int K, const void* x, int64_t ldx, const void* w, float* y,
                             void* ws, size_t ws_bytes, void* stream) {
    if (dtype != DFLASH_F32 && dtype != DFLASH_BF16) return fail(DFLASH_E_ARG, "unknown dtype");
    if (M < 1 || N < 1 || K < 1) return fail(DFLASH_E_ARG, "sizes must be positive");
    if (!x || !w || !y || !ws) return fail(DFLASH_E_ARG, "a required pointer is NULL");
    if (ldx < K) return fail(DFLASH_E_ARG, "ldx < K");
    if (dtype == DFLASH_BF16 && (K % 256 || ldx % 8)) return fail(DFLASH_E_UNSUPPORTED, "bf16 needs K % 256 == 0");
    if (dtype == DFLASH_F32 && (K % 4 || ldx % 4)) return fail(DFLASH_E_UNSUPPORTED, "f32 needs K % 4 == 0");
    if (ws_bytes < dflash_linear_workspace_bytes(dtype, M, N, K)) return fail(DFLASH_E_CAPACITY, "workspace too small");
    if ((((uintptr_t)x) | ((uintptr_t)w) | ((uintptr_t)ws)) & 15)
        return fail(DFLASH_E_ARG, "x, w and the workspace must be 16-byte aligned");
    const GemmPlan p = plan_gemm(dtype == DFLASH_BF16, M, N, K);
    hipStream_t st = (hipStream_t)stream;
    if (dtype == DFLASH_BF16) {
        void* wpk = (char*)ws + linear_part_bytes(dtype, M, N, K);
        HIP_TRY(launch_pack(stack_rows({{w, N}}), N, K, wpk, st));
        HIP_TRY(launch_gemm_bf16(p, x, (int)ldx, 0, M, wpk, N, K, (float*)ws, st));
    } else {
        HIP_TRY(launch_gemm_f32((const float*)x, (int)ldx, M, segs1(w, N), N, K, (float*)ws, st));
    }
    HIP_TRY(launch_reduce_cast(0, (float*)ws, p.splits, M, N, nullptr, y, nullptr, st));
    return DFLASH_OK;
}

// ---------------------------------------------------------------------------------------------------------
// DDTree: wide top-K, tree construction, verifier walk
// ---------------------------------------------------------------------------------------------------------
#define DDT_MAX_K 1024
#define DDT_MAX_DEPTH 16
#define DDT_MAX_BUDGET 2047

extern "C" size_t dflash_topk_logprobs_workspace_bytes(int rows, int vocab, int k) {
    if (rows < 1 || vocab < 1 || k < 1 || k > vocab || k > DDT_MAX_K) return 0;
    return topk_workspace_bytes(rows, vocab, k);
}

extern "C" int dflash_topk_logprobs(int rows, int vocab, int k, const float* logits, int64_t row_stride,
                                    int32_t* ids, float* logprobs, void* workspace, size_t workspace_bytes,
                                    void* stream) {
    if (rows < 1 || vocab < 1) return fail(DFLASH_E_ARG, "rows and vocab must be >= 1");
    if (!logits || !ids || !logprobs) return fail(DFLASH_E_ARG, "a required pointer is NULL");
    if (k < 1 || k > vocab) return fail(DFLASH_E_ARG, "k must be in [1, vocab]");
    if (k > DDT_MAX_K) return fail(DFLASH_E_UNSUPPORTED, "k must be <= %d", DDT_MAX_K);
    if (row_stride < vocab) return fail(DFLASH_E_ARG, "row_stride < vocab");
    const size_t need = topk_workspace_bytes(rows, vocab, k);
    if (need && (!workspace || workspace_bytes < need))
        return fail(DFLASH_E_ARG, "workspace of %zu bytes needed", need);
    if (need && ((uintptr_t)workspace & 15)) return fail(DFLASH_E_ARG, "workspace must be 16-byte aligned");
    HIP_TRY(launch_topk_rows(rows, logits, row_stride, vocab, k, ids, logprobs, workspace, (hipStream_t)stream));
    return DFLASH_OK;
}

static int ddtree_build_impl(int batch, int depth, int k, const float* logprobs, const int32_t* ids,
                             int64_t req_stride, int budget, int32_t* node_token, int32_t* node_parent,
                             int32_t* node_depth, float* node_logq, int32_t* n_nodes, bool select_only,
                             void* stream) {
    if (batch < 1) return fail(DFLASH_E_ARG, "batch must be >= 1");
    if (!logprobs || !ids || !node_token || !node_parent || !node_depth || !node_logq || !n_nodes)
        return fail(DFLASH_E_ARG, "a required pointer is NULL");
    if (depth < 1 || k < 1 || budget < 1) return fail(DFLASH_E_ARG, "depth, k and budget must be >= 1");
    if (depth > DDT_MAX_DEPTH || k > DDT_MAX_K || budget > DDT_MAX_BUDGET)
        return fail(DFLASH_E_UNSUPPORTED, "depth <= %d, k <= %d and budget <= %d", DDT_MAX_DEPTH, DDT_MAX_K,
                    DDT_MAX_BUDGET);
    if (req_stride < (int64_t)depth * k) return fail(DFLASH_E_ARG, "req_stride < depth * k");
    HIP_TRY(launch_ddtree_build(batch, depth, k, logprobs, ids, req_stride, budget, node_token, node_parent,
                                node_depth, node_logq, n_nodes, select_only, (hipStream_t)stream));
    return DFLASH_OK;
}

extern "C" int dflash_ddtree_build(int batch, int depth, int k, const float* logprobs, const int32_t* ids,
                                   int64_t req_stride, int budget, int32_t* node_token, int32_t* node_parent,
                                   int32_t* node_depth, float* node_logq, int32_t* n_nodes, void* stream) {
    return ddtree_build_impl(batch, depth, k, logprobs, ids, req_stride, budget, node_token, node_parent,
                             node_depth, node_logq, n_nodes, false, stream);
}

extern "C" int dflash_ddtree_select(int batch, int depth, int k, const float* logprobs, const int32_t* ids,
                                    int64_t req_stride, int budget, int32_t* node_token, int32_t* node_parent,
                                    int32_t* node_depth, float* node_logq, int32_t* n_nodes, void* stream) {
    return ddtree_build_impl(batch, depth, k, logprobs, ids, req_stride, budget, node_token, node_parent,
                             node_depth, node_logq, n_nodes, true, stream);
}

extern "C" int dflash_ddtree_walk(int batch, int budget, int max_accept, const int32_t* node_token,
                                  const int32_t* node_parent, const int32_t* n_nodes, const int32_t* target_next,
                                  int32_t* accept_len, int32_t* accept_nodes, int32_t* bonus, void* stream) {
    if (batch < 1 || budget < 1 || max_accept < 1) return fail(DFLASH_E_ARG, "batch, budget and max_accept must be >= 1");
    if (budget > DDT_MAX_BUDGET) return fail(DFLASH_E_UNSUPPORTED, "budget must be <= %d", DDT_MAX_BUDGET);
    if (!node_token || !node_parent || !n_nodes || !target_next || !accept_len || !accept_nodes || !bonus)
        return fail(DFLASH_E_ARG, "a required pointer is NULL");
    HIP_TRY(launch_ddtree_walk(batch, budget, max_accept, node_token, node_parent, n_nodes, target_next, accept_len,
                               accept_nodes, bonus, (hipStream_t)stream));
    return DFLASH_OK;
}

extern "C" int dflash_copy(void* dst, const void* src, size_t n_bytes, void* stream) {
    if (!dst || !src) return fail(DFLASH_E_ARG, "a required pointer is NULL");
    if ((n_bytes & 15) || (((uintptr_t)dst | (uintptr_t)src) & 15))
        return fail(DFLASH_E_ARG, "n_bytes and pointers must be multiples of 16");
    HIP_TRY(launch_copy(dst, src, n_bytes / 16, (hipStream_t)stream));
    return DFLASH_OK;
}
