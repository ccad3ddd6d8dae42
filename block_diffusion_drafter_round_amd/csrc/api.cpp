// libdflash C ABI: argument checks, workspace layout and the launch sequence
// of each call.  See include/dflash.h for the contract.
//
// Pages: [DflashDraft] (docs.rs memra_engine::dflash::DflashDraft) sections
// "ctx_features", "forward", "ingest_ctx", "forward_round", "rope_yarn";
// [memra dflash module] "DflashKv"; [atlas dflash_head] "DflashScratch".
#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>
#include <mutex>
#include <vector>

#include "dflash.h"
#include "dflash_policy.h"
#include "dflash_prof.h"
#include "batch.h"
#include "kernels.h"
#include "sround.h"

struct dflash_model {
    dflash_cfg cfg;
    dflash_weights w;
    std::vector<dflash_layer_weights> layers;
    double inv_freq[dfl::MAX_HALF_DIM];
    double mscale;
    char *pk;            // packed GEMM weight stream (dflash_pack_weights), borrowed
    int pk_nwg;          // round-kernel workgroups the stream was packed for
    long long pk_layer;  // bytes of one layer's stream
};

namespace {

thread_local std::string g_err;

int fail(int code, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
    return code;
}

int hip_fail(hipError_t e, const char *where) {
    return fail(DFLASH_E_HIP, "%s: %s", where, hipGetErrorString(e));
}

// ---- measurement hook: HIP events around the launches of one kernel class ----
struct Prof {
    std::mutex mu;
    std::atomic<int> cls{0};
    std::vector<hipEvent_t> ev;   // start, stop pairs
    int used = 0, cap = 0;
} g_prof;
std::atomic<int> g_trace{0};

struct ProfScope {
    int idx = -1;
    hipStream_t s;
    ProfScope(int cls, hipStream_t st) : s(st) {
        if (g_prof.cls.load(std::memory_order_relaxed) != cls) return;
        std::lock_guard<std::mutex> lk(g_prof.mu);
        if (g_prof.cls.load() != cls || g_prof.used >= g_prof.cap) return;
        idx = g_prof.used++;
        hipEventRecord(g_prof.ev[2 * idx], s);
    }
    ~ProfScope() {
        if (idx >= 0) hipEventRecord(g_prof.ev[2 * idx + 1], s);
    }
};

bool aligned(const void *p, size_t a) { return p && (reinterpret_cast<uintptr_t>(p) % a) == 0; }

constexpr int MAX_BLOCK = 16;
constexpr int MAX_ATTN_SPLITS = 64;

size_t align256(size_t x) { return (x + 255) / 256 * 256; }

struct WsLayout {
    size_t gcnt, gpart, ctr, trace, cs, xsave, lay, lay_stride, qkv, feats, total;
    dfl::SrLayout sl;
};

// ingest_ctx projects up to INGEST_FUSE_ROWS / t layers' k|v in one GEMM
// (at most GEMM_MAX_SEG / 2 and ROPE_MAX_LAYERS): few new rows make a skinny,
// latency-bound GEMM per layer, and many rows a GEMM that fills the device
// only with several layers' columns (1024 rows x 5 layers: 640 tiles of the
// tiled kernel, against 128 per layer), so the layers share one launch.  The
// staging buffer holds INGEST_FUSE_ROWS rows of one layer's k|v.
constexpr size_t INGEST_FUSE_ROWS = 8192;

int ingest_layers_per_launch(int t) {
    const int n = t > 0 ? (int)(INGEST_FUSE_ROWS / (size_t)t) : 1;
    return std::max(1, std::min({n, dfl::GEMM_MAX_SEG / 2, dfl::ROPE_MAX_LAYERS}));
}

// workgroups the round kernel is laid out for at most (partial sums of
// squares are stored per workgroup)
constexpr int WS_MAX_NWG = 256;

WsLayout ws_layout(const dflash_cfg &c, int max_rows) {
    const size_t H = c.hidden, kvd = (size_t)c.n_kv_heads * c.head_dim;
    const size_t rows = (size_t)(max_rows > MAX_BLOCK ? max_rows : MAX_BLOCK);
    WsLayout L{};
    size_t off = 0;
    auto take = [&](size_t bytes) { size_t o = off; off += align256(bytes); return o; };
    // fixed-size regions first, so their offsets do not depend on max_rows
    L.gcnt = take(sizeof(unsigned) * dfl::GEMM_MAX_COUNTERS);
    L.gpart = take(4 * dfl::GEMM_PART_FLOATS);
    L.ctr = take(sizeof(unsigned) * dfl::SR_CTR_WORDS);
    L.trace = take(8 * dfl::SR_TRACE);
    L.cs = take(4 * (size_t)MAX_BLOCK * c.head_dim);
    L.xsave = take(4 * (size_t)MAX_BLOCK * H);
    L.sl = dfl::sround_layout(c.hidden, c.intermediate, c.n_q_heads * c.head_dim, (int)kvd, c.n_kv_heads,
                              c.n_q_heads / c.n_kv_heads, c.head_dim, c.weight_dtype, WS_MAX_NWG, c.d2_groups);
    L.lay_stride = (size_t)L.sl.stride;
    L.lay = take(L.lay_stride * (dfl::SR_MAXL + 1));
    // row-dependent regions
    L.qkv = take(4 * std::max<size_t>(rows, INGEST_FUSE_ROWS) * 2 * kvd);
    L.feats = take(4 * rows * H);
    L.total = off;
    return L;
}

int wtype(const dflash_cfg &c) { return c.weight_dtype; }

int check_matrix(const dflash_cfg &c, const dflash_matrix &m, const char *name, int layer) {
    if (!aligned(m.data, 16)) return fail(DFLASH_E_INVAL, "layer %d %s: data pointer null or not 16-byte aligned", layer, name);
    if (c.weight_dtype == DFLASH_FP8_E4M3) {
        if (!aligned(m.scale, 4)) return fail(DFLASH_E_INVAL, "layer %d %s: fp8 weights need a row-scale pointer", layer, name);
    } else if (m.scale) {
        return fail(DFLASH_E_INVAL, "layer %d %s: scale given for non-fp8 weights", layer, name);
    }
    return DFLASH_OK;
}

int check_vec(const float *p, const char *name, int layer) {
    if (!aligned(p, 16)) return fail(DFLASH_E_INVAL, "layer %d %s: gain pointer null or not 16-byte aligned", layer, name);
    return DFLASH_OK;
}

int check_cfg(const dflash_cfg &c) {
    if (c.n_layers < 0 || c.n_layers > 4096) return fail(DFLASH_E_INVAL, "n_layers %d out of range", c.n_layers);
    if (c.hidden <= 0 || c.hidden % 256) return fail(DFLASH_E_UNSUPPORTED, "hidden %d must be a positive multiple of 256", c.hidden);
    if (c.intermediate <= 0 || c.intermediate % 256)
        return fail(DFLASH_E_UNSUPPORTED, "intermediate %d must be a positive multiple of 256", c.intermediate);
    if (c.head_dim != 64 && c.head_dim != 128) return fail(DFLASH_E_UNSUPPORTED, "head_dim %d: only 64 and 128 are built", c.head_dim);
    if (c.n_q_heads <= 0 || c.n_kv_heads <= 0 || c.n_q_heads % c.n_kv_heads)
        return fail(DFLASH_E_INVAL, "n_q_heads %d must be a positive multiple of n_kv_heads %d", c.n_q_heads, c.n_kv_heads);
    if (c.n_q_heads / c.n_kv_heads > dfl::SR_MAXG)
        return fail(DFLASH_E_UNSUPPORTED, "more than %d q heads per kv head", dfl::SR_MAXG);
    if ((c.n_q_heads * c.head_dim) % 256) return fail(DFLASH_E_UNSUPPORTED, "n_q_heads*head_dim must be a multiple of 256");
    if (c.n_taps <= 0 || ((size_t)c.n_taps * c.hidden) % 256) return fail(DFLASH_E_INVAL, "n_taps %d invalid", c.n_taps);
    if (!(c.rms_eps > 0.f) || !std::isfinite(c.rms_eps)) return fail(DFLASH_E_INVAL, "rms_eps must be positive");
    if (!(c.rope_base > 1.0) || !std::isfinite(c.rope_base)) return fail(DFLASH_E_INVAL, "rope_base must be > 1");
    if (c.rope_type == DFLASH_ROPE_YARN) {
        if (!(c.yarn_factor >= 1.0) || c.yarn_orig_ctx <= 0 || !(c.yarn_beta_fast > 0) || !(c.yarn_beta_slow > 0))
            return fail(DFLASH_E_INVAL, "bad YaRN parameters");
    } else if (c.rope_type != DFLASH_ROPE_PLAIN) {
        return fail(DFLASH_E_INVAL, "unknown rope_type %d", c.rope_type);
    }
    const bool ok_types = (c.weight_dtype == DFLASH_F32 && c.kv_dtype == DFLASH_F32) ||
                          (c.weight_dtype == DFLASH_BF16 && c.kv_dtype == DFLASH_BF16) ||
                          (c.weight_dtype == DFLASH_FP8_E4M3 && c.kv_dtype == DFLASH_BF16);
    if (!ok_types) return fail(DFLASH_E_UNSUPPORTED, "weight/kv dtype combination %d/%d not built", c.weight_dtype, c.kv_dtype);
    if (c.kv_dtype == DFLASH_F32 && c.head_dim != 64) return fail(DFLASH_E_UNSUPPORTED, "an f32 KV cache is built for head_dim 64 only");
    if (c.d2_groups < 0) return fail(DFLASH_E_INVAL, "d2_groups must be >= 0");
    if (c.d2_groups > 0) {
        if (c.d2_groups > dfl::SR_MAX_D2 || c.hidden % c.d2_groups || (c.hidden / c.d2_groups) % 16)
            return fail(DFLASH_E_UNSUPPORTED, "d2_groups %d: built for G <= %d with hidden/G a multiple of 16",
                        c.d2_groups, dfl::SR_MAX_D2);
    }
    if (dfl::sround_nwg(c.hidden, c.intermediate, c.n_q_heads * c.head_dim, c.n_kv_heads * c.head_dim, c.weight_dtype,
                        c.d2_groups, WS_MAX_NWG) <= 0)
        return fail(DFLASH_E_UNSUPPORTED, "no workgroup layout of the round kernel fits these dimensions");
    return DFLASH_OK;
}

// YaRN frequency remap (Peng et al., "YaRN", 2023): dimension pairs that
// turn fewer than beta_slow times over the original context are divided by
// the factor, pairs that turn more than beta_fast times keep their
// frequency, and a linear ramp over the pair index blends the two.
void rope_table(const dflash_cfg &c, double *inv_freq, double *mscale) {
    const int half = c.head_dim / 2;
    const double base = c.rope_base, d = c.head_dim;
    for (int j = 0; j < half; ++j) inv_freq[j] = std::pow(base, -2.0 * j / d);
    *mscale = 1.0;
    if (c.rope_type != DFLASH_ROPE_YARN) return;
    const double L0 = c.yarn_orig_ctx, f = c.yarn_factor;
    auto pair_index = [&](double turns) { return d * std::log(L0 / (2.0 * M_PI * turns)) / (2.0 * std::log(base)); };
    double lo = std::floor(pair_index(c.yarn_beta_fast));
    double hi = std::ceil(pair_index(c.yarn_beta_slow));
    if (lo < 0) lo = 0;
    if (hi > d - 1) hi = d - 1;
    if (hi == lo) hi = lo + 0.001;
    for (int j = 0; j < half; ++j) {
        double ramp = (j - lo) / (hi - lo);
        ramp = ramp < 0 ? 0 : ramp > 1 ? 1 : ramp;
        inv_freq[j] *= ramp / f + (1.0 - ramp);
    }
    *mscale = 0.1 * std::log(f) + 1.0;
}

size_t kv_elem(const dflash_cfg &c) { return c.kv_dtype == DFLASH_F32 ? 4 : 2; }

int check_kv(const dflash_model *m, const dflash_kv *kv) {
    if (!kv) return fail(DFLASH_E_INVAL, "kv is null");
    if (!aligned(kv->k, 16) || !aligned(kv->v, 16)) return fail(DFLASH_E_INVAL, "kv->k / kv->v null or not 16-byte aligned");
    if (kv->capacity <= 0 || kv->capacity % 64) return fail(DFLASH_E_INVAL, "kv capacity %d must be a positive multiple of 64", kv->capacity);
    if (kv->len < 0 || kv->len > kv->capacity) return fail(DFLASH_E_INVAL, "kv len %d outside [0, capacity]", kv->len);
    if (kv->ctx_cap < 0) return fail(DFLASH_E_INVAL, "kv ctx_cap %d is negative", kv->ctx_cap);
    if (kv->page_rows < 0) return fail(DFLASH_E_INVAL, "kv page_rows %d is negative", kv->page_rows);
    if (kv->page_rows > 0) {
        if (kv->page_rows % 64 || kv->capacity % kv->page_rows)
            return fail(DFLASH_E_INVAL, "kv page_rows %d must be a multiple of 64 that divides capacity %d", kv->page_rows,
                        kv->capacity);
        if (kv->pool_pages < 1) return fail(DFLASH_E_INVAL, "paged kv needs pool_pages >= 1");
        if (!aligned(kv->block_table, 4)) return fail(DFLASH_E_INVAL, "paged kv needs a block table");
        const size_t pool = (size_t)kv->pool_pages * m->cfg.n_kv_heads * kv->page_rows * m->cfg.head_dim;
        if (pool * 4 > ((size_t)1 << 40)) return fail(DFLASH_E_INVAL, "paged kv pool of %d pages is too large", kv->pool_pages);
    }
    return DFLASH_OK;
}

// the kernels' view of a cache (kvview.h): a contiguous cache is one page
dfl::KvView kv_view(const dflash_model *m, const dflash_kv *kv) {
    const dflash_cfg &c = m->cfg;
    dfl::KvView v{};
    v.k = static_cast<char *>(kv->k);
    v.v = static_cast<char *>(kv->v);
    v.esize = (int)kv_elem(c);
    if (kv->page_rows > 0) {
        v.page_rows = kv->page_rows;
        v.pool_pages = kv->pool_pages;
        v.table = kv->block_table;
    } else {
        v.page_rows = kv->capacity;
        v.pool_pages = 1;
        v.table = nullptr;
    }
    v.lstride = (long long)v.pool_pages * c.n_kv_heads * v.page_rows * c.head_dim * v.esize;
    return v;
}

// first committed row a round attends ([atlas dflash_head] "dflash_ctx_cap")
int window_lo(const dflash_kv *kv) { return kv->ctx_cap > 0 && kv->len > kv->ctx_cap ? kv->len - kv->ctx_cap : 0; }

// a cache the persistent round kernel cannot serve: paged, or with a window
bool needs_layered(const dflash_kv *kv) { return kv->page_rows > 0 || kv->ctx_cap > 0; }

int check_ws(const dflash_model *m, void *ws, size_t ws_bytes, int rows) {
    if (!aligned(ws, 256)) return fail(DFLASH_E_INVAL, "workspace null or not 256-byte aligned");
    const size_t need = ws_layout(m->cfg, rows).total;
    if (ws_bytes < need) return fail(DFLASH_E_INVAL, "workspace of %zu bytes is smaller than the %zu needed for %d rows", ws_bytes, need, rows);
    return DFLASH_OK;
}

template <class T>
T *at(void *ws, size_t off) { return reinterpret_cast<T *>(static_cast<char *>(ws) + off); }

void *layer_ptr(void *base, const dflash_cfg &c, int cap, int l) {
    return static_cast<char *>(base) + (size_t)l * c.n_kv_heads * cap * c.head_dim * kv_elem(c);
}

dfl::GemmSeg seg(const dflash_matrix &m, int n) { return dfl::GemmSeg{m.data, m.scale, n}; }

// ---- launch sequences (arguments already checked) ---------------------------

// fc GEMM (split-K partials in `part`, counters in `cnt`) + hidden_norm
hipError_t run_ctx_features(const dflash_model *m, const float *taps, int t, float *feats, float *part, unsigned *cnt,
                            hipStream_t s) {
    const dflash_cfg &c = m->cfg;
    dfl::GemmArgs g{};
    g.A = taps; g.lda = c.n_taps * c.hidden; g.M = t; g.K = c.n_taps * c.hidden;
    g.seg[0] = seg(m->w.fc, c.hidden); g.nseg = 1;
    g.Y = feats; g.ldy = c.hidden; g.epi = dfl::EPI_STORE; g.wtype = wtype(c);
    hipError_t e;
    {
        ProfScope p(DFLASH_K_GEMM_FC, s);
        e = dfl::gemm(g, part, cnt, s);
    }
    if (e != hipSuccess) return e;
    ProfScope p(DFLASH_K_NORM, s);
    return dfl::rmsnorm(feats, c.hidden, m->w.g_hidden_norm, feats, c.hidden, nullptr, t, c.hidden, c.rms_eps, s);
}

// ingest of t rows into each of S caches (feats / pos: S blocks of t rows)
hipError_t run_ingest(const dflash_model *m, const dflash_kv *kvs, int S, const float *feats, const int32_t *pos, int t,
                      void *ws, const WsLayout &L, hipStream_t s) {
    const dflash_cfg &c = m->cfg;
    const int kvd = c.n_kv_heads * c.head_dim;
    const int rows = S * t;
    const int per = ingest_layers_per_launch(rows);
    float *kvbuf = at<float>(ws, L.qkv);
    for (int l0 = 0; l0 < c.n_layers; l0 += per) {
        const int nl = std::min(per, c.n_layers - l0);
        // k|v of layers l0 .. l0 + nl - 1 side by side: [t][nl * 2 * kvd]
        dfl::GemmArgs g{};
        g.A = feats; g.lda = c.hidden; g.M = rows; g.K = c.hidden;
        for (int i = 0; i < nl; ++i) {
            const dflash_layer_weights &W = m->layers[l0 + i];
            g.seg[2 * i] = seg(W.wk, kvd);
            g.seg[2 * i + 1] = seg(W.wv, kvd);
        }
        g.nseg = 2 * nl;
        g.Y = kvbuf; g.ldy = nl * 2 * kvd; g.epi = dfl::EPI_STORE; g.wtype = wtype(c);
        hipError_t e;
        {
            ProfScope p(DFLASH_K_GEMM_KV, s);
            e = dfl::gemm(g, at<float>(ws, L.gpart), at<unsigned>(ws, L.gcnt), s);
        }
        if (e != hipSuccess) return e;
        dfl::RopeArgs r{};
        r.src = kvbuf; r.ld = nl * 2 * kvd; r.lstride = 2 * kvd; r.nl = nl; r.layer0 = l0;
        for (int i = 0; i < nl; ++i) r.g_k[i] = m->layers[l0 + i].g_k;
        for (int q = 0; q < S; ++q) {
            r.kv[q] = kv_view(m, &kvs[q]);
            r.row0[q] = kvs[q].len;
        }
        r.seq_rows = t;
        r.pos = pos; r.rows = rows; r.nkv = c.n_kv_heads; r.d = c.head_dim; r.eps = c.rms_eps;
        r.mscale = (float)m->mscale; r.kv_f32 = c.kv_dtype == DFLASH_F32;
        memcpy(r.inv_freq, m->inv_freq, sizeof r.inv_freq);
        {
            ProfScope p(DFLASH_K_ROPE, s);
            e = dfl::kv_norm_rope(r, s);
        }
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

int device_cus() {
    static int cus[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
    if (!cus[dev]) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
        cus[dev] = n;
    }
    return cus[dev];
}

dfl::SrMat smat(const dflash_matrix &m) { return dfl::SrMat{m.data, m.scale}; }

// round-kernel workgroups on the current device, or <= 0
int round_nwg(const dflash_cfg &c) {
    return dfl::sround_nwg(c.hidden, c.intermediate, c.n_q_heads * c.head_dim, c.n_kv_heads * c.head_dim, c.weight_dtype,
                           c.d2_groups, std::min(device_cus(), WS_MAX_NWG));
}

long long pack_layer_bytes(const dflash_cfg &c, int nwg) {
    return dfl::sround_pack_layer_bytes(c.hidden, c.intermediate, c.n_q_heads * c.head_dim, c.n_kv_heads * c.head_dim,
                                        c.weight_dtype, c.d2_groups, nwg);
}

// the round kernel's dimensions and the pointers of layers [l0, l0 + nl)
void fill_round_args(const dflash_model *m, int nwg, int l0, int nl, dfl::SrArgs &ra) {
    const dflash_cfg &c = m->cfg;
    dfl::SrScalars &a = ra.s;
    const int qd = c.n_q_heads * c.head_dim, kvd = c.n_kv_heads * c.head_dim;
    a.H = c.hidden; a.I = c.intermediate; a.nq = c.n_q_heads; a.nkv = c.n_kv_heads; a.d = c.head_dim;
    a.qd = qd; a.kvd = kvd; a.G = c.n_q_heads / c.n_kv_heads; a.d2 = c.d2_groups;
    a.nwg = nwg; a.cq = (qd + 2 * kvd) / nwg; a.ch = c.hidden / nwg; a.ci = c.intermediate / nwg;
    a.nl = nl;
    a.first = l0 == 0;
    a.last = l0 + nl == c.n_layers;
    for (int i = 0; i < nl; ++i) {
        const dflash_layer_weights &W = m->layers[l0 + i];
        dfl::SrLayer &R = ra.L[i];
        R.q = smat(W.wq); R.k = smat(W.wk); R.v = smat(W.wv); R.o = smat(W.wo);
        R.g = smat(W.wg); R.u = smat(W.wu); R.d = smat(W.wd);
        R.g_in = W.g_in; R.g_post = W.g_post; R.g_q = W.g_q; R.g_k = W.g_k;
        if (c.d2_groups > 0) {
            R.aw = smat(W.attn_w_dyn); R.mw = smat(W.mlp_w_dyn);
            R.abase = W.attn_base; R.mbase = W.mlp_base;
        }
        R.pk = m->pk ? m->pk + (long long)(l0 + i) * m->pk_layer : nullptr;
    }
}

// the packed stream must exist and match the current device's launch shape
int check_packed(const dflash_model *m) {
    if (!m->pk) return fail(DFLASH_E_INVAL, "weights not packed: call dflash_pack_weights first");
    const int nwg = round_nwg(m->cfg);
    if (nwg != m->pk_nwg)
        return fail(DFLASH_E_INVAL, "weights packed for %d workgroups, this device runs %d: pack again", m->pk_nwg, nwg);
    return DFLASH_OK;
}

// forward_round: the streamed round kernel, one launch per SR_MAXL layers
hipError_t run_round(const dflash_model *m, const dflash_kv *kv, const float *noise, const int32_t *pos, int b, float *out,
                     void *ws, const WsLayout &L, hipStream_t s) {
    const dflash_cfg &c = m->cfg;
    const int nwg = round_nwg(c);
    if (nwg <= 0 || nwg != m->pk_nwg) return hipErrorInvalidDevice;
    dfl::SrArgs ra{};
    dfl::SrScalars &a = ra.s;
    a.b = b; a.len = kv->len; a.cap = kv->capacity;
    // attention key splits: at most one item per workgroup; one split per
    // kv head for the block's own keys, the others runs of whole 32-key
    // blocks of the cache (the kernel spreads the blocks evenly)
    a.nkb = (kv->len + 31) / 32;
    a.nsplit = std::max(1, std::min({dfl::SR_MAX_SPLITS, nwg / c.n_kv_heads, a.nkb + 1}));
    a.eps = c.rms_eps; a.mscale = (float)m->mscale;
    a.qscale = (float)(1.4426950408889634 / std::sqrt((double)c.head_dim));
    a.noise = noise; a.pos = pos; a.out = out; a.g_norm = m->w.g_norm;
    a.kv_lstride = (long long)c.n_kv_heads * kv->capacity * c.head_dim * (long long)kv_elem(c);
    a.ctr = at<unsigned>(ws, L.ctr);
    a.cs = at<float>(ws, L.cs);
    a.xsave = at<float>(ws, L.xsave);
    a.lay = at<char>(ws, L.lay);
    a.lay_stride = (long long)L.lay_stride;
    a.o_xa = L.sl.xa; a.o_ssa = L.sl.ssa; a.o_qkv = L.sl.qkv; a.o_po = L.sl.po; a.o_pml = L.sl.pml;
    a.o_of = L.sl.of; a.o_xm = L.sl.xm; a.o_ssm = L.sl.ssm; a.o_zf = L.sl.zf; a.o_da = L.sl.da; a.o_dm = L.sl.dm;
    a.trace = g_trace.load() ? at<unsigned long long>(ws, L.trace) : nullptr;
    memcpy(ra.inv_freq, m->inv_freq, sizeof ra.inv_freq);
    int l0 = 0;
    do {
        const int nl = std::min(dfl::SR_MAXL, c.n_layers - l0);
        fill_round_args(m, nwg, l0, nl, ra);
        a.kc = static_cast<char *>(layer_ptr(kv->k, c, kv->capacity, l0));
        a.vc = static_cast<char *>(layer_ptr(kv->v, c, kv->capacity, l0));
        hipError_t e;
        {
            ProfScope p(DFLASH_K_ROUND, s);
            e = dfl::sround_launch(ra, c.weight_dtype, nwg, s);
        }
        if (e != hipSuccess) return e;
        l0 += nl;
    } while (l0 < c.n_layers);
    return hipSuccess;
}

// ---- the layered round path (batched sequences, paged or windowed caches) ----

struct BatchLayout {
    size_t x, xn, qkv, q, po, pml, attn, z, xc, y, dc, bytes;
};

// buffers of the layered path for up to S sequences of MAX_BLOCK rows,
// relative to the start of its region
BatchLayout batch_layout(const dflash_cfg &c, int S) {
    const size_t rows = (size_t)S * MAX_BLOCK, H = c.hidden, qd = (size_t)c.n_q_heads * c.head_dim;
    const size_t kvd = (size_t)c.n_kv_heads * c.head_dim, G = (size_t)(c.n_q_heads / c.n_kv_heads);
    BatchLayout B{};
    size_t off = 0;
    auto take = [&](size_t bytes) { size_t o = off; off += align256(bytes); return o; };
    B.x = take(4 * rows * H);
    B.xn = take(4 * rows * H);
    B.qkv = take(4 * rows * (qd + 2 * kvd));
    B.q = take(2 * (size_t)S * c.n_kv_heads * G * 16 * c.head_dim);
    B.po = take(4 * (size_t)dfl::BATCH_MAX_ITEMS * G * 16 * c.head_dim);
    B.pml = take(4 * (size_t)dfl::BATCH_MAX_ITEMS * G * 16 * 2);
    B.attn = take(4 * rows * qd);
    B.z = take(4 * rows * c.intermediate);
    // DFlash2 conv wrap: the convolved input, the sublayer output, the coefficients
    const bool d2 = c.d2_groups > 0;
    B.xc = take(d2 ? 4 * rows * H : 0);
    B.y = take(d2 ? 4 * rows * H : 0);
    B.dc = take(d2 ? 4 * rows * 4 * (size_t)c.d2_groups : 0);
    B.bytes = off;
    return B;
}

int check_layered(const dflash_model *m, int S) {
    const dflash_cfg &c = m->cfg;
    if (c.kv_dtype != DFLASH_BF16)
        return fail(DFLASH_E_UNSUPPORTED, "the layered round (batched, paged or windowed caches) needs a bf16 KV cache");
    if (S < 1 || S > dfl::BATCH_MAX_SEQ) return fail(DFLASH_E_INVAL, "n_seqs %d outside [1, %d]", S, dfl::BATCH_MAX_SEQ);
    if (S * c.n_kv_heads > dfl::BATCH_MAX_ITEMS)
        return fail(DFLASH_E_UNSUPPORTED, "%d sequences x %d kv heads exceed %d attention items", S, c.n_kv_heads,
                    dfl::BATCH_MAX_ITEMS);
    return DFLASH_OK;
}

// One round of S sequences through separate kernels; `base` is the offset of
// the layered path's region in the workspace (after the standard layout).
hipError_t run_round_layered(const dflash_model *m, const dflash_kv *kvs, int S, const float *noise, const int32_t *pos,
                             int b, float *out, void *ws, const WsLayout &L, size_t base, hipStream_t s) {
    const dflash_cfg &c = m->cfg;
    const BatchLayout B = batch_layout(c, S);
    const int H = c.hidden, I = c.intermediate, qd = c.n_q_heads * c.head_dim, kvd = c.n_kv_heads * c.head_dim;
    const int M = S * b;
    float *x = at<float>(ws, base + B.x), *xn = at<float>(ws, base + B.xn), *qkv = at<float>(ws, base + B.qkv);
    float *attn = at<float>(ws, base + B.attn), *z = at<float>(ws, base + B.z);
    float *part = at<float>(ws, L.gpart);
    unsigned *cnt = at<unsigned>(ws, L.gcnt);

    dfl::BatchArgs a{};
    int nmax = 1;
    for (int i = 0; i < S; ++i) {
        a.seq[i].kv = kv_view(m, &kvs[i]);
        a.seq[i].len = kvs[i].len;
        a.seq[i].win_lo = window_lo(&kvs[i]);
        nmax = std::max(nmax, kvs[i].len + b - (a.seq[i].win_lo & ~31));
    }
    a.S = S; a.b = b; a.nq = c.n_q_heads; a.nkv = c.n_kv_heads; a.G = c.n_q_heads / c.n_kv_heads; a.d = c.head_dim;
    a.qd = qd; a.kvd = kvd;
    a.qkv = qkv; a.qkv_ld = qd + 2 * kvd;
    a.pos = pos; a.eps = c.rms_eps; a.mscale = (float)m->mscale;
    a.qscale = (float)(1.4426950408889634 / std::sqrt((double)c.head_dim));
    memcpy(a.inv_freq, m->inv_freq, sizeof a.inv_freq);
    a.q = at<uint16_t>(ws, base + B.q);
    a.po = at<float>(ws, base + B.po);
    a.pml = at<float>(ws, base + B.pml);
    a.attn = attn;
    // key splits: about BATCH_MAX_ITEMS items in all, whole staged chunks per split
    const int chunk = dfl::BATCH_CHUNK_KEYS;
    int ns = std::max(1, std::min(dfl::BATCH_MAX_SPLITS, dfl::BATCH_MAX_ITEMS / (S * c.n_kv_heads)));
    a.kps = std::max(chunk, ((nmax + ns - 1) / ns + chunk - 1) / chunk * chunk);
    a.nsplit = (nmax + a.kps - 1) / a.kps;

    auto gemm = [&](const float *A, int lda, int K, std::initializer_list<dfl::GemmSeg> segs, float *Y, int ldy, int epi,
                    int cls) {
        dfl::GemmArgs g{};
        g.A = A; g.lda = lda; g.M = M; g.K = K;
        for (const dfl::GemmSeg &sg : segs) g.seg[g.nseg++] = sg;
        g.Y = Y; g.ldy = ldy; g.epi = epi; g.wtype = wtype(c);
        // the round's projections take single-plane bf16 activations (as the
        // persistent kernel does) except under the DFlash2 wrap
        g.planes = c.d2_groups > 0 ? 2 : 1;
        ProfScope p(cls, s);
        return dfl::gemm(g, part, cnt, s);
    };
    // DFlash2 conv wrap: coefficients of the sublayer's normed input (kept
    // for its finish conv), and the prepare conv of that input into xc
    const bool d2 = c.d2_groups > 0;
    float *xc = at<float>(ws, base + B.xc), *y = at<float>(ws, base + B.y), *dc = at<float>(ws, base + B.dc);
    auto d2_in = [&](const float *src, const dflash_matrix &w_dyn, const float *wbase) {
        hipError_t r = dfl::d2_dyn_launch(src, H, w_dyn.data, w_dyn.scale, c.weight_dtype, 4 * c.d2_groups, M, dc, s);
        if (r == hipSuccess) r = dfl::d2_conv_launch(src, dc, 0, wbase, H, c.d2_groups, b, M, xc, false, s);
        return r;
    };
    hipError_t e = hipMemcpyAsync(x, noise, sizeof(float) * (size_t)M * H, hipMemcpyDeviceToDevice, s);
    for (int l = 0; l < c.n_layers && e == hipSuccess; ++l) {
        const dflash_layer_weights &W = m->layers[l];
        a.layer = l;
        a.g_q = W.g_q;
        a.g_k = W.g_k;
        {
            ProfScope p(DFLASH_K_NORM, s);
            e = dfl::rmsnorm(x, H, W.g_in, xn, H, nullptr, M, H, c.rms_eps, s);
        }
        // DFlash2: the attention sublayer sees the prepare conv of its normed input
        if (e == hipSuccess && d2) e = d2_in(xn, W.attn_w_dyn, W.attn_base);
        if (e == hipSuccess)
            e = gemm(d2 ? xc : xn, H, H, {seg(W.wq, qd), seg(W.wk, kvd), seg(W.wv, kvd)}, qkv, qd + 2 * kvd,
                     dfl::EPI_STORE, DFLASH_K_GEMM_QKV);
        if (e == hipSuccess) {
            ProfScope p(DFLASH_K_ROPE, s);
            e = dfl::batch_qk_rope_launch(a, s);
        }
        if (e == hipSuccess) {
            ProfScope p(DFLASH_K_ATTN, s);
            e = dfl::batch_attn_launch(a, s);
        }
        if (e == hipSuccess) {
            if (d2) {   // o_proj, then its finish conv into the residual
                e = gemm(attn, qd, qd, {seg(W.wo, H)}, y, H, dfl::EPI_STORE, DFLASH_K_GEMM_O);
                if (e == hipSuccess) e = dfl::d2_conv_launch(y, dc, 1, W.attn_base, H, c.d2_groups, b, M, x, true, s);
            } else {
                e = gemm(attn, qd, qd, {seg(W.wo, H)}, x, H, dfl::EPI_ADD, DFLASH_K_GEMM_O);
            }
        }
        if (e == hipSuccess) {
            ProfScope p(DFLASH_K_NORM, s);
            e = dfl::rmsnorm(x, H, W.g_post, xn, H, nullptr, M, H, c.rms_eps, s);
        }
        if (e == hipSuccess && d2) e = d2_in(xn, W.mlp_w_dyn, W.mlp_base);
        if (e == hipSuccess)
            e = gemm(d2 ? xc : xn, H, H, {seg(W.wg, I), seg(W.wu, I)}, z, I, dfl::EPI_SWIGLU, DFLASH_K_GEMM_GATEUP);
        if (e == hipSuccess) {
            if (d2) {
                e = gemm(z, I, I, {seg(W.wd, H)}, y, H, dfl::EPI_STORE, DFLASH_K_GEMM_DOWN);
                if (e == hipSuccess) e = dfl::d2_conv_launch(y, dc, 1, W.mlp_base, H, c.d2_groups, b, M, x, true, s);
            } else {
                e = gemm(z, I, I, {seg(W.wd, H)}, x, H, dfl::EPI_ADD, DFLASH_K_GEMM_DOWN);
            }
        }
    }
    if (e == hipSuccess) {
        ProfScope p(DFLASH_K_NORM, s);
        e = dfl::rmsnorm(x, H, m->w.g_norm, out, H, nullptr, M, H, c.rms_eps, s);
    }
    return e;
}

}  // namespace

extern "C" {

const char *dflash_last_error(void) { return g_err.c_str(); }

size_t dflash_batch_workspace_bytes(const dflash_model *m, int32_t n_seqs, int32_t max_rows) {
    if (!m || n_seqs < 1 || n_seqs > dfl::BATCH_MAX_SEQ || max_rows < 0) return 0;
    return ws_layout(m->cfg, max_rows).total + batch_layout(m->cfg, n_seqs).bytes;
}

int dflash_forward_round_batch(const dflash_model *m, dflash_kv *kvs, int32_t n_seqs, const float *noise_emb,
                               const int32_t *pos_block, int32_t b, float *out, void *ws, size_t ws_bytes,
                               void *stream) {
    g_err.clear();
    if (!m) return fail(DFLASH_E_INVAL, "model is null");
    if (!kvs) return fail(DFLASH_E_INVAL, "kvs is null");
    int rc = check_layered(m, n_seqs);
    if (rc) return rc;
    if (b < 1 || b > MAX_BLOCK) return fail(DFLASH_E_INVAL, "block size b = %d outside [1, 16]", b);
    for (int i = 0; i < n_seqs; ++i) {
        if ((rc = check_kv(m, &kvs[i]))) return fail(rc, "sequence %d: %s", i, g_err.c_str());
        if ((int64_t)kvs[i].len + b > kvs[i].capacity)
            return fail(DFLASH_E_CAPACITY, "sequence %d: len %d + b %d exceeds capacity %d", i, kvs[i].len, b,
                        kvs[i].capacity);
        for (int j = 0; j < i; ++j)
            if (kvs[j].k == kvs[i].k || kvs[j].v == kvs[i].v)
                return fail(DFLASH_E_INVAL, "sequences %d and %d share KV storage", j, i);
    }
    if (!aligned(noise_emb, 16) || !aligned(out, 16) || !aligned(pos_block, 4))
        return fail(DFLASH_E_INVAL, "noise_emb / out / pos_block null or misaligned");
    if (!aligned(ws, 256)) return fail(DFLASH_E_INVAL, "workspace null or not 256-byte aligned");
    const size_t need = dflash_batch_workspace_bytes(m, n_seqs, 0);
    if (ws_bytes < need)
        return fail(DFLASH_E_INVAL, "workspace of %zu bytes is smaller than the %zu the batched round needs", ws_bytes, need);
    const WsLayout L = ws_layout(m->cfg, 0);
    hipError_t e = run_round_layered(m, kvs, n_seqs, noise_emb, pos_block, b, out, ws, L, L.total, (hipStream_t)stream);
    return e == hipSuccess ? DFLASH_OK : hip_fail(e, "forward_round_batch");
}

int dflash_load_weights(const dflash_cfg *cfg, const dflash_weights *w, dflash_model **out) {
    g_err.clear();
    if (!cfg || !w || !out) return fail(DFLASH_E_INVAL, "null argument");
    *out = nullptr;
    int rc = check_cfg(*cfg);
    if (rc) return rc;
    const dflash_cfg &c = *cfg;
    if ((rc = check_matrix(c, w->fc, "fc", -1))) return rc;
    if ((rc = check_vec(w->g_hidden_norm, "hidden_norm", -1)) || (rc = check_vec(w->g_norm, "norm", -1))) return rc;
    if (c.n_layers > 0 && !w->layers) return fail(DFLASH_E_INVAL, "layers array is null");
    for (int l = 0; l < c.n_layers; ++l) {
        const dflash_layer_weights &L = w->layers[l];
        const dflash_matrix *mats[] = {&L.wq, &L.wk, &L.wv, &L.wo, &L.wg, &L.wu, &L.wd};
        const char *names[] = {"wq", "wk", "wv", "wo", "wg", "wu", "wd"};
        for (int i = 0; i < 7; ++i)
            if ((rc = check_matrix(c, *mats[i], names[i], l))) return rc;
        if ((rc = check_vec(L.g_in, "g_in", l)) || (rc = check_vec(L.g_post, "g_post", l)) ||
            (rc = check_vec(L.g_q, "g_q", l)) || (rc = check_vec(L.g_k, "g_k", l)))
            return rc;
        if (c.d2_groups > 0) {
            if ((rc = check_matrix(c, L.attn_w_dyn, "attn_w_dyn", l)) || (rc = check_matrix(c, L.mlp_w_dyn, "mlp_w_dyn", l)) ||
                (rc = check_vec(L.attn_base, "attn_base", l)) || (rc = check_vec(L.mlp_base, "mlp_base", l)))
                return rc;
        }
    }
    dflash_model *m = new dflash_model{};
    m->cfg = c;
    m->w = *w;
    m->layers.assign(w->layers, w->layers + c.n_layers);
    m->w.layers = m->layers.data();
    rope_table(c, m->inv_freq, &m->mscale);
    *out = m;
    return DFLASH_OK;
}

void dflash_free(dflash_model *m) { delete m; }

size_t dflash_packed_bytes(const dflash_model *m) {
    g_err.clear();
    if (!m) { fail(DFLASH_E_INVAL, "model is null"); return 0; }
    const int nwg = round_nwg(m->cfg);
    if (nwg <= 0) { fail(DFLASH_E_HIP, "no usable device for the round kernel"); return 0; }
    return (size_t)pack_layer_bytes(m->cfg, nwg) * m->cfg.n_layers;
}

int dflash_pack_weights(dflash_model *m, void *dst, size_t bytes, void *stream) {
    g_err.clear();
    if (!m) return fail(DFLASH_E_INVAL, "model is null");
    if (!aligned(dst, 256)) return fail(DFLASH_E_INVAL, "dst null or not 256-byte aligned");
    const int nwg = round_nwg(m->cfg);
    if (nwg <= 0) return fail(DFLASH_E_HIP, "no usable device for the round kernel");
    const long long per = pack_layer_bytes(m->cfg, nwg);
    if (bytes < (size_t)per * m->cfg.n_layers)
        return fail(DFLASH_E_INVAL, "dst holds %zu bytes, the packed weights need %lld", bytes, per * m->cfg.n_layers);
    m->pk = static_cast<char *>(dst);
    m->pk_nwg = nwg;
    m->pk_layer = per;
    for (int l0 = 0; l0 < m->cfg.n_layers; l0 += dfl::SR_MAXL) {
        dfl::SrArgs ra{};
        fill_round_args(m, nwg, l0, std::min(dfl::SR_MAXL, m->cfg.n_layers - l0), ra);
        const hipError_t e = dfl::sround_pack_launch(ra, m->cfg.weight_dtype, nwg, (hipStream_t)stream);
        if (e != hipSuccess) { m->pk = nullptr; return hip_fail(e, "pack_weights"); }
    }
    return DFLASH_OK;
}

size_t dflash_workspace_bytes(const dflash_model *m, int32_t max_rows) {
    if (!m || max_rows < 0) return 0;
    return ws_layout(m->cfg, max_rows).total;
}

int dflash_rope_table(const dflash_model *m, double *inv_freq, int32_t n, double *mscale) {
    g_err.clear();
    if (!m || !inv_freq || !mscale) return fail(DFLASH_E_INVAL, "null argument");
    if (n != m->cfg.head_dim / 2) return fail(DFLASH_E_INVAL, "table has head_dim/2 = %d entries", m->cfg.head_dim / 2);
    memcpy(inv_freq, m->inv_freq, sizeof(double) * n);
    *mscale = m->mscale;
    return DFLASH_OK;
}

int dflash_ctx_features(const dflash_model *m, const float *taps, int32_t t, float *feats, void *ws, size_t ws_bytes,
                        void *stream) {
    g_err.clear();
    if (!m) return fail(DFLASH_E_INVAL, "model is null");
    if (t < 0) return fail(DFLASH_E_INVAL, "t = %d is negative", t);
    if (t == 0) return DFLASH_OK;
    if (!aligned(taps, 16) || !aligned(feats, 16)) return fail(DFLASH_E_INVAL, "taps / feats null or not 16-byte aligned");
    int rc = check_ws(m, ws, ws_bytes, t);
    if (rc) return rc;
    const WsLayout L = ws_layout(m->cfg, t);
    hipError_t e = run_ctx_features(m, taps, t, feats, at<float>(ws, L.gpart), at<unsigned>(ws, L.gcnt), (hipStream_t)stream);
    return e == hipSuccess ? DFLASH_OK : hip_fail(e, "ctx_features");
}

int dflash_ctx_features_noalloc(const dflash_model *m, const float *taps, int32_t t, float *feats, void *stream) {
    g_err.clear();
    if (!m) return fail(DFLASH_E_INVAL, "model is null");
    if (t < 0) return fail(DFLASH_E_INVAL, "t = %d is negative", t);
    if (t > DFLASH_NOALLOC_MAX_ROWS)
        return fail(DFLASH_E_INVAL, "t = %d exceeds the allocation-free entry point's maximum of %d rows", t,
                    DFLASH_NOALLOC_MAX_ROWS);
    if (t == 0) return DFLASH_OK;
    if (!aligned(taps, 16) || !aligned(feats, 16)) return fail(DFLASH_E_INVAL, "taps / feats null or not 16-byte aligned");
    void *sp = nullptr;
    hipError_t e = dfl::noalloc_scratch(&sp, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "ctx_features_noalloc scratch");
    float *part = static_cast<float *>(sp);
    unsigned *cnt = reinterpret_cast<unsigned *>(static_cast<char *>(sp) + dfl::NOALLOC_PART_BYTES);
    e = run_ctx_features(m, taps, t, feats, part, cnt, (hipStream_t)stream);
    return e == hipSuccess ? DFLASH_OK : hip_fail(e, "ctx_features_noalloc");
}

int dflash_ingest_ctx(const dflash_model *m, dflash_kv *kv, const float *feats, const int32_t *pos_new, int32_t t,
                      void *ws, size_t ws_bytes, void *stream) {
    g_err.clear();
    if (!m) return fail(DFLASH_E_INVAL, "model is null");
    int rc = check_kv(m, kv);
    if (rc) return rc;
    if (t < 0) return fail(DFLASH_E_INVAL, "t = %d is negative", t);
    if ((int64_t)kv->len + t > kv->capacity)
        return fail(DFLASH_E_CAPACITY, "len %d + t %d exceeds capacity %d", kv->len, t, kv->capacity);
    if (t == 0) return DFLASH_OK;
    if (!aligned(feats, 16) || !aligned(pos_new, 4)) return fail(DFLASH_E_INVAL, "feats / pos_new null or misaligned");
    if ((rc = check_ws(m, ws, ws_bytes, t))) return rc;
    hipError_t e = run_ingest(m, kv, 1, feats, pos_new, t, ws, ws_layout(m->cfg, t), (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "ingest_ctx");
    kv->len += t;
    return DFLASH_OK;
}

int dflash_ingest_ctx_batch(const dflash_model *m, dflash_kv *kvs, int32_t n_seqs, const float *feats,
                            const int32_t *pos_new, int32_t t, void *ws, size_t ws_bytes, void *stream) {
    g_err.clear();
    if (!m) return fail(DFLASH_E_INVAL, "model is null");
    if (!kvs) return fail(DFLASH_E_INVAL, "kvs is null");
    if (n_seqs < 1 || n_seqs > dfl::ROPE_MAX_SEQ) return fail(DFLASH_E_INVAL, "n_seqs %d outside [1, %d]", n_seqs, dfl::ROPE_MAX_SEQ);
    if (t < 0) return fail(DFLASH_E_INVAL, "t = %d is negative", t);
    int rc;
    for (int i = 0; i < n_seqs; ++i) {
        if ((rc = check_kv(m, &kvs[i]))) return fail(rc, "sequence %d: %s", i, g_err.c_str());
        if ((int64_t)kvs[i].len + t > kvs[i].capacity)
            return fail(DFLASH_E_CAPACITY, "sequence %d: len %d + t %d exceeds capacity %d", i, kvs[i].len, t, kvs[i].capacity);
        for (int j = 0; j < i; ++j)
            if (kvs[j].k == kvs[i].k || kvs[j].v == kvs[i].v)
                return fail(DFLASH_E_INVAL, "sequences %d and %d share KV storage", j, i);
    }
    if (t == 0) return DFLASH_OK;
    if (!aligned(feats, 16) || !aligned(pos_new, 4)) return fail(DFLASH_E_INVAL, "feats / pos_new null or misaligned");
    const int rows = n_seqs * t;
    if ((rc = check_ws(m, ws, ws_bytes, rows))) return rc;
    hipError_t e = run_ingest(m, kvs, n_seqs, feats, pos_new, t, ws, ws_layout(m->cfg, rows), (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "ingest_ctx_batch");
    for (int i = 0; i < n_seqs; ++i) kvs[i].len += t;
    return DFLASH_OK;
}

int dflash_forward_round(const dflash_model *m, dflash_kv *kv, const float *noise_emb, const int32_t *pos_block,
                         int32_t b, float *out, void *ws, size_t ws_bytes, void *stream) {
    g_err.clear();
    if (!m) return fail(DFLASH_E_INVAL, "model is null");
    int rc = check_kv(m, kv);
    if (rc) return rc;
    if (b < 1 || b > MAX_BLOCK) return fail(DFLASH_E_INVAL, "block size b = %d outside [1, 16]", b);
    if ((int64_t)kv->len + b > kv->capacity)
        return fail(DFLASH_E_CAPACITY, "len %d + b %d exceeds capacity %d", kv->len, b, kv->capacity);
    if (!aligned(noise_emb, 16) || !aligned(out, 16) || !aligned(pos_block, 4))
        return fail(DFLASH_E_INVAL, "noise_emb / out / pos_block null or misaligned");
    if (needs_layered(kv)) {
        // paged or windowed cache: the layered path with one sequence
        if ((rc = check_layered(m, 1))) return rc;
        if (!aligned(ws, 256)) return fail(DFLASH_E_INVAL, "workspace null or not 256-byte aligned");
        const size_t need = dflash_batch_workspace_bytes(m, 1, 0);
        if (ws_bytes < need)
            return fail(DFLASH_E_INVAL, "a paged or windowed cache needs a workspace of %zu bytes, got %zu", need, ws_bytes);
        const WsLayout L = ws_layout(m->cfg, 0);
        hipError_t e = run_round_layered(m, kv, 1, noise_emb, pos_block, b, out, ws, L, L.total, (hipStream_t)stream);
        return e == hipSuccess ? DFLASH_OK : hip_fail(e, "forward_round");
    }
    if ((rc = check_ws(m, ws, ws_bytes, 0)) || (rc = check_packed(m))) return rc;
    hipError_t e = run_round(m, kv, noise_emb, pos_block, b, out, ws, ws_layout(m->cfg, 0), (hipStream_t)stream);
    return e == hipSuccess ? DFLASH_OK : hip_fail(e, "forward_round");
}

int dflash_forward_full(const dflash_model *m, const float *taps, const float *noise_emb, const int32_t *pos, int32_t n,
                        int32_t b, float *out, dflash_kv *scratch, void *ws, size_t ws_bytes, void *stream) {
    g_err.clear();
    if (!m) return fail(DFLASH_E_INVAL, "model is null");
    int rc = check_kv(m, scratch);
    if (rc) return rc;
    if (n < 0) return fail(DFLASH_E_INVAL, "n = %d is negative", n);
    if (b < 1 || b > MAX_BLOCK) return fail(DFLASH_E_INVAL, "block size b = %d outside [1, 16]", b);
    if ((int64_t)n + b > scratch->capacity)
        return fail(DFLASH_E_CAPACITY, "n %d + b %d exceeds scratch capacity %d", n, b, scratch->capacity);
    if ((n > 0 && !aligned(taps, 16)) || !aligned(noise_emb, 16) || !aligned(out, 16) || !aligned(pos, 4))
        return fail(DFLASH_E_INVAL, "taps / noise_emb / out / pos null or misaligned");
    if (scratch->ctx_cap != 0) return fail(DFLASH_E_INVAL, "the first-light forward attends every row: scratch ctx_cap must be 0");
    const bool layered = needs_layered(scratch);
    if (layered) {
        if ((rc = check_layered(m, 1))) return rc;
        if (!aligned(ws, 256)) return fail(DFLASH_E_INVAL, "workspace null or not 256-byte aligned");
        const size_t need = dflash_batch_workspace_bytes(m, 1, n);
        if (ws_bytes < need)
            return fail(DFLASH_E_INVAL, "a paged scratch cache needs a workspace of %zu bytes, got %zu", need, ws_bytes);
    } else if ((rc = check_ws(m, ws, ws_bytes, n)) || (rc = check_packed(m))) {
        return rc;
    }
    const WsLayout L = ws_layout(m->cfg, n);
    hipStream_t s = (hipStream_t)stream;
    float *feats = at<float>(ws, L.feats);
    hipError_t e = hipSuccess;
    dflash_kv kv = *scratch;
    kv.len = 0;
    if (n > 0) {
        e = run_ctx_features(m, taps, n, feats, at<float>(ws, L.gpart), at<unsigned>(ws, L.gcnt), s);
        if (e == hipSuccess) e = run_ingest(m, &kv, 1, feats, pos, n, ws, L, s);
        kv.len = n;
    }
    if (e == hipSuccess) {
        if (layered) e = run_round_layered(m, &kv, 1, noise_emb, pos + n, b, out, ws, L, L.total, s);
        else e = run_round(m, &kv, noise_emb, pos + n, b, out, ws, L, s);
    }
    if (e != hipSuccess) return hip_fail(e, "forward_full");
    scratch->len = n;
    return DFLASH_OK;
}

int dflash_workspace_status(const dflash_model *m, void *ws, size_t ws_bytes, void *stream) {
    g_err.clear();
    if (!m) return fail(DFLASH_E_INVAL, "model is null");
    int rc = check_ws(m, ws, ws_bytes, 0);
    if (rc) return rc;
    const WsLayout L = ws_layout(m->cfg, 0);
    unsigned *ctr = at<unsigned>(ws, L.ctr);
    unsigned h = 0;
    hipError_t e = hipStreamSynchronize((hipStream_t)stream);
    if (e == hipSuccess) e = hipMemcpy(&h, ctr + dfl::SR_CTR_ERR, sizeof h, hipMemcpyDeviceToHost);
    if (e != hipSuccess) return hip_fail(e, "workspace_status");
    if (h != 0) {
        // the phase counters are inconsistent after a timed-out wait: start them over
        e = hipMemset(ctr, 0, sizeof(unsigned) * dfl::SR_CTR_WORDS);
        if (e == hipSuccess) e = hipDeviceSynchronize();
        if (e != hipSuccess) return hip_fail(e, "workspace_status");
        if (h == 2) return fail(DFLASH_E_HIP, "the round kernel found its arguments at an unexpected place; its output is NaN");
        return fail(DFLASH_E_HIP, "a bounded wait of the round kernel timed out (not all workgroups were resident); "
                                  "its output is NaN");
    }
    return DFLASH_OK;
}

// ---- DFlash2 proposal ([DflashDraft] "dflash2_propose_greedy") ----------------

namespace {

// device step into `packed`: [nd][k] values, [nd][k] indices, [nd][rank] projection
int propose_prepare(const dflash_model *m, const dflash2_selector *sel, const float *logits, const float *hidden, int b,
                    uint32_t *packed, void *ws, size_t ws_bytes, hipStream_t s) {
    if (!m || !sel) return fail(DFLASH_E_INVAL, "model / selector is null");
    if (sel->vocab <= 0 || sel->top_k < 1 || sel->top_k > DFLASH2_MAX_TOPK || sel->rank < 1 || sel->rank > DFLASH2_MAX_RANK)
        return fail(DFLASH_E_INVAL, "selector: vocab %d, top_k %d (1..%d), rank %d (1..%d)", sel->vocab, sel->top_k,
                    DFLASH2_MAX_TOPK, sel->rank, DFLASH2_MAX_RANK);
    if (sel->top_k > sel->vocab) return fail(DFLASH_E_INVAL, "top_k %d exceeds the vocabulary %d", sel->top_k, sel->vocab);
    if (!aligned(sel->w_hidden_proj, 16)) return fail(DFLASH_E_INVAL, "selector w_hidden_proj null or not 16-byte aligned");
    if (b < 2 || b > MAX_BLOCK) return fail(DFLASH_E_INVAL, "block size b = %d outside [2, 16] (row 0 is the anchor)", b);
    if (!aligned(logits, 4) || !aligned(hidden, 4) || !aligned(packed, 4))
        return fail(DFLASH_E_INVAL, "draft logits / hidden / output null or misaligned");
    const int nd = b - 1, k = sel->top_k;
    int rc = check_ws(m, ws, ws_bytes, 0);
    if (rc) return rc;
    const WsLayout L = ws_layout(m->cfg, 0);
    const size_t part = dfl::topk_scratch_entries(nd, sel->vocab, k);
    if (2 * part * 4 > 4 * dfl::GEMM_PART_FLOATS)
        return fail(DFLASH_E_UNSUPPORTED, "top-k candidates of %zu bytes exceed the workspace's %zu", 2 * part * 4,
                    4 * dfl::GEMM_PART_FLOATS);
    float *pv = at<float>(ws, L.gpart);
    int32_t *pi = reinterpret_cast<int32_t *>(pv + part);
    float *vals = reinterpret_cast<float *>(packed);
    int32_t *idx = reinterpret_cast<int32_t *>(packed + (size_t)nd * k);
    float *hp = reinterpret_cast<float *>(packed + (size_t)2 * nd * k);
    const long long V = sel->vocab;
    hipError_t e = dfl::topk_rows(logits + V, V, nd, sel->vocab, k, pv, pi, vals, idx, hidden + m->cfg.hidden,
                                  m->cfg.hidden, sel->w_hidden_proj, sel->rank, hp, s);
    return e == hipSuccess ? DFLASH_OK : hip_fail(e, "dflash2_propose");
}

}  // namespace

int dflash2_propose_prepare(const dflash_model *m, const dflash2_selector *sel, const float *draft_logits,
                            const float *hidden, int32_t b, uint32_t *packed, void *ws, size_t ws_bytes, void *stream) {
    g_err.clear();
    return propose_prepare(m, sel, draft_logits, hidden, b, packed, ws, ws_bytes, (hipStream_t)stream);
}

int dflash2_propose_greedy(const dflash_model *m, const dflash2_selector *sel, const float *draft_logits,
                           const float *hidden, int32_t b, int32_t anchor, int32_t *drafts, void *ws, size_t ws_bytes,
                           void *stream) {
    g_err.clear();
    if (!drafts) return fail(DFLASH_E_INVAL, "drafts is null");
    if (!m || !sel) return fail(DFLASH_E_INVAL, "model / selector is null");
    if (!sel->pred_codebook || !sel->succ_codebook) return fail(DFLASH_E_INVAL, "selector codebooks are null");
    if (b < 2 || b > MAX_BLOCK) return fail(DFLASH_E_INVAL, "block size b = %d outside [2, 16] (row 0 is the anchor)", b);
    if (anchor < 0 || anchor >= sel->vocab) return fail(DFLASH_E_INVAL, "anchor %d outside the vocabulary", anchor);
    const int nd = b - 1, k = sel->top_k, rank = sel->rank;
    // the packed block sits after the top-k partials in the GEMM scratch region
    if (!aligned(ws, 256)) return fail(DFLASH_E_INVAL, "workspace null or not 256-byte aligned");
    const WsLayout L = ws_layout(m->cfg, 0);
    const size_t words = (size_t)nd * (2 * k + rank);
    const size_t part_bytes = 2 * dfl::topk_scratch_entries(nd, std::max(sel->vocab, 1), std::max(k, 1)) * 4;
    if (part_bytes + 4 * words > 4 * dfl::GEMM_PART_FLOATS)
        return fail(DFLASH_E_UNSUPPORTED, "top-k partials and packed block exceed the workspace's scratch region");
    uint32_t *packed = at<uint32_t>(ws, L.gpart + (part_bytes + 255) / 256 * 256);
    hipStream_t s = (hipStream_t)stream;
    int rc = propose_prepare(m, sel, draft_logits, hidden, b, packed, ws, ws_bytes, s);
    if (rc) return rc;
    // the one small device-to-host copy of the round, into pinned memory (a
    // copy into pageable memory goes through the runtime's staging buffer),
    // then the host walk.  Each host thread allocates its buffer once, at
    // the largest packed block, and holds it until the process ends.
    constexpr size_t MAX_WORDS = (size_t)(MAX_BLOCK - 1) * (2 * DFLASH2_MAX_TOPK + DFLASH2_MAX_RANK);
    thread_local uint32_t *host = nullptr;
    if (!host) {
        void *p = nullptr;
        hipError_t ea = hipHostMalloc(&p, 4 * MAX_WORDS, hipHostMallocDefault);
        if (ea != hipSuccess) return hip_fail(ea, "dflash2_propose_greedy pinned host buffer");
        host = static_cast<uint32_t *>(p);
    }
    if (words > MAX_WORDS) return fail(DFLASH_E_INVAL, "packed block larger than its bound");
    hipError_t e = hipMemcpyAsync(host, packed, 4 * words, hipMemcpyDeviceToHost, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e != hipSuccess) return hip_fail(e, "dflash2_propose_greedy copy");
    const float *vals = reinterpret_cast<const float *>(host);
    const int32_t *idx = reinterpret_cast<const int32_t *>(host + (size_t)nd * k);
    const float *hp = reinterpret_cast<const float *>(host + (size_t)2 * nd * k);
    rc = dflash2_walk_greedy(sel, vals, idx, hp, nd, anchor, drafts);
    return rc ? fail(rc, "dflash2_propose_greedy: walk rejected its inputs") : DFLASH_OK;
}

int dflash_prof_trace(int32_t enable) {
    g_trace.store(enable ? 1 : 0);
    return DFLASH_OK;
}

int dflash_prof_trace_read(const dflash_model *m, void *ws, size_t ws_bytes, uint64_t *out, int32_t n, void *stream) {
    g_err.clear();
    if (!m || !out || n < 0 || n > dfl::SR_TRACE) return fail(DFLASH_E_INVAL, "bad trace read arguments");
    int rc = check_ws(m, ws, ws_bytes, 0);
    if (rc) return rc;
    const WsLayout L = ws_layout(m->cfg, 0);
    hipError_t e = hipStreamSynchronize((hipStream_t)stream);
    if (e == hipSuccess) e = hipMemcpy(out, at<unsigned long long>(ws, L.trace), sizeof(uint64_t) * n, hipMemcpyDeviceToHost);
    return e == hipSuccess ? DFLASH_OK : hip_fail(e, "trace_read");
}

int dflash_prof_start(int32_t kernel_class, int32_t max_launches) {
    g_err.clear();
    if (kernel_class < DFLASH_K_GEMM_FC || kernel_class > DFLASH_K_ROUND || max_launches <= 0 || max_launches > (1 << 20))
        return fail(DFLASH_E_INVAL, "bad kernel class %d or launch count %d", kernel_class, max_launches);
    std::lock_guard<std::mutex> lk(g_prof.mu);
    while ((int)g_prof.ev.size() < 2 * max_launches) {
        hipEvent_t e;
        hipError_t r = hipEventCreate(&e);
        if (r != hipSuccess) return hip_fail(r, "prof_start");
        g_prof.ev.push_back(e);
    }
    g_prof.cap = max_launches;
    g_prof.used = 0;
    g_prof.cls.store(kernel_class);
    return DFLASH_OK;
}

int dflash_prof_stop(double *total_ms, int32_t *launches) {
    g_err.clear();
    if (!total_ms || !launches) return fail(DFLASH_E_INVAL, "null argument");
    std::lock_guard<std::mutex> lk(g_prof.mu);
    g_prof.cls.store(0);
    double tot = 0.0;
    for (int i = 0; i < g_prof.used; ++i) {
        hipError_t r = hipEventSynchronize(g_prof.ev[2 * i + 1]);
        if (r != hipSuccess) return hip_fail(r, "prof_stop");
        float ms = 0.f;
        r = hipEventElapsedTime(&ms, g_prof.ev[2 * i], g_prof.ev[2 * i + 1]);
        if (r != hipSuccess) return hip_fail(r, "prof_stop");
        tot += ms;
    }
    *total_ms = tot;
    *launches = g_prof.used;
    g_prof.used = 0;
    return DFLASH_OK;
}

}  // extern "C"
