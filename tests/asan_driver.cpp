// Host-side driver of libdflash's argument checks, size queries and host
// policy functions, built with AddressSanitizer and UBSan
// (tests/test_asan_host.py).  Every call here returns before any device
// work, so it runs without a GPU.  Exit status 0 means every expectation held.
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <vector>

#include "dflash.h"
#include "dflash_policy.h"

static int g_bad = 0;
#define EXPECT(cond)                                                              \
    do {                                                                          \
        if (!(cond)) {                                                            \
            std::printf("expectation failed at line %d: %s\n", __LINE__, #cond);  \
            ++g_bad;                                                              \
        }                                                                         \
    } while (0)

// distinct, aligned addresses that are never dereferenced on the host
static uintptr_t g_addr = 0x100000;
static const void *fake() { g_addr += 0x1000; return reinterpret_cast<const void *>(g_addr); }

static dflash_cfg cfg_c3() {
    dflash_cfg c{};
    c.n_layers = 8; c.hidden = 2048; c.n_q_heads = 32; c.n_kv_heads = 4; c.head_dim = 128;
    c.intermediate = 6144; c.n_taps = 5; c.rms_eps = 1e-6f; c.rope_base = 1e6; c.rope_type = DFLASH_ROPE_PLAIN;
    c.weight_dtype = DFLASH_BF16; c.kv_dtype = DFLASH_BF16; c.d2_groups = 0;
    return c;
}

int main() {
    dflash_cfg c = cfg_c3();
    std::vector<dflash_layer_weights> layers(c.n_layers);
    for (auto &L : layers) {
        dflash_matrix *m[] = {&L.wq, &L.wk, &L.wv, &L.wo, &L.wg, &L.wu, &L.wd};
        for (auto *x : m) { x->data = fake(); x->scale = nullptr; }
        L.g_in = (const float *)fake(); L.g_post = (const float *)fake();
        L.g_q = (const float *)fake(); L.g_k = (const float *)fake();
    }
    dflash_weights w{};
    w.fc = {fake(), nullptr};
    w.g_hidden_norm = (const float *)fake();
    w.g_norm = (const float *)fake();
    w.layers = layers.data();

    // config and weight validation
    dflash_model *m = nullptr;
    EXPECT(dflash_load_weights(nullptr, &w, &m) == DFLASH_E_INVAL);
    dflash_cfg bad = c; bad.head_dim = 96;
    EXPECT(dflash_load_weights(&bad, &w, &m) == DFLASH_E_UNSUPPORTED && std::strlen(dflash_last_error()) > 0);
    bad = c; bad.n_q_heads = 30;                       // not a multiple of n_kv_heads
    EXPECT(dflash_load_weights(&bad, &w, &m) == DFLASH_E_INVAL);
    bad = c; bad.n_kv_heads = 2;                       // 16 q heads per kv head
    EXPECT(dflash_load_weights(&bad, &w, &m) == DFLASH_E_UNSUPPORTED);
    layers[3].wq.data = reinterpret_cast<const void *>(g_addr + 4);
    EXPECT(dflash_load_weights(&c, &w, &m) == DFLASH_E_INVAL);
    layers[3].wq.data = fake();
    EXPECT(dflash_load_weights(&c, &w, &m) == DFLASH_OK && m != nullptr);

    // sizes
    EXPECT(dflash_workspace_bytes(m, 0) > 0 && dflash_workspace_bytes(m, 1024) > dflash_workspace_bytes(m, 0));
    EXPECT(dflash_workspace_bytes(m, -1) == 0);
    EXPECT(dflash_batch_workspace_bytes(m, 0, 0) == 0 && dflash_batch_workspace_bytes(m, 9, 0) == 0);
    EXPECT(dflash_batch_workspace_bytes(m, 8, 0) > dflash_batch_workspace_bytes(m, 1, 0));
    EXPECT(dflash_batch_workspace_bytes(m, 1, 0) > dflash_workspace_bytes(m, 0));
    double inv[64], ms = 0;
    EXPECT(dflash_rope_table(m, inv, 64, &ms) == DFLASH_OK && ms == 1.0 && inv[0] == 1.0);
    EXPECT(dflash_rope_table(m, inv, 32, &ms) == DFLASH_E_INVAL);

    // argument errors of the compute calls: all rejected before any HIP call
    const size_t wsb = dflash_batch_workspace_bytes(m, 8, 64);
    void *ws = const_cast<void *>(fake());
    dflash_kv kv{};
    kv.k = const_cast<void *>(fake()); kv.v = const_cast<void *>(fake()); kv.capacity = 4160; kv.len = 4096;
    const float *f = (const float *)fake();
    const int32_t *p = (const int32_t *)fake();
    float *o = (float *)fake();
    EXPECT(dflash_forward_round(m, nullptr, f, p, 16, o, ws, wsb, nullptr) == DFLASH_E_INVAL);
    EXPECT(dflash_forward_round(m, &kv, f, p, 17, o, ws, wsb, nullptr) == DFLASH_E_INVAL);
    EXPECT(dflash_forward_round(m, &kv, f, p, 0, o, ws, wsb, nullptr) == DFLASH_E_INVAL);
    dflash_kv full = kv; full.len = 4150;
    EXPECT(dflash_forward_round(m, &full, f, p, 16, o, ws, wsb, nullptr) == DFLASH_E_CAPACITY);
    dflash_kv odd = kv; odd.capacity = 4100;
    EXPECT(dflash_forward_round(m, &odd, f, p, 16, o, ws, wsb, nullptr) == DFLASH_E_INVAL);
    dflash_kv paged = kv; paged.page_rows = 96;        // not a multiple of 64
    EXPECT(dflash_forward_round(m, &paged, f, p, 16, o, ws, wsb, nullptr) == DFLASH_E_INVAL);
    paged.page_rows = 64; paged.pool_pages = 0;
    EXPECT(dflash_forward_round(m, &paged, f, p, 16, o, ws, wsb, nullptr) == DFLASH_E_INVAL);
    paged.pool_pages = 70; paged.block_table = nullptr;
    EXPECT(dflash_forward_round(m, &paged, f, p, 16, o, ws, wsb, nullptr) == DFLASH_E_INVAL);
    dflash_kv win = kv; win.ctx_cap = -5;
    EXPECT(dflash_forward_round(m, &win, f, p, 16, o, ws, wsb, nullptr) == DFLASH_E_INVAL);
    win.ctx_cap = 1024;                                // needs the layered workspace
    EXPECT(dflash_forward_round(m, &win, f, p, 16, o, ws, dflash_workspace_bytes(m, 0), nullptr) == DFLASH_E_INVAL);
    EXPECT(dflash_forward_round(m, &kv, f, p, 16, o, ws, 10, nullptr) == DFLASH_E_INVAL);
    EXPECT(dflash_ingest_ctx(m, &full, f, p, 16, ws, wsb, nullptr) == DFLASH_E_CAPACITY && full.len == 4150);
    EXPECT(dflash_ingest_ctx(m, &kv, f, p, -1, ws, wsb, nullptr) == DFLASH_E_INVAL);
    EXPECT(dflash_ctx_features(m, f, -3, o, ws, wsb, nullptr) == DFLASH_E_INVAL);
    EXPECT(dflash_ctx_features_noalloc(m, f, 65537, o, nullptr) == DFLASH_E_INVAL);
    dflash_kv two[2] = {kv, kv};                       // shared storage
    EXPECT(dflash_forward_round_batch(m, two, 2, f, p, 16, o, ws, wsb, nullptr) == DFLASH_E_INVAL);
    EXPECT(dflash_forward_round_batch(m, two, 9, f, p, 16, o, ws, wsb, nullptr) == DFLASH_E_INVAL);
    two[1].k = const_cast<void *>(fake()); two[1].v = const_cast<void *>(fake()); two[1].len = 4150;
    EXPECT(dflash_forward_round_batch(m, two, 2, f, p, 16, o, ws, wsb, nullptr) == DFLASH_E_CAPACITY);
    EXPECT(dflash_ingest_ctx_batch(m, two, 2, f, p, 16, ws, wsb, nullptr) == DFLASH_E_CAPACITY &&
           two[0].len == 4096 && two[1].len == 4150);
    dflash_kv scratch = kv; scratch.len = 0; scratch.ctx_cap = 8;
    EXPECT(dflash_forward_full(m, f, f, p, 64, 16, o, &scratch, ws, wsb, nullptr) == DFLASH_E_INVAL);

    // the proposal's argument checks
    std::vector<uint16_t> cb(100 * 8);
    dflash2_selector sel{100, 8, 101, cb.data(), cb.data(), fake()};   // top_k > vocab
    int32_t drafts[15];
    EXPECT(dflash2_propose_greedy(m, &sel, f, f, 16, 0, drafts, ws, wsb, nullptr) == DFLASH_E_INVAL);
    sel.top_k = 8;
    EXPECT(dflash2_propose_greedy(m, &sel, f, f, 1, 0, drafts, ws, wsb, nullptr) == DFLASH_E_INVAL);
    EXPECT(dflash2_propose_greedy(m, &sel, f, f, 16, 100, drafts, ws, wsb, nullptr) == DFLASH_E_INVAL);

    // host policy functions on real host data
    int32_t cand[5] = {7, 1, 2, 3, 4}, vam[5] = {1, 2, 9, 4, 5}, mm = -1;
    EXPECT(dflash_accept_prefix(cand, 5, vam, 5, &mm) == DFLASH_OK && mm == 2);
    EXPECT(dflash_accept_prefix(cand, 5, vam, 0, &mm) == DFLASH_E_INVAL);
    double pp[3] = {0.3, 0.2, 0.9}, qq[3] = {0.3, 0.9, 0.95}, uu[3] = {0.2, 0.5, 0.0};
    int32_t acc = -1;
    EXPECT(dflash_rejection_accept_len(pp, qq, uu, 3, &acc) == DFLASH_OK && acc == 1);
    float raws[6] = {3, 3, -3, 3, 3, 3};
    int32_t vt = 0;
    EXPECT(dflash_slot_confidence_vt(raws, 6, 0.5, 16, &vt) == DFLASH_OK && vt == 3);
    EXPECT(dflash_confidence_vt(raws, 6, 0.5, 1, &vt) == DFLASH_E_INVAL);
    EXPECT(dflash_confidence_vt(raws, 6, 0.0, 4, &vt) == DFLASH_OK && vt == 4);
    for (size_t i = 0; i < cb.size(); ++i) cb[i] = (uint16_t)(0x3F80 + (i % 7));   // bf16 values near 1
    float unary[2 * 8], hproj[2 * 8];
    int32_t cands[2 * 8], path[2];
    for (int i = 0; i < 16; ++i) { unary[i] = (float)(16 - i) * 0.1f; hproj[i] = 0.01f * i; cands[i] = (i * 13) % 100; }
    EXPECT(dflash2_walk_greedy(&sel, unary, cands, hproj, 2, 3, path) == DFLASH_OK);
    double uni[2] = {0.25, 0.75}, qc[2], qr[16];
    EXPECT(dflash2_walk_sampled(&sel, unary, cands, hproj, 2, 3, 0.7, uni, path, qc, qr) == DFLASH_OK);
    double tot = 0;
    for (int i = 0; i < 8; ++i) tot += qr[i];
    EXPECT(tot > 0.999999 && tot < 1.000001);
    cands[3] = 1000;                                   // out of the vocabulary
    EXPECT(dflash2_walk_greedy(&sel, unary, cands, hproj, 2, 3, path) == DFLASH_E_INVAL);

    dflash_free(m);
    dflash_free(nullptr);
    std::printf("%s: %d failed expectations\n", g_bad ? "FAIL" : "OK", g_bad);
    return g_bad ? 1 : 0;
}
