/*
 * dflash.h — C ABI of the MI355X (gfx950) DFlash block-diffusion drafter
 * forward.
 *
 * The drafter is a small Qwen3-class transformer that drafts a whole block of
 * b <= 16 tokens in one non-causal forward.  It is conditioned on context
 * features hidden_norm(fc(concat of the target's tapped hidden states)),
 * which are served from an append-only draft KV cache.
 *
 * Sources (the pages these calls implement):
 *  [memra dflash module]  docs.rs memra_engine::dflash, module index
 *                         (overview, "DflashKv", "Dflash2Conv").
 *  [DflashDraft]          docs.rs memra_engine::dflash::DflashDraft, struct page
 *                         (fields, "ctx_features", "forward", "forward_block",
 *                          "ingest_ctx", "forward_round", "d2_conv_prepare",
 *                          "d2_conv_finish", "rope_yarn").
 *  [atlas dflash_head]    spark_model::layers::dflash_head, module page
 *                         (overview, "DflashLayer", "DflashQuantization",
 *                          "DflashScratch", "DflashProposerState").
 *
 * Conventions for every call
 *  - Pointers named "device" point into GPU memory of the current HIP device.
 *    Pointers named "host" point into host memory.  The caller owns all
 *    memory.  The library allocates no device memory, and it copies nothing
 *    between host and device.
 *  - Compute calls are asynchronous on `stream` (a hipStream_t; NULL means the
 *    default stream).  They never synchronise the host.  Inputs must stay
 *    alive and unchanged until the stream has passed the call.
 *  - Return value: DFLASH_OK (0) or an error code.  dflash_last_error()
 *    returns a message for the calling thread's last error.  All argument
 *    checks run before anything is enqueued (device-attribute queries aside).
 *    On an error nothing has been enqueued, and kv->len is unchanged.  A HIP
 *    launch failure is DFLASH_E_HIP.
 *  - Call order: dflash_load_weights, then dflash_pack_weights once per
 *    model and device, then any number of ctx_features / ingest_ctx /
 *    forward_round calls.
 *  - One round at a time per device.  forward_round and forward_full run a
 *    persistent kernel that needs one resident workgroup on every compute
 *    unit and spins at grid-wide barriers.  While it runs, no other kernel
 *    may occupy the device's compute units: the caller keeps at most one
 *    forward_round / forward_full in flight per device, and does not overlap
 *    it with other work on other streams.  (ctx_features and ingest_ctx are
 *    ordinary kernels; the same rule covers them only because they share
 *    the device.)  One dflash_kv and one workspace must never be used by
 *    two calls in flight at the same time.
 *  - If that rule is broken and the round kernel cannot get every
 *    workgroup resident, its bounded barrier waits expire after about a
 *    second.  The call has already returned DFLASH_OK (the library never
 *    synchronises), so the failure shows in the data instead: every output
 *    row of that round is NaN, an error flag is set in the workspace, and
 *    every later round on that workspace also yields NaN until
 *    dflash_workspace_status reports the flag and clears it.
 */
#ifndef DFLASH_H
#define DFLASH_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- error codes ------------------------------------------------------- */
#define DFLASH_OK            0
#define DFLASH_E_INVAL       1  /* null/misaligned pointer, bad size or count */
#define DFLASH_E_CAPACITY    2  /* kv->len + rows would exceed kv->capacity */
#define DFLASH_E_UNSUPPORTED 3  /* a dtype / shape combination not built */
#define DFLASH_E_HIP         4  /* HIP runtime or launch error */

/* ---- storage types ----------------------------------------------------- */
#define DFLASH_F32       0
#define DFLASH_BF16      1
#define DFLASH_FP8_E4M3  2   /* OCP e4m3fn codes + one f32 scale per row */

#define DFLASH_ROPE_PLAIN 0
#define DFLASH_ROPE_YARN  1

/* Model dimensions and options ([DflashDraft] field "cfg"; [atlas
 * dflash_head] overview).  Supported: hidden, intermediate, n_q_heads*head_dim
 * and n_taps*hidden are multiples of 256.  head_dim is 64 or 128.  n_q_heads is
 * a multiple of n_kv_heads, with n_q_heads/n_kv_heads <= 8 (the round
 * kernel's attention item holds one q head per compute wave; a larger ratio
 * is DFLASH_E_UNSUPPORTED).  For DFLASH_F32
 * weights the KV dtype must be DFLASH_F32; otherwise it must be DFLASH_BF16.
 * d2_groups divides hidden; 0 disables the DFlash2 conv wrap. */
typedef struct dflash_cfg {
    int32_t n_layers;
    int32_t hidden;
    int32_t n_q_heads;
    int32_t n_kv_heads;
    int32_t head_dim;
    int32_t intermediate;
    int32_t n_taps;           /* tapped target layers; fc input = n_taps*hidden */
    float   rms_eps;          /* every RMSNorm (hidden_norm, layer norms, q/k head norms, final norm) */
    double  rope_base;
    int32_t rope_type;        /* DFLASH_ROPE_PLAIN | DFLASH_ROPE_YARN */
    double  yarn_factor;      /* YaRN only ([DflashDraft] "rope_yarn") */
    int32_t yarn_orig_ctx;
    double  yarn_beta_fast;
    double  yarn_beta_slow;
    int32_t weight_dtype;     /* DFLASH_F32 | DFLASH_BF16 | DFLASH_FP8_E4M3 */
    int32_t kv_dtype;         /* DFLASH_F32 | DFLASH_BF16 */
    int32_t d2_groups;        /* DFlash2 conv groups G; 0 = no conv wrap */
} dflash_cfg;

/* One projection matrix, [N_out, K_in] row-major (torch Linear layout), in
 * cfg.weight_dtype.  For DFLASH_FP8_E4M3, `scale` holds N_out f32 row scales
 * and W[n,k] = scale[n] * e4m3fn(data[n,k]).  Otherwise `scale` is NULL.
 * Device pointers, 16-byte aligned. */
typedef struct dflash_matrix {
    const void  *data;
    const float *scale;
} dflash_matrix;

/* One drafter layer ([atlas dflash_head] "DflashLayer": Qwen3-style weights,
 * no biases).  Gains are f32 device vectors. */
typedef struct dflash_layer_weights {
    dflash_matrix wq;         /* [n_q_heads*head_dim, hidden] */
    dflash_matrix wk;         /* [n_kv_heads*head_dim, hidden] */
    dflash_matrix wv;         /* [n_kv_heads*head_dim, hidden] */
    dflash_matrix wo;         /* [hidden, n_q_heads*head_dim] */
    dflash_matrix wg;         /* [intermediate, hidden]  SwiGLU gate */
    dflash_matrix wu;         /* [intermediate, hidden]  SwiGLU up */
    dflash_matrix wd;         /* [hidden, intermediate]  down */
    const float  *g_in;       /* [hidden]   input RMSNorm */
    const float  *g_post;     /* [hidden]   post-attention RMSNorm */
    const float  *g_q;        /* [head_dim] q head RMSNorm */
    const float  *g_k;        /* [head_dim] k head RMSNorm */
    /* DFlash2 conv wrap ([memra dflash module] "Dflash2Conv"); used iff
     * cfg.d2_groups > 0.  w_dyn: [2*G*2, hidden] in cfg.weight_dtype, output
     * laid out [half][group][tap].  base: f32 [2][hidden][2] = [half][channel][tap]. */
    dflash_matrix attn_w_dyn;
    const float  *attn_base;
    dflash_matrix mlp_w_dyn;
    const float  *mlp_base;
} dflash_layer_weights;

/* All drafter weights ([DflashDraft] fields "fc", "hidden_norm", "norm",
 * "layers"). */
typedef struct dflash_weights {
    dflash_matrix fc;                     /* [hidden, n_taps*hidden] */
    const float  *g_hidden_norm;          /* [hidden] */
    const float  *g_norm;                 /* [hidden] final norm */
    const dflash_layer_weights *layers;   /* host array of cfg.n_layers entries */
} dflash_weights;

/* Draft KV cache ([memra dflash module] "DflashKv"; one per sequence, as
 * [atlas dflash_head] "DflashProposerState").  It holds, per layer, the
 * normed+roped ctx K and the raw ctx V, append-only in committed order.
 *
 * Contiguous storage (page_rows = 0):
 *   k: device, [n_layers][n_kv_heads][capacity][head_dim]   (row-major rows)
 *   v: device, [n_layers][n_kv_heads][capacity / 32][head_dim][32]
 *      (transposed per tile of 32 rows: row r, dimension j at
 *      [r / 32][j][r % 32], so that a 32-key block's V is one contiguous run
 *      and the attention's P.V product streams contiguous keys)
 *   capacity is a positive multiple of 64.
 *
 * Paged storage (page_rows > 0; [atlas dflash_head] "DflashProposerState":
 * one paged cache per drafter layer, one block table shared by all layers):
 *   k: device, [n_layers][pool_pages][n_kv_heads][page_rows][head_dim]
 *   v: device, [n_layers][pool_pages][n_kv_heads][page_rows / 32][head_dim][32]
 *   block_table: device int32 [capacity / page_rows]; logical row r lives in
 *      physical page block_table[r / page_rows], row r % page_rows, of every
 *      layer.  page_rows is a positive multiple of 64 that divides capacity;
 *      pool_pages >= 1.  Entries must lie in [0, pool_pages) for every page
 *      the call touches (the kernels clamp other values into the pool, so a
 *      bad table gives wrong results, never an access outside it).
 *
 * Context window ([atlas dflash_head] "dflash_ctx_cap": the drafter attends
 * only the most recent target positions): ctx_cap = 0 attends every
 * committed row; ctx_cap = N > 0 attends committed rows
 * [max(0, len - N), len) plus the block.  Rows before the window are never
 * read, so a paged caller may recycle pages that lie wholly before it.
 *
 * Both are in cfg.kv_dtype.  Rows [0, len) are committed.  forward_round
 * overwrites rows [len, len+b) with the block's K/V while it runs, and never
 * commits them.  A struct with page_rows = ctx_cap = 0 (the zero fill of the
 * last four fields) is the plain contiguous cache. */
typedef struct dflash_kv {
    void   *k;
    void   *v;
    int32_t capacity;
    int32_t len;
    int32_t page_rows;
    int32_t pool_pages;
    const int32_t *block_table;
    int32_t ctx_cap;
} dflash_kv;

typedef struct dflash_model dflash_model;   /* opaque host handle */

/* Validate cfg and weights, precompute the rope tables on the host (plain:
 * inv_freq[j] = base^(-2j/d); YaRN: divided by the per-dimension YaRN ramp
 * factor, and mscale = 0.1*ln(factor)+1, as [DflashDraft] "rope_yarn"
 * describes), and return a host handle in *out.  The weight pointers are
 * borrowed: the caller keeps them alive and unchanged while the model is
 * used.  Makes no HIP call. */
int dflash_load_weights(const dflash_cfg *cfg, const dflash_weights *w, dflash_model **out);

/* Release a handle from dflash_load_weights (NULL is allowed). */
void dflash_free(dflash_model *m);

/* Bytes of device memory that dflash_pack_weights needs for this model on
 * the current device (the layout depends on the device's CU count).
 * Returns 0 for a model without layers, and 0 with dflash_last_error set if
 * m is NULL or no device is usable.  Makes no allocation. */
size_t dflash_packed_bytes(const dflash_model *m);

/* Rearrange the layer GEMM weights (the [DflashDraft] layer fields wq, wk,
 * wv, wo, wg, wu, wd and, with the DFlash2 wrap, the dynamic-coefficient
 * projections) into `dst`, in the order in which forward_round streams them:
 * per layer and projection, per workgroup of the round kernel, contiguous
 * 8 KiB runs.  The values are copied unchanged (same dtype; fp8 row scales
 * stay where dflash_load_weights found them).
 *   dst  : device memory of >= dflash_packed_bytes(m) bytes, 256-byte
 *          aligned, owned by the caller, kept alive and unchanged while the
 *          model is used.  Borrowed like the weights themselves.
 * forward_round and forward_full fail with DFLASH_E_INVAL until this has been
 * called, or if the current device's CU count differs from the one packed
 * for.  Asynchronous on `stream`: calls on other streams must be ordered
 * after it by the caller.  Call again after changing the weights.
 * Errors: DFLASH_E_INVAL (null/misaligned dst, too small), DFLASH_E_HIP (no
 * usable device, launch error); nothing is enqueued on an argument error. */
int dflash_pack_weights(dflash_model *m, void *dst, size_t bytes, void *stream);

/* Bytes of device workspace (the per-step scratch of [atlas dflash_head]
 * "DflashScratch") needed by calls that process up to `max_rows` ctx rows at
 * once: ctx_features t, ingest_ctx t, or forward_full n.  The workspace must
 * be 256-byte aligned and zero-filled once before its first use.  It then
 * belongs to one device: the round kernel's grid-barrier counters only grow,
 * and their meaning depends on that device's CU count.  The other counters
 * are left at zero after every call.  Returns 0 if max_rows < 0. */
size_t dflash_workspace_bytes(const dflash_model *m, int32_t max_rows);

/* Context features ([DflashDraft] "ctx_features"): feats = hidden_norm(fc(taps)).
 *   taps : device f32 [t, n_taps*hidden], the raw tapped target states, taps
 *          concatenated in order along each row.
 *   feats: device f32 [t, hidden] (written).
 * t = 0 is a no-op.  Needs t <= the workspace's max_rows. */
int dflash_ctx_features(const dflash_model *m, const float *taps, int32_t t,
                        float *feats, void *ws, size_t ws_bytes, void *stream);

/* Allocation-free variant of dflash_ctx_features, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation): same arguments and result, but no
 * workspace.  Its scratch (the fc GEMM's split-K partial sums and counters,
 * 4 MiB + 64 KiB) is a static device array inside the library, one per
 * device, held until the process ends; the first call on a device looks up
 * that array's address and enqueues a kernel that zeroes its counters.  The
 * call allocates nothing (no hipMalloc, no allocating library routine).
 * t <= DFLASH_NOALLOC_MAX_ROWS, else DFLASH_E_INVAL.  Every call on one
 * device shares that device's array: two such calls that overlap on one
 * device (different streams, or different threads without ordering) race
 * and give wrong results; calls ordered on one stream are fine. */
#define DFLASH_NOALLOC_MAX_ROWS 65536
int dflash_ctx_features_noalloc(const dflash_model *m, const float *taps, int32_t t, float *feats, void *stream);

/* Append t committed ctx rows to the draft KV cache ([DflashDraft]
 * "ingest_ctx").  Per layer: k/v projections of the features, k head-norm,
 * rope (times the YaRN mscale), and the rows stored at kv->len.  Then
 * kv->len += t on the host, at enqueue time.
 *   feats  : device f32 [t, hidden] (from dflash_ctx_features).
 *   pos_new: device int32 [t], the rows' absolute positions.
 * DFLASH_E_CAPACITY if kv->len + t > kv->capacity. */
int dflash_ingest_ctx(const dflash_model *m, dflash_kv *kv, const float *feats,
                      const int32_t *pos_new, int32_t t, void *ws, size_t ws_bytes,
                      void *stream);

/* ingest_ctx for n_seqs sequences at once ([atlas dflash_head]
 * "DflashProposerState": one cache per sequence): t new rows per sequence,
 * whose k|v projections share one pass over each layer's W_k / W_v.
 *   feats  : device f32 [n_seqs][t][hidden]; pos_new: device int32 [n_seqs][t].
 *   kvs    : host array of n_seqs caches with distinct storage; each
 *            kvs[i].len += t on the host, at enqueue time.
 * 1 <= n_seqs <= 8; n_seqs * t <= the workspace's max_rows.  Any cache's
 * capacity error rejects the whole call (no len changes). */
int dflash_ingest_ctx_batch(const dflash_model *m, dflash_kv *kvs, int32_t n_seqs, const float *feats,
                            const int32_t *pos_new, int32_t t, void *ws, size_t ws_bytes, void *stream);

/* One drafting round over the cached ctx K/V ([DflashDraft] "forward_round").
 * Only the b block rows are projected per layer.  Their K/V land transiently
 * at rows [kv->len, kv->len + b), and attention over all kv->len + b keys is
 * full and non-causal.  kv->len is unchanged.
 *   noise_emb: device f32 [b, hidden], the block's input embeddings.
 *   pos_block: device int32 [b], the block rows' absolute positions.
 *   out      : device f32 [b, hidden], the final normed hidden states (fed to
 *              the target's lm_head by the caller).
 * 1 <= b <= 16.  DFLASH_E_CAPACITY if kv->len + b > kv->capacity.
 * A paged or windowed cache (page_rows or ctx_cap set) runs the layered
 * path of dflash_forward_round_batch with one sequence, so `ws` must then
 * hold dflash_batch_workspace_bytes(m, 1, 0) bytes; a plain contiguous
 * cache runs the persistent round kernel. */
int dflash_forward_round(const dflash_model *m, dflash_kv *kv, const float *noise_emb,
                         const int32_t *pos_block, int32_t b, float *out,
                         void *ws, size_t ws_bytes, void *stream);

/* Bytes of device workspace for the layered round path: calls of
 * dflash_forward_round_batch over up to n_seqs sequences, and calls on a
 * paged or windowed cache (n_seqs = 1), that also process up to max_rows
 * ctx rows at once (as dflash_workspace_bytes).  It is
 * dflash_workspace_bytes(m, max_rows) plus the stacked block rows' buffers
 * and the attention partials.  Such a workspace serves every other call
 * too.  Returns 0 for n_seqs outside [1, 8] or max_rows < 0. */
size_t dflash_batch_workspace_bytes(const dflash_model *m, int32_t n_seqs, int32_t max_rows);

/* Batched round: one drafting round of n_seqs independent sequences, each
 * over its own draft KV cache ([atlas dflash_head] "DflashProposerState"),
 * with the same result per sequence as n_seqs forward_round calls.  The
 * sequences' n_seqs * b block rows go through every projection together,
 * so each layer's weights are read once per call instead of once per
 * sequence.  The steps are separate kernels (RMSNorm, the projections,
 * q/k head-norm + rope + block K/V stores, split-K attention, split merge).
 *   kvs       : host array of n_seqs caches (distinct storage; contiguous or
 *               paged, with or without a window); lens unchanged.
 *   noise_emb : device f32 [n_seqs][b][hidden].
 *   pos_block : device int32 [n_seqs][b].
 *   out       : device f32 [n_seqs][b][hidden].
 *   ws        : >= dflash_batch_workspace_bytes(m, n_seqs, 0) bytes, 256-byte
 *               aligned (zero-filled once, like every workspace).
 * 1 <= n_seqs <= 8, 1 <= b <= 16.  DFLASH_E_UNSUPPORTED for an f32 KV
 * cache.  No grid-wide barriers: unlike the persistent round kernel, it may
 * share the device with other work. */
int dflash_forward_round_batch(const dflash_model *m, dflash_kv *kvs, int32_t n_seqs, const float *noise_emb,
                               const int32_t *pos_block, int32_t b, float *out, void *ws, size_t ws_bytes,
                               void *stream);

/* First-light forward ([DflashDraft] "forward"): full non-causal attention
 * over [ctx features ; block], with no persistent cache.  It runs
 * ctx_features over all n ctx rows, resets `scratch` to len 0, ingests the n
 * rows, and runs one round.  `scratch` is caller KV storage with
 * capacity >= n + b; afterwards its len is n.
 *   taps: device f32 [n, n_taps*hidden]; noise_emb: device f32 [b, hidden]
 *   pos : device int32 [n + b], the ctx positions, then the block positions.
 *   out : device f32 [b, hidden].
 * n >= 0, 1 <= b <= 16, and n <= the workspace's max_rows.  scratch may be
 * paged (then ws must hold dflash_batch_workspace_bytes(m, 1, n) bytes); it
 * must have no window (ctx_cap = 0): the first-light forward attends
 * everything. */
int dflash_forward_full(const dflash_model *m, const float *taps, const float *noise_emb,
                        const int32_t *pos, int32_t n, int32_t b, float *out,
                        dflash_kv *scratch, void *ws, size_t ws_bytes, void *stream);

/* Synchronise `stream`, then report whether a round kernel that used `ws`
 * failed.  The persistent round kernel needs one resident workgroup per CU;
 * if some could not start, its barriers time out after about a second, it
 * writes NaN over its output rows and sets a flag in the workspace.  The
 * kernel also sets the flag (and writes NaN) if it finds its arguments
 * somewhere other than where its code expects them.  Returns DFLASH_E_HIP
 * (and clears the flag and the barrier counters, so that later rounds work
 * again) if the flag was set, else DFLASH_OK.  A diagnostic call: it blocks
 * the host. */
int dflash_workspace_status(const dflash_model *m, void *ws, size_t ws_bytes, void *stream);

/* Message for the calling thread's last error ("" if none). */
const char *dflash_last_error(void);

/* Host-side copy of the rope tables of a loaded model: inv_freq[head_dim/2]
 * (f64) and the q/k scale.  Lets a caller check them against their own.
 * Makes no HIP call. */
int dflash_rope_table(const dflash_model *m, double *inv_freq, int32_t n, double *mscale);

#ifdef __cplusplus
}
#endif
#endif /* DFLASH_H */
