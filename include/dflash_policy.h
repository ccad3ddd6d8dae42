/*
 * dflash_policy.h — host-side policy functions around the DFlash drafter:
 * the verify-side accept rules and confidence windows, and the DFlash2
 * candidate selector.
 *
 * Sources:
 *  [memra dflash module]  docs.rs memra_engine::dflash, module index, sections
 *                         "dspark_accept_prefix", "rejection_accept_len",
 *                         "dspark_confidence_vt", "dspark_slot_confidence_vt",
 *                         "dflash2_walk_greedy", "dflash2_walk_sampled".
 *  [DflashDraft]          docs.rs memra_engine::dflash::DflashDraft, section
 *                         "dflash2_propose_greedy".
 *
 * The accept rules, windows and walks are pure host code over caller-owned
 * host arrays: no HIP call, no allocation, no global state.  Each returns
 * DFLASH_OK, or DFLASH_E_INVAL for a null pointer, a negative count or a
 * value outside its stated range, in which case no output is written.  The
 * two dflash2_propose_* calls at the end run device kernels and follow the
 * conventions of dflash.h (dflash_last_error holds their messages).
 */
#ifndef DFLASH_POLICY_H
#define DFLASH_POLICY_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Accepted prefix of a round's candidates against the target's verify
 * argmaxes ([memra dflash module] "dspark_accept_prefix").
 *   cand[0]           the round's anchor (already decided);
 *   cand[1..n_cand-1] the drafts;
 *   vam[j]            the target's argmax for the position after anchor + j.
 * *m = the number of leading drafts with cand[j] == vam[j-1]; cand[1..m]
 * are committed and vam[m] is the next anchor, so m <= n_vam - 1 as well as
 * m <= n_cand - 1.  Needs n_cand >= 1 and n_vam >= 1. */
int dflash_accept_prefix(const int32_t *cand, int32_t n_cand, const int32_t *vam, int32_t n_vam, int32_t *m);

/* Rejection-sampling prefix walk ([memra dflash module]
 * "rejection_accept_len"): draft j is accepted while u[j] * q[j] < p[j]
 * (strict, float64), where p and q are the target's and the proposal's
 * filtered probabilities of the drafted tokens and u the slots' uniforms.
 * *accepted = the number of leading accepted drafts (0..n). */
int dflash_rejection_accept_len(const double *p, const double *q, const double *u, int32_t n, int32_t *accepted);

/* Verify-window sizing from cumulative survival ([memra dflash module]
 * "dspark_confidence_vt").  raws[k] is the accept-rate head's pre-sigmoid
 * score of draft slot k+1; S_k = prod_{j<=k} sigmoid(raws[j]) in float64;
 * leading slots are kept while S_k >= tau.  *vt = 1 + kept, clamped to
 * [2, vt_cap]; vt_cap >= 2. */
int dflash_confidence_vt(const float *raws, int32_t n, double tau, int32_t vt_cap, int32_t *vt);

/* Verify-window sizing from per-slot confidence ([memra dflash module]
 * "dspark_slot_confidence_vt"): the longest prefix of slots whose own
 * sigmoid(raws[k]) >= tau (float64); the first slot below tau ends it.
 * *vt = 1 + kept, clamped to [2, vt_cap]; vt_cap >= 2. */
int dflash_slot_confidence_vt(const float *raws, int32_t n, double tau, int32_t vt_cap, int32_t *vt);

/* ---- DFlash2 candidate selector --------------------------------------- */
#define DFLASH2_MAX_TOPK 64
#define DFLASH2_MAX_RANK 256

/* The selector's trained tensors ([memra dflash module] "dflash2_walk_greedy":
 * host-resident bf16 codebooks; [DflashDraft] "dflash2_propose_greedy": the
 * rank-r hidden projection).
 *   pred_codebook, succ_codebook: host, bf16 bit patterns [vocab][rank].
 *   w_hidden_proj: device, bf16 [rank][hidden] (used by the device step of
 *                  dflash2_propose_greedy only; may be NULL for the walks).
 * 1 <= top_k <= DFLASH2_MAX_TOPK, 1 <= rank <= DFLASH2_MAX_RANK. */
typedef struct dflash2_selector {
    int32_t vocab;
    int32_t rank;
    int32_t top_k;
    const uint16_t *pred_codebook;
    const uint16_t *succ_codebook;
    const void *w_hidden_proj;
} dflash2_selector;

/* Greedy selector walk ([memra dflash module] "dflash2_walk_greedy").  For
 * draft slot p = 0..nd-1, with prev the previous slot's chosen token (the
 * anchor for p = 0):
 *   score(k) = unary[p][k] + sum_r pred[prev][r] * hproj[p][r] * succ[cand[p][k]][r]
 * in float64 over the stored values; path[p] = cand[p][argmax_k score], ties
 * to the lowest k.  unary, cand: [nd][top_k] (the slot's top-k draft logits
 * and their token ids); hproj: [nd][rank].  A token id outside [0, vocab)
 * is DFLASH_E_INVAL (path may then be partly written). */
int dflash2_walk_greedy(const dflash2_selector *s, const float *unary, const int32_t *cand, const float *hproj,
                        int32_t nd, int32_t anchor, int32_t *path);

/* Sampled selector walk ([memra dflash module] "dflash2_walk_sampled"): the
 * same pair scores become a softmax at `temperature` (> 0) per slot; the
 * slot's uniform uniforms[p] in [0, 1) picks the first candidate whose
 * cumulative probability (candidate order) exceeds it (the last one if
 * rounding leaves it at or above the total), and the chosen token seeds
 * the next slot.  Writes path[nd], q_chosen[nd] and q_rows[nd][top_k] (the
 * slot's candidate probabilities); q_chosen[p] == q_rows[p][chosen]. */
int dflash2_walk_sampled(const dflash2_selector *s, const float *unary, const int32_t *cand, const float *hproj,
                         int32_t nd, int32_t anchor, double temperature, const double *uniforms, int32_t *path,
                         double *q_chosen, double *q_rows);

/* Device step of the DFlash2 proposal ([DflashDraft] "dflash2_propose_greedy"):
 * for the draft rows 1..b-1 (row 0 is the anchor row, not a draft), the
 * top_k largest draft logits of each row (larger first, equal values in
 * increasing index order) with their token ids, and the rank-r projection
 * hproj = hidden . w_hidden_proj^T (f32 accumulation).  Asynchronous on
 * `stream`; makes no host synchronisation.
 *   m            : a loaded model (its hidden size and workspace layout).
 *   sel          : vocab, rank, top_k and the device w_hidden_proj (bf16
 *                  [rank][hidden]); the codebooks are not used here.
 *   draft_logits : device f32 [b][vocab] (the target lm_head applied to the
 *                  round's output; finite values).
 *   hidden       : device f32 [b][hidden] (the round's output rows).
 *   packed       : device, nd*(2*top_k + rank) 32-bit words, nd = b - 1:
 *                  f32 values [nd][top_k], int32 ids [nd][top_k], f32
 *                  hproj [nd][rank].
 *   ws           : the model's workspace (dflash_workspace_bytes).
 * 2 <= b <= 16.  DFLASH_E_UNSUPPORTED if the top-k candidates of the draft
 * rows do not fit the workspace's 4 MiB scratch region (about
 * (b-1) * vocab * top_k / 128 bytes: vocabularies of up to ~1.5M tokens at
 * top_k 64). */
int dflash2_propose_prepare(const struct dflash_model *m, const dflash2_selector *sel, const float *draft_logits,
                            const float *hidden, int32_t b, uint32_t *packed, void *ws, size_t ws_bytes, void *stream);

/* The whole greedy proposal ([DflashDraft] "dflash2_propose_greedy"): the
 * device step into the workspace, ONE device-to-host copy of its
 * nd*(2*top_k + rank) words, then dflash2_walk_greedy from `anchor` on the
 * host codebooks.  Writes the nd = b - 1 drafted tokens to host `drafts`.
 * Synchronises `stream` (the walk needs the copied values).  The copy lands
 * in pinned host memory: each calling host thread allocates one buffer of
 * 15 * (2 * DFLASH2_MAX_TOPK + DFLASH2_MAX_RANK) words (23 KiB) on its first
 * call and keeps it until the process ends. */
int dflash2_propose_greedy(const struct dflash_model *m, const dflash2_selector *sel, const float *draft_logits,
                           const float *hidden, int32_t b, int32_t anchor, int32_t *drafts, void *ws, size_t ws_bytes,
                           void *stream);

#ifdef __cplusplus
}
#endif
#endif /* DFLASH_POLICY_H */
