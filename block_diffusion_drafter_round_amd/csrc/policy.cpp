// Host-side policy functions of the drafter: the verify-side accept rules
// and confidence windows ([memra dflash module] "dspark_accept_prefix",
// "rejection_accept_len", "dspark_confidence_vt",
// "dspark_slot_confidence_vt") and the DFlash2 candidate-selector walks
// ("dflash2_walk_greedy", "dflash2_walk_sampled").  Pure functions over
// host arrays; include/dflash_policy.h states the contracts.
#include <cmath>
#include <cstdint>
#include <cstring>

#include "dflash.h"
#include "dflash_policy.h"

namespace {

double sigmoid(double x) {
    if (x >= 0) return 1.0 / (1.0 + std::exp(-x));
    const double e = std::exp(x);
    return e / (1.0 + e);
}

int32_t clamp_vt(int32_t kept, int32_t vt_cap) {
    int32_t vt = 1 + kept;
    if (vt < 2) vt = 2;
    return vt > vt_cap ? vt_cap : vt;
}

float bf16_to_f32(uint16_t h) {
    const uint32_t u = (uint32_t)h << 16;
    float f;
    std::memcpy(&f, &u, 4);
    return f;
}

// pair scores of one slot: unary[k] + sum_r pred[prev][r] * hproj[r] * succ[cand[k]][r]
// (float64 over the stored values, r in increasing order); returns false on
// an out-of-vocabulary token.  pred[prev][r] * hproj[r] is formed once per
// slot (the product is evaluated left to right either way), and four
// candidates' sums run side by side, each in its own order, so every score
// has the same bits as a one-at-a-time evaluation.
bool slot_scores(const dflash2_selector *s, const float *unary, const int32_t *cand, int32_t prev,
                 const float *hproj, double *score) {
    if (prev < 0 || prev >= s->vocab) return false;
    const int R = s->rank, K = s->top_k;
    for (int k = 0; k < K; ++k)
        if (cand[k] < 0 || cand[k] >= s->vocab) return false;
    const uint16_t *pv = s->pred_codebook + (size_t)prev * R;
    double w[DFLASH2_MAX_RANK];
    for (int r = 0; r < R; ++r) w[r] = (double)bf16_to_f32(pv[r]) * (double)hproj[r];
    int k = 0;
    for (; k + 4 <= K; k += 4) {
        const uint16_t *s0 = s->succ_codebook + (size_t)cand[k] * R, *s1 = s->succ_codebook + (size_t)cand[k + 1] * R,
                       *s2 = s->succ_codebook + (size_t)cand[k + 2] * R, *s3 = s->succ_codebook + (size_t)cand[k + 3] * R;
        double a0 = 0.0, a1 = 0.0, a2 = 0.0, a3 = 0.0;
        for (int r = 0; r < R; ++r) {
            a0 += w[r] * (double)bf16_to_f32(s0[r]);
            a1 += w[r] * (double)bf16_to_f32(s1[r]);
            a2 += w[r] * (double)bf16_to_f32(s2[r]);
            a3 += w[r] * (double)bf16_to_f32(s3[r]);
        }
        score[k] = (double)unary[k] + a0;
        score[k + 1] = (double)unary[k + 1] + a1;
        score[k + 2] = (double)unary[k + 2] + a2;
        score[k + 3] = (double)unary[k + 3] + a3;
    }
    for (; k < K; ++k) {
        const uint16_t *sv = s->succ_codebook + (size_t)cand[k] * R;
        double pair = 0.0;
        for (int r = 0; r < R; ++r) pair += w[r] * (double)bf16_to_f32(sv[r]);
        score[k] = (double)unary[k] + pair;
    }
    return true;
}

bool selector_ok(const dflash2_selector *s) {
    return s && s->pred_codebook && s->succ_codebook && s->rank > 0 && s->rank <= DFLASH2_MAX_RANK && s->top_k > 0 &&
           s->top_k <= DFLASH2_MAX_TOPK && s->vocab > 0;
}

}  // namespace

extern "C" {

int dflash_accept_prefix(const int32_t *cand, int32_t n_cand, const int32_t *vam, int32_t n_vam, int32_t *m) {
    if (!cand || !vam || !m || n_cand < 1 || n_vam < 1) return DFLASH_E_INVAL;
    int32_t k = 0;
    while (k + 1 < n_cand && k + 1 < n_vam && cand[k + 1] == vam[k]) ++k;
    *m = k;
    return DFLASH_OK;
}

int dflash_rejection_accept_len(const double *p, const double *q, const double *u, int32_t n, int32_t *accepted) {
    if (!accepted || n < 0 || (n > 0 && (!p || !q || !u))) return DFLASH_E_INVAL;
    int32_t k = 0;
    while (k < n && u[k] * q[k] < p[k]) ++k;
    *accepted = k;
    return DFLASH_OK;
}

int dflash_confidence_vt(const float *raws, int32_t n, double tau, int32_t vt_cap, int32_t *vt) {
    if (!vt || n < 0 || (n > 0 && !raws) || vt_cap < 2 || std::isnan(tau)) return DFLASH_E_INVAL;
    double surv = 1.0;
    int32_t kept = 0;
    for (; kept < n; ++kept) {
        surv *= sigmoid((double)raws[kept]);
        if (!(surv >= tau)) break;
    }
    *vt = clamp_vt(kept, vt_cap);
    return DFLASH_OK;
}

int dflash_slot_confidence_vt(const float *raws, int32_t n, double tau, int32_t vt_cap, int32_t *vt) {
    if (!vt || n < 0 || (n > 0 && !raws) || vt_cap < 2 || std::isnan(tau)) return DFLASH_E_INVAL;
    int32_t kept = 0;
    while (kept < n && sigmoid((double)raws[kept]) >= tau) ++kept;
    *vt = clamp_vt(kept, vt_cap);
    return DFLASH_OK;
}

int dflash2_walk_greedy(const dflash2_selector *s, const float *unary, const int32_t *cand, const float *hproj,
                        int32_t nd, int32_t anchor, int32_t *path) {
    if (!selector_ok(s) || nd < 0 || (nd > 0 && (!unary || !cand || !hproj || !path))) return DFLASH_E_INVAL;
    double score[DFLASH2_MAX_TOPK];
    int32_t prev = anchor;
    for (int p = 0; p < nd; ++p) {
        if (!slot_scores(s, unary + (size_t)p * s->top_k, cand + (size_t)p * s->top_k, prev, hproj + (size_t)p * s->rank,
                         score))
            return DFLASH_E_INVAL;
        int best = 0;
        for (int k = 1; k < s->top_k; ++k)
            if (score[k] > score[best]) best = k;          // strict: ties keep the lowest k
        prev = cand[(size_t)p * s->top_k + best];
        path[p] = prev;
    }
    return DFLASH_OK;
}

int dflash2_walk_sampled(const dflash2_selector *s, const float *unary, const int32_t *cand, const float *hproj,
                         int32_t nd, int32_t anchor, double temperature, const double *uniforms, int32_t *path,
                         double *q_chosen, double *q_rows) {
    if (!selector_ok(s) || nd < 0 || !(temperature > 0.0) || !std::isfinite(temperature)) return DFLASH_E_INVAL;
    if (nd > 0 && (!unary || !cand || !hproj || !uniforms || !path || !q_chosen || !q_rows)) return DFLASH_E_INVAL;
    double score[DFLASH2_MAX_TOPK];
    int32_t prev = anchor;
    const int K = s->top_k;
    for (int p = 0; p < nd; ++p) {
        if (!slot_scores(s, unary + (size_t)p * K, cand + (size_t)p * K, prev, hproj + (size_t)p * s->rank, score))
            return DFLASH_E_INVAL;
        double mx = score[0];
        for (int k = 1; k < K; ++k) mx = score[k] > mx ? score[k] : mx;
        double tot = 0.0;
        double *q = q_rows + (size_t)p * K;
        for (int k = 0; k < K; ++k) {
            q[k] = std::exp((score[k] - mx) / temperature);
            tot += q[k];
        }
        for (int k = 0; k < K; ++k) q[k] /= tot;
        int pick = K - 1;
        double acc = 0.0;
        for (int k = 0; k < K; ++k) {
            acc += q[k];
            if (uniforms[p] < acc) { pick = k; break; }
        }
        prev = cand[(size_t)p * K + pick];
        path[p] = prev;
        q_chosen[p] = q[pick];
    }
    return DFLASH_OK;
}

}  // extern "C"
