// Host/device interface of the batched multi-sequence round (batch.hip).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kvview.h"

namespace dfl {

constexpr int BATCH_MAX_SEQ = 8;          // sequences per call (128 stacked rows at b = 16)
constexpr int BATCH_MAX_ITEMS = 512;      // attention items (sequence, kv head, split) per launch
constexpr int BATCH_MAX_SPLITS = 64;      // key splits per (sequence, kv head): one per lane in the merge
constexpr int BATCH_ATTN_THREADS = 512;   // eight waves: one q head each (G <= 8)
constexpr int BATCH_CHUNK_KEYS = 64;      // keys staged per step; key splits are multiples of it

struct BatchSeq {
    KvView kv;
    int len;          // committed rows; the block goes to [len, len + b)
    int win_lo;       // first committed row attended (context window), 0 without one
};

struct BatchArgs {
    BatchSeq seq[BATCH_MAX_SEQ];
    int S, b, nq, nkv, G, d, qd, kvd, layer;
    const float *qkv; int qkv_ld;   // [S*b][qd + 2 kvd] raw projections
    const float *g_q, *g_k;
    const int32_t *pos;             // [S][b] block positions
    float eps, mscale, qscale;      // qscale = log2(e) / sqrt(d)
    double inv_freq[64];
    uint16_t *q;                    // [S][nkv][G][16][d] bf16
    int nsplit, kps;                // key splits per (sequence, kv head), keys per split
    float *po, *pml;                // [S][nkv][nsplit][G][16][d], [...][16][2]
    float *attn;                    // [S*b][qd]
};

hipError_t batch_qk_rope_launch(const BatchArgs &a, hipStream_t s);
// DFlash2 conv wrap: D[rows][nj] = xn . W_dyn^T (weight type wt), and the
// two-tap causal conv over each sequence's b rows (dst = or += result)
hipError_t d2_dyn_launch(const float *xn, int H, const void *w, const float *scale, int wt, int nj, int rows, float *D,
                         hipStream_t s);
hipError_t d2_conv_launch(const float *src, const float *D, int half, const float *base, int H, int G, int b, int rows,
                          float *dst, bool accumulate, hipStream_t s);
// attention splits, then their merge into a.attn
hipError_t batch_attn_launch(const BatchArgs &a, hipStream_t s);

}  // namespace dfl
