// Internal interface between the host API (api.cpp) and the gfx950 kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "kvview.h"

namespace dfl {

// ---- skinny GEMM:  Y[M, N] (epi)= A[M, K] . W[N, K]^T  ---------------------
enum { EPI_STORE = 0, EPI_ADD = 1, EPI_SWIGLU = 2 };

struct GemmSeg {
    const void  *w;      // [n, K] in the weight dtype
    const float *scale;  // fp8 row scales [n], else nullptr
    int          n;      // output columns of this segment (multiple of 16)
};

constexpr int GEMM_MAX_SEG = 16;

struct GemmArgs {
    const float *A; int lda; int M; int K;
    GemmSeg seg[GEMM_MAX_SEG]; int nseg;  // the output columns are the segments side by side
                                          // (EPI_SWIGLU: seg[0] = gate, seg[1] = up, same n)
    float *Y; int ldy;
    int epi;
    int wtype;
    int planes;       // bf16 / fp8 weights: activations as 2 bf16 planes (hi + lo; also when 0) or 1 (bf16 rounding)
    // filled by the launcher
    int ksplit, kchunk, mt, ngroups, mgroups;   // ngroups: 64-column groups
    float *part; unsigned *cnt;
};

// workspace needed by gemm split-K partials / counters
constexpr size_t GEMM_PART_FLOATS = 1u << 20;   // 4 MiB
constexpr int    GEMM_MAX_COUNTERS = 1 << 14;
constexpr int    GEMM_CUS = 256;                  // compute units the K-split plan is balanced for (MI355X)

// Plans the split and launches.  part/cnt must point at workspace regions of
// GEMM_PART_FLOATS floats / GEMM_MAX_COUNTERS counters (zero-filled counters).
// The plan never needs more: it lowers the K split until the partials fit.
// Shapes gemm_tall_ok accepts run the tiled kernel instead (no workspace).
hipError_t gemm(GemmArgs a, float *part, unsigned *cnt, hipStream_t s);

// Tiled kernel for tall activations (gemm_tall.hip): bf16 weights, M >= 256,
// store epilogue, K a multiple of 64, every segment's width a multiple of
// 128, and at least GEMM_CUS work items (tiles of 128 x 128, each split
// into two K halves when the tiles alone are fewer).  The K halves use two
// of the zero-filled counters per tile in `cnt` and leave them zero.
bool gemm_tall_ok(const GemmArgs &a);
hipError_t gemm_tall(const GemmArgs &a, unsigned *cnt, hipStream_t s);

// ---- DFlash2 proposal: top-k over draft logits, rank-r hidden projection ----
constexpr int TOPK_CHUNK = 1024;     // candidates per wave and stage (16 per lane)
constexpr int TOPK_MERGE_LISTS = 256; // first-stage lists one merge wave takes (4 per lane)
constexpr int TOPK_MERGE_LDS = 57344; // LDS bytes of those lists (8 per entry; 8 KiB more for the ranking)
constexpr int TOPK_QUOTA = 8;         // entries per chunk the first stage keeps before the merge
int topk_chunks(int n);
// entries part_v / part_i must hold for rows of a vocabulary (k <= 64, so
// each stage shrinks the candidates at least 16-fold)
size_t topk_scratch_entries(int rows, int vocab, int k);
// Per row: the k largest logits (larger first, then lower index) and their
// indices; with them, hout[r][j] = hidden[r] . w[j] (as hidden_projection,
// in the same launch as the last top-k step where it can be).
hipError_t topk_rows(const float *logits, long long ld, int rows, int vocab, int k, float *part_v, int32_t *part_i,
                     float *vals, int32_t *idx, const float *hidden, int H, const void *w, int rank, float *hout,
                     hipStream_t s);
// out[r][j] = hidden[r] . w[j] for bf16 w [rank][H], f32 accumulation
hipError_t hidden_projection(const float *hidden, int H, const void *w, int rank, int rows, float *out, hipStream_t s);

// ---- allocation-free entry point: one static device scratch array ---------
// The split-K partials, then the counters, of the ctx_features GEMM.
constexpr size_t NOALLOC_PART_BYTES = 4 * GEMM_PART_FLOATS;
constexpr size_t NOALLOC_SCRATCH_BYTES = NOALLOC_PART_BYTES + sizeof(unsigned) * GEMM_MAX_COUNTERS;
// Device address of the current device's scratch array (looked up, and its
// counters cleared by a kernel on `stream`, on the first call per device).
hipError_t noalloc_scratch(void **out, hipStream_t stream);
// number of workgroups a plan would use (for tests / diagnostics)
int gemm_plan(GemmArgs &a);

// ---- RMSNorm over rows ------------------------------------------------------
// y[r] = g * x[r] / sqrt(mean(x[r]^2) + eps); if xcopy, also xcopy[r] = x[r]
hipError_t rmsnorm(const float *x, int ldx, const float *g, float *y, int ldy,
                   float *xcopy, int rows, int H, float eps, hipStream_t s);

// ---- k head norm + rope (+ mscale) and KV stores, several layers at once ----
constexpr int MAX_HALF_DIM = 64;
constexpr int ROPE_MAX_LAYERS = 8;
constexpr int ROPE_MAX_SEQ = 8;
struct RopeArgs {
    const float *src; int ld;     // [rows, ld] projection output; layer i's k heads start at
    int lstride;                  // column i * lstride, its v heads kvd = nkv * d further on
    int nl;                       // layers in this launch (<= ROPE_MAX_LAYERS)
    int layer0;                   // cache layer of launch layer 0
    const float *g_k[ROPE_MAX_LAYERS];
    KvView kv[ROPE_MAX_SEQ];      // the caches (contiguous or paged) of the sequences
    int row0[ROPE_MAX_SEQ];       // sequence s's rows go to its cache rows row0[s] ..
    int seq_rows;                 // rows per sequence: row r belongs to sequence r / seq_rows
    const int32_t *pos;
    int rows, nkv, d;
    float eps; float mscale;
    int kv_f32;                   // 1: f32 cache, 0: bf16 cache
    double inv_freq[MAX_HALF_DIM];
};
hipError_t kv_norm_rope(const RopeArgs &a, hipStream_t s);


}  // namespace dfl
