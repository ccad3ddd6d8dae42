// Internal interface between the host API (api.cpp) and the gfx950 kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace dfl {

// ---- skinny GEMM:  Y[M, N] (epi)= A[M, K] . W[N, K]^T  ---------------------
enum { EPI_STORE = 0, EPI_ADD = 1, EPI_SWIGLU = 2 };

struct GemmSeg {
    const void  *w;      // [n, K] in the weight dtype
    const float *scale;  // fp8 row scales [n], else nullptr
    int          n;      // output columns of this segment (multiple of 16)
};

struct GemmArgs {
    const float *A; int lda; int M; int K;
    GemmSeg seg[3]; int nseg;     // the output columns are the segments side by side
                                  // (EPI_SWIGLU: seg[0] = gate, seg[1] = up, same n)
    float *Y; int ldy;
    int epi;
    int wtype;
    // filled by the launcher
    int ksplit, kchunk, mt, ngroups, mgroups;   // ngroups: 64-column groups
    float *part; unsigned *cnt;
};

// workspace needed by gemm split-K partials / counters
constexpr size_t GEMM_PART_FLOATS = 1u << 20;   // 4 MiB
constexpr int    GEMM_MAX_COUNTERS = 1 << 14;

// Plans the split and launches.  part/cnt must point at workspace regions of
// GEMM_PART_FLOATS floats / GEMM_MAX_COUNTERS counters (zero-filled counters).
hipError_t gemm(GemmArgs a, float *part, unsigned *cnt, hipStream_t s);
// number of workgroups a plan would use (for tests / diagnostics)
int gemm_plan(GemmArgs &a);

// ---- RMSNorm over rows ------------------------------------------------------
// y[r] = g * x[r] / sqrt(mean(x[r]^2) + eps); if xcopy, also xcopy[r] = x[r]
hipError_t rmsnorm(const float *x, int ldx, const float *g, float *y, int ldy,
                   float *xcopy, int rows, int H, float eps, hipStream_t s);

// ---- q/k head norm + rope (+ mscale) and KV stores --------------------------
constexpr int MAX_HALF_DIM = 64;
struct RopeArgs {
    const float *src; int ld;     // [rows, ld] projection output
    int q_off, k_off, v_off;      // column offsets; q_off < 0: no q heads
    const float *g_q, *g_k;
    const int32_t *pos;
    int rows, nq, nkv, d;
    float eps; float mscale;
    float *q_out;                 // [rows][nq][d] f32
    void *kc; void *vc;           // this layer's K [nkv][cap][d] and V [nkv][d][cap]
    int cap; int row0;            // cache rows row0 .. row0 + rows - 1
    int kv_f32;                   // 1: f32 cache, 0: bf16 cache
    double inv_freq[MAX_HALF_DIM];
};
hipError_t qk_norm_rope(const RopeArgs &a, hipStream_t s);


}  // namespace dfl
