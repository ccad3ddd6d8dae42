// Host/device interface of the persistent forward_round kernel (round.hip).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dfl {

constexpr int RND_THREADS = 512;     // 8 waves per workgroup, one workgroup per CU
constexpr int RND_MAXL = 8;          // layers per launch (weight table in the kernel arguments)
constexpr int MAXSLOT = 4;           // partial tiles one workgroup may leave per GEMM
constexpr int MAX_NWG = 320;         // workgroups (CUs) the workspace is sized for
constexpr int RND_MAX_SPLITS = 64;   // attention key splits per kv head
// barrier state words (each group 128 bytes apart)
constexpr int BAR_XCNT = 0, BAR_GCNT = 256, BAR_GEN = 288, BAR_ERR = 544, BAR_WORDS = 576;

struct MatRef {
    const void *w;       // [n][K] in the weight dtype
    const float *s;      // fp8 row scales [n], else nullptr
    int n;               // output columns (a multiple of 16)
    int pad;
};

struct GemmPlanDev {
    int K;               // reduction length
    int steps;           // K steps per 128-column group
    int total;           // groups * steps
    int upw;             // units per workgroup
};

struct LayerRefs {
    MatRef q, k, v, o, g, u, d;
    MatRef aw, mw;                   // DFlash2 dynamic-kernel projections [4G][H] (attention, MLP)
    const float *g_in, *g_post, *g_q, *g_k;
    const float *abase, *mbase;      // DFlash2 static taps f32 [2][H][2]
};

// Scalars of a launch (kept in registers by value).
struct RoundScalars {
    int H, nq, nkv, d, I, qd, kvd;
    int wt, kv_f32;
    int b, len, cap;
    int nl, first, last;             // layers in this launch; first / last launch of the call
    float eps, mscale, scale_log2;
    int attn_nsplit, attn_kps, qpad;
    const float *noise;              // [b][H]
    const int32_t *pos;              // [b]
    float *out;                      // [b][H]
    const float *g_norm;
    char *kc, *vc;                   // cache bases of this launch's first layer
    long long kv_lstride;            // bytes per layer (K and V alike)
    float *X, *ssq, *Q, *O, *Z, *part, *attn_o, *attn_ml;
    unsigned *bar;
    unsigned long long *trace;       // phase timestamps (workgroup 0), or nullptr
    GemmPlanDev p_qkv, p_o, p_gu, p_d;
    int d2;                          // DFlash2 conv groups G (0: no conv wrap)
    float *d2_Da, *d2_Dm;            // per-row dynamic coefficients [16][4G] (attention, MLP)
    float *d2_rinv;                  // 1/rms of the rows the last coefficient phase normalised [16]
};
constexpr int RND_TRACE_WORDS = 1024;
constexpr int RND_MAX_D2 = 64;       // DFlash2 groups G: 4G coefficients per row

// Kernel arguments.  The arrays are indexed at run time, so the kernel reads
// them in place from the kernel-argument segment.
struct RoundArgs {
    RoundScalars s;
    double inv_freq[64];
    LayerRefs L[RND_MAXL];
};

// Kernel launch (one workgroup per CU, nwg of them).
hipError_t round_launch(const RoundArgs &a, int nwg, hipStream_t s);

}  // namespace dfl
