// Host/device interface of the streamed forward_round kernel (sround.hip).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dfl {

constexpr int SR_CW = 8;                      // compute waves per workgroup
constexpr int SR_THREADS = 64 * (SR_CW + 2);  // plus one loader and one service wave
constexpr int SR_PART = 1024;                 // one wave-wide load: 64 lanes x 16 bytes
constexpr int SR_SLOT = SR_CW * SR_PART;      // a ring slot holds one part per compute wave
constexpr int SR_NSLOT = 15;                  // ring slots (120 KiB of LDS)
constexpr int SR_DEPTH = 3;                   // slots the loader keeps in flight (3 x 8 loads)
constexpr int SR_MAXT = 4;                    // output tiles of 16 columns per workgroup and GEMM
constexpr int SR_MAXSTEP = 24;                // k steps of one wave per GEMM
constexpr int SR_ACTREG = 12;                 // 16-byte activation fragments a lane holds at once
constexpr int SR_MAXL = 8;                    // layers per launch
constexpr int SR_MAX_SPLITS = 64;             // attention key splits per kv head
constexpr int SR_MAXCH = 48;                  // residual columns owned by one workgroup
constexpr int SR_MAXG = 8;                    // q heads per kv head
constexpr int SR_MAX_D2 = 64;                 // DFlash2 conv groups
constexpr int SR_TRACE = 4096;                // phase time stamps
// counter words: SR_NCTR phase counters 32 words (128 bytes) apart, workgroup w
// signalling counter w % SR_NCTR, then the epoch and the error word.  Few
// workgroups per counter keep the same-line atomics of a phase end short.
constexpr int SR_NCTR = 64;
constexpr int SR_CTR_EPOCH = SR_NCTR * 32, SR_CTR_ERR = SR_CTR_EPOCH + 32, SR_CTR_WORDS = SR_CTR_ERR + 32;

struct SrMat {
    const void *w;    // [n][K], torch Linear layout, in the weight dtype
    const float *s;   // fp8: per-row f32 scales [n]; otherwise nullptr
};

struct SrLayer {
    SrMat q, k, v, o, g, u, d;
    SrMat aw, mw;                          // DFlash2 dynamic-coefficient projections [4G][H]
    const float *g_in, *g_post, *g_q, *g_k;
    const float *abase, *mbase;            // DFlash2 static taps [2][H][2] (attention, MLP)
    char *pk;                              // the layer's packed GEMM weight stream (sround_pack_layer_bytes)
};

struct SrScalars {
    int H, I, nq, nkv, d, qd, kvd, G;
    int b, len, cap, nl, first, last, d2;
    int nwg, cq, ch, ci;                   // columns per workgroup: q|k|v, hidden, intermediate
    int nsplit, nkb;                       // attention: key splits per kv head, 32-key blocks of the cache
    float eps, mscale, qscale;             // qscale = log2(e) / sqrt(head_dim)
    const float *noise;                    // [b][H]
    const int32_t *pos;                    // [b]
    float *out;                            // [b][H]
    const float *g_norm;
    char *kc, *vc;                         // cache bases of this launch's first layer
    long long kv_lstride;                  // bytes per layer (K and V alike)
    unsigned *ctr;                         // SR_CTR_WORDS counter words
    float *cs;                             // cos / sin of the block positions [16][d/2][2]
    float *xsave;                          // residual [16][H] f32 carried between launches
    char *lay;                             // per-layer buffers, lay_stride bytes apart
    long long lay_stride;
    long long o_xa, o_ssa, o_qkv, o_po, o_pml, o_of, o_xm, o_ssm, o_zf, o_da, o_dm;
    unsigned long long *trace;             // phase stamps of workgroup 0, or nullptr
};

// Kernel arguments; read in place from the kernel-argument segment.
struct SrArgs {
    SrScalars s;
    double inv_freq[64];
    SrLayer L[SR_MAXL];
};

// Bytes of one per-layer buffer block and the offsets inside it.
struct SrLayout {
    long long xa, ssa, qkv, po, pml, of, xm, ssm, zf, da, dm, stride;
};
SrLayout sround_layout(int H, int I, int qd, int kvd, int nkv, int G, int d, int wt, int nwg, int d2);

// Number of workgroups the streamed kernel uses for these dimensions on a
// device with `cus` compute units, or 0 if the shape is not supported.
int sround_nwg(int H, int I, int qd, int kvd, int wt, int d2, int cus);

hipError_t sround_launch(const SrArgs &a, int wt, int nwg, hipStream_t s);

// Packed weight stream: bytes per layer for a launch of nwg workgroups, and
// the kernel that writes the stream of every layer of `a` (L[i].pk).
long long sround_pack_layer_bytes(int H, int I, int qd, int kvd, int wt, int d2, int nwg);
hipError_t sround_pack_launch(const SrArgs &a, int wt, int nwg, hipStream_t s);

}  // namespace dfl
