// Skinny GEMM for the drafter's projections:  Y[M, N] (epi)= A[M, K] . W[N, K]^T
//
// A: f32 activations (M = 16 block rows on the round path; ctx rows on the
//    ingest / first-light path).
// W: f32, bf16 or fp8 e4m3fn weights in torch Linear layout [N, K], streamed
//    from HBM once per call.  This stream is the dominant cost of a round.
//
// Work item = (group of MT 16-row tiles, one 16-column tile, one K split).
// A workgroup of 4 waves takes one item.  The waves interleave over K chunks,
// so at any moment the workgroup reads 16 weight rows x 4 adjacent chunks.
// Each lane issues one 16-byte load per chunk and weight row:
//   bf16: 8 values (K chunk 32), one MFMA 16x16x32 each on the hi and lo
//         bf16 halves of the activations;
//   fp8 : 16 codes (K chunk 64), decoded exactly to bf16, 4 MFMAs;
//   f32 : 4 values (K chunk 16), 4 MFMAs 16x16x4 f32.
// The 4 wave accumulators are summed in LDS in a fixed order.  With a K
// split, each workgroup writes its partial tile.  The last workgroup of a
// tile to finish (an atomic counter) sums the partials in split order and
// applies the epilogue, so results do not depend on scheduling.
#include "common.h"
#include "kernels.h"

namespace dfl {

template <int WT> struct WCfg;
template <> struct WCfg<WT_BF16> { static constexpr int KC = 32, E = 8,  ES = 2; };
template <> struct WCfg<WT_FP8>  { static constexpr int KC = 64, E = 16, ES = 1; };
template <> struct WCfg<WT_F32>  { static constexpr int KC = 16, E = 4,  ES = 4; };

// One K chunk of one 16x16 tile: acc += A_frag . W_frag.
template <int WT>
__device__ __forceinline__ void mac_chunk(f32x4 &acc, const u32x4 &wv, const float *a, bool valid) {
    if constexpr (WT == WT_BF16) {
        float x[8];
        if (valid) {
            float4 p = ld_f4(a), q = ld_f4(a + 4);
            x[0] = p.x; x[1] = p.y; x[2] = p.z; x[3] = p.w; x[4] = q.x; x[5] = q.y; x[6] = q.z; x[7] = q.w;
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) x[i] = 0.f;
        }
        bf16x8 hi, lo;
        split_bf16x8(x, hi, lo);
        bf16x8 b = __builtin_bit_cast(bf16x8, wv);
        acc = mfma_bf16(hi, b, acc);
        acc = mfma_bf16(lo, b, acc);
    } else if constexpr (WT == WT_FP8) {
        bf16x8 b0 = fp8x8_to_bf16x8(wv.x, wv.y);
        bf16x8 b1 = fp8x8_to_bf16x8(wv.z, wv.w);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            float x[8];
            if (valid) {
                float4 p = ld_f4(a + 8 * h), q = ld_f4(a + 8 * h + 4);
                x[0] = p.x; x[1] = p.y; x[2] = p.z; x[3] = p.w; x[4] = q.x; x[5] = q.y; x[6] = q.z; x[7] = q.w;
            } else {
#pragma unroll
                for (int i = 0; i < 8; ++i) x[i] = 0.f;
            }
            bf16x8 hi, lo;
            split_bf16x8(x, hi, lo);
            acc = mfma_bf16(hi, h ? b1 : b0, acc);
            acc = mfma_bf16(lo, h ? b1 : b0, acc);
        }
    } else {
        float4 p = valid ? ld_f4(a) : make_float4(0.f, 0.f, 0.f, 0.f);
        float4 w = __builtin_bit_cast(float4, wv);
        acc = mfma_f32(p.x, w.x, acc);
        acc = mfma_f32(p.y, w.y, acc);
        acc = mfma_f32(p.z, w.z, acc);
        acc = mfma_f32(p.w, w.w, acc);
    }
}

__device__ __forceinline__ float silu(float x) { return x / (1.f + __expf(-x)); }

template <int WT, int MT, int EPI, int U>
__global__ __launch_bounds__(256) void gemm_kernel(GemmArgs p) {
    constexpr int KC = WCfg<WT>::KC, E = WCfg<WT>::E, ES = WCfg<WT>::ES;
    constexpr int NACC = (EPI == EPI_SWIGLU) ? 2 : 1;
    constexpr int NT = MT * NACC;  // 16x16 tiles per workgroup

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 4, r16 = lane & 15;
    const int ntile = blockIdx.x / p.ksplit, split = blockIdx.x - ntile * p.ksplit;
    const int mgroup = blockIdx.y;
    const int n0 = ntile * 16;
    const int m0 = mgroup * MT * 16;

    // weight segment(s) of this column tile
    const char *wbase[NACC];
    const float *wscale[NACC];
    int ncol0 = n0;  // column within the segment
    if constexpr (EPI == EPI_SWIGLU) {
        wbase[0] = (const char *)p.seg[0].w; wscale[0] = p.seg[0].scale;
        wbase[1] = (const char *)p.seg[1].w; wscale[1] = p.seg[1].scale;
    } else {
        int s = 0;
        while (s + 1 < p.nseg && ncol0 >= p.seg[s].n) { ncol0 -= p.seg[s].n; ++s; }
        wbase[0] = (const char *)p.seg[s].w; wscale[0] = p.seg[s].scale;
    }

    const int K = p.K;
    const int kbeg = split * p.kchunk;
    const int klen = min(p.kchunk, K - kbeg);
    const int nch = klen / KC;

    const char *wrow[NACC];
#pragma unroll
    for (int a = 0; a < NACC; ++a)
        wrow[a] = wbase[a] + ((size_t)(ncol0 + r16) * K + kbeg + g * E) * ES;
    const float *arow[MT];
    bool avalid[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        int row = m0 + mt * 16 + r16;
        avalid[mt] = row < p.M;
        arow[mt] = p.A + (size_t)(avalid[mt] ? row : 0) * p.lda + kbeg + g * E;
    }

    f32x4 acc[MT][NACC];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int a = 0; a < NACC; ++a) acc[mt][a] = f32x4{0.f, 0.f, 0.f, 0.f};

    for (int c0 = wave; c0 < nch; c0 += 4 * U) {
        u32x4 wv[U][NACC];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int c = c0 + 4 * u;
            if (c < nch) {
#pragma unroll
                for (int a = 0; a < NACC; ++a) wv[u][a] = ld_stream16(wrow[a] + (size_t)c * KC * ES);
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int c = c0 + 4 * u;
            if (c < nch) {
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                    for (int a = 0; a < NACC; ++a)
                        mac_chunk<WT>(acc[mt][a], wv[u][a], arow[mt] + (size_t)c * KC, avalid[mt]);
            }
        }
    }

    // ---- sum the 4 waves' tiles in LDS (fixed order) ----
    __shared__ float red[4][NT][256];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int a = 0; a < NACC; ++a)
            *reinterpret_cast<f32x4 *>(&red[wave][mt * NACC + a][lane * 4]) = acc[mt][a];
    __syncthreads();
    float v[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) v[t] = ((red[0][t][tid] + red[1][t][tid]) + red[2][t][tid]) + red[3][t][tid];

    // ---- split-K: the last workgroup of the tile reduces in split order ----
    if (p.ksplit > 1) {
        const int tile_id = mgroup * p.ntiles + ntile;
        float *part = p.part + (size_t)tile_id * p.ksplit * (NT * 256);
#pragma unroll
        for (int t = 0; t < NT; ++t)
            __hip_atomic_store(part + (size_t)split * (NT * 256) + t * 256 + tid, v[t], __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
        __threadfence();
        __syncthreads();
        __shared__ int is_last;
        if (tid == 0) {
            unsigned prev = __hip_atomic_fetch_add(p.cnt + tile_id, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
            is_last = (prev == (unsigned)(p.ksplit - 1));
        }
        __syncthreads();
        if (!is_last) return;
        __threadfence();
#pragma unroll
        for (int t = 0; t < NT; ++t) v[t] = 0.f;
        for (int s = 0; s < p.ksplit; ++s)
#pragma unroll
            for (int t = 0; t < NT; ++t)
                v[t] += __hip_atomic_load(part + (size_t)s * (NT * 256) + t * 256 + tid, __ATOMIC_RELAXED,
                                          __HIP_MEMORY_SCOPE_AGENT);
        if (tid == 0) __hip_atomic_store(p.cnt + tile_id, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }

    // ---- epilogue: element tid of each 16x16 tile ----
    const int el = tid >> 2, j = tid & 3;
    const int row_in = 4 * (el >> 4) + j, col = el & 15;
    const int ccol = ncol0 + col;  // column inside the segment (for scales)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        const int row = m0 + mt * 16 + row_in;
        if (row >= p.M) continue;
        float *y = p.Y + (size_t)row * p.ldy + n0 + col;
        if constexpr (EPI == EPI_SWIGLU) {
            float gv = v[mt * 2 + 0], uv = v[mt * 2 + 1];
            if constexpr (WT == WT_FP8) { gv *= wscale[0][ccol]; uv *= wscale[1][ccol]; }
            *y = silu(gv) * uv;
        } else {
            float r = v[mt];
            if constexpr (WT == WT_FP8) r *= wscale[0][ccol];
            if constexpr (EPI == EPI_ADD) *y += r;
            else *y = r;
        }
    }
}

// ---------------------------------------------------------------------------
// host side: plan the split and launch
// ---------------------------------------------------------------------------
static int kc_of(int wt) { return wt == WT_BF16 ? 32 : wt == WT_FP8 ? 64 : 16; }

int gemm_plan(GemmArgs &a) {
    const int nacc = a.epi == EPI_SWIGLU ? 2 : 1;
    int ncols = 0;
    if (a.epi == EPI_SWIGLU) ncols = a.seg[0].n;
    else for (int s = 0; s < a.nseg; ++s) ncols += a.seg[s].n;
    a.ntiles = ncols / 16;
    a.mt = a.M <= 16 ? 1 : a.M <= 32 ? 2 : 4;
    a.mgroups = (a.M + 16 * a.mt - 1) / (16 * a.mt);
    const int kstep = 4 * kc_of(a.wtype);        // 4 waves x one chunk
    const int base = a.ntiles * a.mgroups;
    int ksplit = 1;
    const int target = 1024;                     // ~4 workgroups per CU
    if (base < target) ksplit = (target + base - 1) / base;
    int maxsplit = a.K / kstep;
    if (ksplit > maxsplit) ksplit = maxsplit;
    if (ksplit < 1) ksplit = 1;
    // partial storage bound
    const size_t per = (size_t)a.mt * nacc * 256;
    while (ksplit > 1 && (size_t)base * ksplit * per > GEMM_PART_FLOATS) --ksplit;
    if (ksplit > 1 && base > GEMM_MAX_COUNTERS) ksplit = 1;
    int kchunk = (a.K + ksplit - 1) / ksplit;
    kchunk = (kchunk + kstep - 1) / kstep * kstep;
    ksplit = (a.K + kchunk - 1) / kchunk;
    a.ksplit = ksplit;
    a.kchunk = kchunk;
    return base * ksplit;
}

template <int WT, int EPI>
static hipError_t launch_wt_epi(GemmArgs &a, hipStream_t s) {
    dim3 grid(a.ntiles * a.ksplit, a.mgroups), block(256);
    constexpr int U = WT == WT_F32 ? 4 : 8;
    switch (a.mt) {
        case 1: hipLaunchKernelGGL((gemm_kernel<WT, 1, EPI, U>), grid, block, 0, s, a); break;
        case 2: hipLaunchKernelGGL((gemm_kernel<WT, 2, EPI, U>), grid, block, 0, s, a); break;
        default: hipLaunchKernelGGL((gemm_kernel<WT, 4, EPI, (U > 4 ? 4 : U)>), grid, block, 0, s, a); break;
    }
    return hipGetLastError();
}

template <int WT>
static hipError_t launch_wt(GemmArgs &a, hipStream_t s) {
    switch (a.epi) {
        case EPI_STORE: return launch_wt_epi<WT, EPI_STORE>(a, s);
        case EPI_ADD: return launch_wt_epi<WT, EPI_ADD>(a, s);
        default: return launch_wt_epi<WT, EPI_SWIGLU>(a, s);
    }
}

hipError_t gemm(GemmArgs a, float *part, unsigned *cnt, hipStream_t s) {
    if (a.M <= 0) return hipSuccess;
    gemm_plan(a);
    a.part = part;
    a.cnt = cnt;
    switch (a.wtype) {
        case WT_BF16: return launch_wt<WT_BF16>(a, s);
        case WT_FP8: return launch_wt<WT_FP8>(a, s);
        default: return launch_wt<WT_F32>(a, s);
    }
}

}  // namespace dfl
