// Device step of the DFlash2 proposal ([DflashDraft] "dflash2_propose_greedy"):
// top-k over each draft row's logits and the rank-r projection of the draft
// rows' hidden states, packed for one small device-to-host copy.
//
// Top-k runs in two stages of the same kernel.  One wave takes a chunk of
// one row, keeps up to VPL values per lane in registers and extracts the
// chunk's k best by k rounds of a wave-wide argmax (order: larger value
// first, then lower index), marking each winner as taken.  Stage 1 runs one
// wave per (row, 2048-value chunk); stage 2 one wave per row over the
// stage-1 candidates.  Every load is in bounds (lanes past the chunk hold
// "taken" entries), and every wave runs exactly k rounds.
#include <climits>

#include "common.h"
#include "kernels.h"

namespace dfl {
namespace {

// (value, index) ordering of the selection: true if a ranks before b
__device__ __forceinline__ bool before(float va, int ia, float vb, int ib) {
    return va > vb || (va == vb && ia < ib);
}

template <int VPL>
__global__ __launch_bounds__(64) void topk_wave(const float *in, const int32_t *in_idx, int n, long long ld, int chunk,
                                                int k, float *out_v, int32_t *out_i, int out_ld) {
    const int lane = threadIdx.x, row = blockIdx.y, c = blockIdx.x;
    const int lo = c * chunk, hi = min(n, lo + chunk);
    const float *src = in + (size_t)row * ld;
    const int32_t *isrc = in_idx ? in_idx + (size_t)row * ld : nullptr;
    float v[VPL];
    int id[VPL];
#pragma unroll
    for (int j = 0; j < VPL; ++j) {
        const int e = lo + j * 64 + lane;
        const bool ok = e < hi;
        const int es = ok ? e : lo;                         // in-bounds address for every lane
        const float x = src[es];
        const int xi = isrc ? isrc[es] : es;
        v[j] = ok ? x : -INFINITY;
        id[j] = ok ? xi : INT_MAX;                          // never ranks before a real entry
    }
    float *ov = out_v + (size_t)row * out_ld + (size_t)c * k;
    int32_t *oi = out_i + (size_t)row * out_ld + (size_t)c * k;
    for (int r = 0; r < k; ++r) {
        // this lane's best remaining entry
        float bv = v[0];
        int bi = id[0], bj = 0;
#pragma unroll
        for (int j = 1; j < VPL; ++j)
            if (before(v[j], id[j], bv, bi)) { bv = v[j]; bi = id[j]; bj = j; }
        // wave-wide best (value, index)
        float wv = bv;
        int wi = bi;
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) {
            const float ov2 = __shfl_xor(wv, o, 64);
            const int oi2 = __shfl_xor(wi, o, 64);
            if (before(ov2, oi2, wv, wi)) { wv = ov2; wi = oi2; }
        }
        if (lane == 0) { ov[r] = wv; oi[r] = wi; }
        // the owner marks it taken (indices are unique within a row)
        if (bi == wi && bv == wv) {
#pragma unroll
            for (int j = 0; j < VPL; ++j)
                if (j == bj) { v[j] = -INFINITY; id[j] = INT_MAX; }
        }
    }
}

// hproj[r][j] = sum_c hidden[r][c] * W[j][c]: one wave per output, f32 accumulation
__global__ __launch_bounds__(256) void hidden_proj(const float *hidden, int H, const uint16_t *w, int rank, int rows,
                                                   float *out) {
    const int wave = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
    if (wave >= rows * rank) return;
    const int r = wave / rank, j = wave - r * rank;
    const float *x = hidden + (size_t)r * H;
    const uint16_t *wr = w + (size_t)j * H;
    float s = 0.f;
    for (int c = lane; c < H; c += 64) s += x[c] * bf16_bits_to_f32(wr[c]);
    s = wave_sum(s);
    if (lane == 0) out[(size_t)r * rank + j] = s;
}

}  // namespace

int topk_chunks(int vocab) { return (vocab + TOPK_CHUNK - 1) / TOPK_CHUNK; }

hipError_t topk_rows(const float *logits, long long ld, int rows, int vocab, int k, float *part_v, int32_t *part_i,
                     float *vals, int32_t *idx, hipStream_t s) {
    const int nc = topk_chunks(vocab);
    hipLaunchKernelGGL(topk_wave<TOPK_CHUNK / 64>, dim3(nc, rows), dim3(64), 0, s, logits, (const int32_t *)nullptr,
                       vocab, ld, TOPK_CHUNK, k, part_v, part_i, nc * k);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int n2 = nc * k;                               // <= TOPK_STAGE2 (checked by the caller)
    hipLaunchKernelGGL(topk_wave<TOPK_STAGE2 / 64>, dim3(1, rows), dim3(64), 0, s, (const float *)part_v,
                       (const int32_t *)part_i, n2, (long long)n2, TOPK_STAGE2, k, vals, idx, k);
    return hipGetLastError();
}

hipError_t hidden_projection(const float *hidden, int H, const void *w, int rank, int rows, float *out, hipStream_t s) {
    const int waves = rows * rank;
    hipLaunchKernelGGL(hidden_proj, dim3((waves + 3) / 4), dim3(256), 0, s, hidden, H, (const uint16_t *)w, rank, rows,
                       out);
    return hipGetLastError();
}

}  // namespace dfl
