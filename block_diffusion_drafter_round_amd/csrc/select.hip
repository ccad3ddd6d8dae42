// Device step of the DFlash2 proposal ([DflashDraft] "dflash2_propose_greedy"):
// top-k over each draft row's logits and the rank-r projection of the draft
// rows' hidden states, packed for one small device-to-host copy.
//
// Top-k runs in stages of one kernel.  One wave takes a chunk of 1024
// candidates of one row, 16 per lane in registers, sorts each lane's 16
// once (Batcher's odd-even merge network), and extracts the chunk's k best
// by k rounds of a wave-wide argmax over the lanes' heads (order: larger
// value first, then lower index); the winner's lane shifts its list up.  Each stage keeps k of every
// 1024 candidates, until a single chunk holds them all.  Every load is in
// bounds (lanes past the chunk hold "taken" entries), and every wave runs
// exactly k rounds.
//
// A chunk's k best come out in selection order, so after the first stage a
// row holds one sorted list per chunk.  When those lists fit in LDS (149
// lists of 32 for a 151,936-token vocabulary), one wave per row merges them
// instead of the further stages: lane j owns lists j, j + 64, ..., each
// round picks the best list head across the wave, and the owner advances
// that list.  The merge of sorted lists yields the row's k best in the same
// total order, so both routes give the same result.
#include <climits>

#include "common.h"
#include "kernels.h"

namespace dfl {
namespace {

// (value, index) ordering of the selection: true if a ranks before b
__device__ __forceinline__ bool before(float va, int ia, float vb, int ib) {
    return va > vb || (va == vb && ia < ib);
}
__device__ __forceinline__ void keep_best(float &wv, int &wi, float ov, int oi) {
    if (before(ov, oi, wv, wi)) { wv = ov; wi = oi; }
}
// The wave's best (value, index): the selection order is total, so any
// reduction tree picks the same entry.  Within 16-lane rows by DPP row
// rotations, across rows by the lane swaps (a register swapped with itself
// leaves a lane its own entry in one result and its partner's in the
// other; values and indices move alike).  No LDS round trip.
template <int N>
__device__ __forceinline__ int ror_i(int x) { return __builtin_amdgcn_update_dpp(0, x, 0x120 + N, 0xF, 0xF, false); }
__device__ __forceinline__ void wave_best(float &wv, int &wi) {
    keep_best(wv, wi, __int_as_float(ror_i<1>(__float_as_int(wv))), ror_i<1>(wi));
    keep_best(wv, wi, __int_as_float(ror_i<2>(__float_as_int(wv))), ror_i<2>(wi));
    keep_best(wv, wi, __int_as_float(ror_i<4>(__float_as_int(wv))), ror_i<4>(wi));
    keep_best(wv, wi, __int_as_float(ror_i<8>(__float_as_int(wv))), ror_i<8>(wi));
    {
        const auto pv = __builtin_amdgcn_permlane16_swap(__float_as_uint(wv), __float_as_uint(wv), false, false);
        const auto pi = __builtin_amdgcn_permlane16_swap((unsigned)wi, (unsigned)wi, false, false);
        wv = __uint_as_float(pv[0]); wi = (int)pi[0];
        keep_best(wv, wi, __uint_as_float(pv[1]), (int)pi[1]);
    }
    {
        const auto pv = __builtin_amdgcn_permlane32_swap(__float_as_uint(wv), __float_as_uint(wv), false, false);
        const auto pi = __builtin_amdgcn_permlane32_swap((unsigned)wi, (unsigned)wi, false, false);
        wv = __uint_as_float(pv[0]); wi = (int)pi[0];
        keep_best(wv, wi, __uint_as_float(pv[1]), (int)pi[1]);
    }
}

// Batcher's odd-even merge sort network on N (a power of two) entries: the
// comparator list, built at compile time, so that every register index in
// the sort is a constant.
struct Cmp {
    int a, b;
};
template <int N>
struct OemNet {
    Cmp c[8 * N];
    int n;
    constexpr OemNet() : c{}, n(0) {
        for (int p = 1; p < N; p <<= 1)
            for (int k = p; k >= 1; k >>= 1)
                for (int j = k % p; j + k < N; j += 2 * k)
                    for (int i = 0; i < (k < N - j - k ? k : N - j - k); ++i)
                        if ((i + j) / (2 * p) == (i + j + k) / (2 * p)) c[n++] = Cmp{i + j, i + j + k};
    }
};
static_assert(OemNet<16>{}.n == 63, "odd-even merge sort of 16 takes 63 comparators");
// comparators I.. of the network: entry a ends up ranking before entry b
template <int I, int N>
__device__ __forceinline__ void oem_sort(float (&v)[N], int (&id)[N]) {
    if constexpr (I < OemNet<N>{}.n) {
        constexpr Cmp c = OemNet<N>{}.c[I];
        const bool sw = before(v[c.b], id[c.b], v[c.a], id[c.a]);
        const float va = v[c.a], vb = v[c.b];
        const int ia = id[c.a], ib = id[c.b];
        v[c.a] = sw ? vb : va;
        id[c.a] = sw ? ib : ia;
        v[c.b] = sw ? va : vb;
        id[c.b] = sw ? ia : ib;
        oem_sort<I + 1, N>(v, id);
    }
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
    static_assert((VPL & (VPL - 1)) == 0, "the sort network takes a power of two");
    oem_sort<0, VPL>(v, id);                                // v[0] is this lane's best
    for (int r = 0; r < k; ++r) {
        // wave-wide best (value, index) of the lanes' heads
        float wv = v[0];
        int wi = id[0];
        wave_best(wv, wi);
        if (lane == 0) { ov[r] = wv; oi[r] = wi; }
        // the owner's list moves up (indices are unique within a row; several
        // lanes match only when the winner is a "taken" entry, and then all
        // their entries are)
        if (v[0] == wv && id[0] == wi) {
#pragma unroll
            for (int j = 0; j + 1 < VPL; ++j) { v[j] = v[j + 1]; id[j] = id[j + 1]; }
            v[VPL - 1] = -INFINITY;
            id[VPL - 1] = INT_MAX;
        }
    }
}

// Merge of a row's nl sorted lists of k (value, index) entries (one per
// first-stage chunk, row stride ld) into the row's k best, in order.  The
// four waves copy the lists to LDS (several loads in flight per lane), then
// wave 0 merges them: lane j holds the heads of lists j + 64 u.
constexpr int MERGE_THREADS = 256;
template <int LMAX>
__global__ __launch_bounds__(MERGE_THREADS) void topk_merge(const float *in_v, const int32_t *in_i, int nl, int k,
                                                            long long ld, float *out_v, int32_t *out_i) {
    extern __shared__ float2 lst[];                          // [nl][k]: (value, index bits)
    const int lane = threadIdx.x, row = blockIdx.x;
    const float *sv = in_v + (size_t)row * ld;
    const int32_t *si = in_i + (size_t)row * ld;
    const int ne = nl * k;
#pragma unroll 4
    for (int e = threadIdx.x; e < ne; e += MERGE_THREADS) lst[e] = make_float2(sv[e], __int_as_float(si[e]));
    __syncthreads();
    if (threadIdx.x >= 64) return;
    float hv[LMAX];
    int hi[LMAX], pos[LMAX];
#pragma unroll
    for (int u = 0; u < LMAX; ++u) {
        const int li = lane + 64 * u;
        const bool ok = li < nl;
        const float2 h = lst[ok ? li * k : 0];
        hv[u] = ok ? h.x : -INFINITY;
        hi[u] = ok ? __float_as_int(h.y) : INT_MAX;
        pos[u] = ok ? 0 : k;
    }
    float *ov = out_v + (size_t)row * k;
    int32_t *oi = out_i + (size_t)row * k;
    for (int r = 0; r < k; ++r) {
        float bv = hv[0];
        int bi = hi[0], bu = 0;
#pragma unroll
        for (int u = 1; u < LMAX; ++u)
            if (before(hv[u], hi[u], bv, bi)) { bv = hv[u]; bi = hi[u]; bu = u; }
        float wv = bv;
        int wi = bi;
        wave_best(wv, wi);
        if (lane == 0) { ov[r] = wv; oi[r] = wi; }
        // the owner of the winning head moves to that list's next entry (a
        // "taken" entry past the list's end).  Several lanes match only when
        // the winner is such an entry, and then every head left is one too.
        if (bi == wi && bv == wv) {
#pragma unroll
            for (int u = 0; u < LMAX; ++u)
                if (u == bu) {
                    const int nx = ++pos[u];
                    const float2 h = lst[nx < k ? (lane + 64 * u) * k + nx : 0];
                    hv[u] = nx < k ? h.x : -INFINITY;
                    hi[u] = nx < k ? __float_as_int(h.y) : INT_MAX;
                }
        }
    }
}

// hproj[r][j] = sum_c hidden[r][c] * W[j][c]: one wave per output, f32
// accumulation; lane l takes 8 consecutive columns per 512, with the loads
// of up to four such groups in flight at once (H is a multiple of 256)
__global__ __launch_bounds__(256) void hidden_proj(const float *hidden, int H, const uint16_t *w, int rank, int rows,
                                                   float *out) {
    const int wave = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
    if (wave >= rows * rank) return;
    const int r = wave / rank, j = wave - r * rank;
    const float *x = hidden + (size_t)r * H;
    const uint16_t *wr = w + (size_t)j * H;
    float s = 0.f;
    for (int c0 = 0; c0 < H; c0 += 4 * 512) {
        u32x4 wv[4];
        float4 xa[4], xb[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int c = min(c0 + u * 512 + 8 * lane, H - 8);
            wv[u] = *reinterpret_cast<const u32x4 *>(wr + c);
            xa[u] = *reinterpret_cast<const float4 *>(x + c);
            xb[u] = *reinterpret_cast<const float4 *>(x + c + 4);
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            if (c0 + u * 512 + 8 * lane >= H) continue;
            const float xs[8] = {xa[u].x, xa[u].y, xa[u].z, xa[u].w, xb[u].x, xb[u].y, xb[u].z, xb[u].w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                s += xs[2 * i] * bf16_bits_to_f32(wv[u][i] & 0xFFFFu);
                s += xs[2 * i + 1] * __uint_as_float(wv[u][i] & 0xFFFF0000u);
            }
        }
    }
    s = wave_sum(s);
    if (lane == 0) out[(size_t)r * rank + j] = s;
}

}  // namespace

int topk_chunks(int vocab) { return (vocab + TOPK_CHUNK - 1) / TOPK_CHUNK; }

size_t topk_scratch_entries(int rows, int vocab, int k) {
    // the first stage's candidates, then the second stage's, side by side
    const size_t n1 = (size_t)topk_chunks(vocab) * k;
    return (size_t)rows * (n1 + (size_t)topk_chunks((int)n1) * k);
}

hipError_t topk_rows(const float *logits, long long ld, int rows, int vocab, int k, float *part_v, int32_t *part_i,
                     float *vals, int32_t *idx, hipStream_t s) {
    // each stage keeps the k best of every TOPK_CHUNK candidates, until one
    // chunk holds them all; stages alternate between two candidate regions
    const float *in = logits;
    const int32_t *in_i = nullptr;
    long long in_ld = ld;
    int n = vocab;
    // region A holds the first stage's output, region B (right after it) the
    // second's; every later stage is smaller than both
    const size_t region_b = (size_t)rows * topk_chunks(vocab) * k;
    size_t off = 0;
    const int nc1 = topk_chunks(vocab);
    if (nc1 > 1 && nc1 <= TOPK_MERGE_LISTS && (size_t)nc1 * k * sizeof(float2) <= TOPK_MERGE_LDS) {
        // first stage, then the merge of its sorted per-chunk lists
        hipLaunchKernelGGL(topk_wave<TOPK_CHUNK / 64>, dim3(nc1, rows), dim3(64), 0, s, logits, (const int32_t *)nullptr,
                           vocab, ld, TOPK_CHUNK, k, part_v, part_i, nc1 * k);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(topk_merge<TOPK_MERGE_LISTS / 64>, dim3(rows), dim3(MERGE_THREADS), (size_t)nc1 * k * sizeof(float2), s,
                           part_v, part_i, nc1, k, (long long)nc1 * k, vals, idx);
        return hipGetLastError();
    }
    while (true) {
        const int nc = topk_chunks(n);
        const bool last = nc == 1;
        float *ov = last ? vals : part_v + off;
        int32_t *oi = last ? idx : part_i + off;
        const int out_ld = nc * k;
        hipLaunchKernelGGL(topk_wave<TOPK_CHUNK / 64>, dim3(nc, rows), dim3(64), 0, s, in, in_i, n, in_ld, TOPK_CHUNK,
                           k, ov, oi, out_ld);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess || last) return e;
        in = ov;
        in_i = oi;
        in_ld = out_ld;
        n = out_ld;
        off = off == 0 ? region_b : 0;                  // the next stage writes the other region
    }
}

hipError_t hidden_projection(const float *hidden, int H, const void *w, int rank, int rows, float *out, hipStream_t s) {
    const int waves = rows * rank;
    hipLaunchKernelGGL(hidden_proj, dim3((waves + 3) / 4), dim3(256), 0, s, hidden, H, (const uint16_t *)w, rank, rows,
                       out);
    return hipGetLastError();
}

}  // namespace dfl
