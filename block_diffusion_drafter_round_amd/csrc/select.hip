// Device step of the DFlash2 proposal ([DflashDraft] "dflash2_propose_greedy"):
// top-k over each draft row's logits and the rank-r projection of the draft
// rows' hidden states, packed for one small device-to-host copy.
//
// Top-k runs in stages of one kernel.  One wave takes a chunk of 1024
// candidates of one row, 16 per lane in registers, sorts each lane's 16
// once (Batcher's odd-even merge network), and extracts the chunk's k best
// by k rounds of a wave-wide argmax over the lanes' heads (order: larger
// value first, then lower index; a -0 logit is reported as +0); the
// winner's lane shifts its list up.  Each stage keeps k of every 1024
// candidates, until a single chunk holds them all.  Every load is in bounds
// (lanes past the chunk hold "taken" entries), and every wave runs exactly
// k rounds.
//
// A chunk's best come out in selection order, so after the first stage a
// row holds one sorted list per chunk.  When k-entry lists fit in LDS (149
// lists of 32 for a 151,936-token vocabulary), the first stage keeps only
// each chunk's TOPK_QUOTA best and one wave per row merges the lists instead
// of the further stages: lane j owns lists j, j + 64, ..., each round picks
// the best list head across the wave, and the owner advances that list; a
// list that runs out before the row's k are found is refilled with its
// chunk's k best.  The merge of sorted lists yields the row's k best in the
// same total order, so both routes give the same result.  Most rows skip
// the k rounds: the merge ranks the few candidates that can reach the k
// best among themselves instead (see topk_merge).
#include <algorithm>
#include <climits>
#include <cstdint>

#include "common.h"
#include "kernels.h"

namespace dfl {
namespace {

// The selection order (larger value first, then lower index) as the
// unsigned order of one 64-bit key: the high word is the value's bits made
// monotonic (positive values with the sign bit set, negative ones
// complemented; -0 is taken as +0, which compares equal to it), the low word
// the complemented index.  Every comparison below is one 64-bit compare.
// "Taken" entries are the key of (-inf, INT_MAX), below every real entry.
typedef unsigned long long Key;
__device__ __forceinline__ Key sel_key(float v, int i) {
    unsigned u = __float_as_uint(v == 0.f ? 0.f : v);
    u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
    return ((Key)u << 32) | (unsigned)~i;
}
__device__ __forceinline__ float key_value(Key k) {
    const unsigned u = (unsigned)(k >> 32);
    return __uint_as_float((u & 0x80000000u) ? (u & 0x7fffffffu) : ~u);
}
__device__ __forceinline__ int key_index(Key k) { return (int)~(unsigned)k; }
__device__ __forceinline__ Key taken_key() { return sel_key(-INFINITY, INT_MAX); }

// The wave's best key: the order is total, so any reduction tree picks the
// same entry.  Within 16-lane rows by DPP row rotations, across rows by the
// lane swaps (a register swapped with itself leaves a lane its own word in
// one result and its partner's in the other).  No LDS round trip.
template <int N>
__device__ __forceinline__ unsigned ror_u(unsigned x) { return __builtin_amdgcn_update_dpp(0u, x, 0x120 + N, 0xF, 0xF, false); }
template <int N>
__device__ __forceinline__ Key ror_key(Key k) {
    return ((Key)ror_u<N>((unsigned)(k >> 32)) << 32) | ror_u<N>((unsigned)k);
}
__device__ __forceinline__ Key wave_best(Key k) {
    Key o = ror_key<1>(k); k = o > k ? o : k;
    o = ror_key<2>(k); k = o > k ? o : k;
    o = ror_key<4>(k); k = o > k ? o : k;
    o = ror_key<8>(k); k = o > k ? o : k;
    {
        const auto h = __builtin_amdgcn_permlane16_swap((unsigned)(k >> 32), (unsigned)(k >> 32), false, false);
        const auto l = __builtin_amdgcn_permlane16_swap((unsigned)k, (unsigned)k, false, false);
        const Key a = ((Key)h[0] << 32) | l[0], c = ((Key)h[1] << 32) | l[1];
        k = a > c ? a : c;
    }
    {
        const auto h = __builtin_amdgcn_permlane32_swap((unsigned)(k >> 32), (unsigned)(k >> 32), false, false);
        const auto l = __builtin_amdgcn_permlane32_swap((unsigned)k, (unsigned)k, false, false);
        const Key a = ((Key)h[0] << 32) | l[0], c = ((Key)h[1] << 32) | l[1];
        k = a > c ? a : c;
    }
    return k;
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
__device__ __forceinline__ void oem_sort(Key (&x)[N]) {
    if constexpr (I < OemNet<N>{}.n) {
        constexpr Cmp c = OemNet<N>{}.c[I];
        const Key a = x[c.a], b = x[c.b];
        x[c.a] = a > b ? a : b;
        x[c.b] = a > b ? b : a;
        oem_sort<I + 1, N>(x);
    }
}

// Loads one chunk [lo, hi) of a row (16 candidates per lane; lanes past
// the chunk hold "taken" entries, every address in bounds) and sorts each
// lane's candidates, best first.  A whole chunk of 16-byte aligned logits
// is read as 16 contiguous candidates per lane in 16-byte loads; otherwise
// lane l takes candidates l, l + 64, ... (the choice is the same for the
// whole wave, so each candidate is read exactly once).
template <int VPL>
__device__ __forceinline__ void load_sorted(Key (&x)[VPL], const float *src, const int32_t *isrc, int lo, int hi) {
    const int lane = threadIdx.x & 63;
    const bool vec = !isrc && hi - lo == 64 * VPL && (reinterpret_cast<uintptr_t>(src + lo) & 15) == 0;
    if (vec) {
        static_assert(VPL % 4 == 0, "16-byte loads");
        const int e0 = lo + lane * VPL;
        float4 v[VPL / 4];
#pragma unroll
        for (int j = 0; j < VPL / 4; ++j) v[j] = *reinterpret_cast<const float4 *>(src + e0 + 4 * j);
#pragma unroll
        for (int j = 0; j < VPL / 4; ++j) {
            x[4 * j] = sel_key(v[j].x, e0 + 4 * j);
            x[4 * j + 1] = sel_key(v[j].y, e0 + 4 * j + 1);
            x[4 * j + 2] = sel_key(v[j].z, e0 + 4 * j + 2);
            x[4 * j + 3] = sel_key(v[j].w, e0 + 4 * j + 3);
        }
    } else {
#pragma unroll
        for (int j = 0; j < VPL; ++j) {
            const int e = lo + j * 64 + lane;
            const bool ok = e < hi;
            const int es = ok ? e : lo;
            const float v = src[es];
            const int vi = isrc ? isrc[es] : es;
            x[j] = ok ? sel_key(v, vi) : taken_key();
        }
    }
    static_assert((VPL & (VPL - 1)) == 0, "the sort network takes a power of two");
    oem_sort<0, VPL>(x);
}
// The best key left in the wave (of the lanes' heads); the owner's list
// moves up (keys are unique within a row except "taken" ones, and a lane
// whose head is taken holds only those).
template <int VPL>
__device__ __forceinline__ Key take_best(Key (&x)[VPL]) {
    const Key w = wave_best(x[0]);
    if (x[0] == w) {
#pragma unroll
        for (int j = 0; j + 1 < VPL; ++j) x[j] = x[j + 1];
        x[VPL - 1] = taken_key();
    }
    return w;
}

template <int VPL>
__global__ __launch_bounds__(64) void topk_wave(const float *in, const int32_t *in_idx, int n, long long ld, int chunk,
                                                int k, float *out_v, int32_t *out_i, int out_ld) {
    const int lane = threadIdx.x, row = blockIdx.y, c = blockIdx.x;
    const int lo = c * chunk, hi = min(n, lo + chunk);
    Key x[VPL];
    load_sorted(x, in + (size_t)row * ld, in_idx ? in_idx + (size_t)row * ld : nullptr, lo, hi);
    float *ov = out_v + (size_t)row * out_ld + (size_t)c * k;
    int32_t *oi = out_i + (size_t)row * out_ld + (size_t)c * k;
    for (int r = 0; r < k; ++r) {
        const Key w = take_best(x);
        if (lane == 0) { ov[r] = key_value(w); oi[r] = key_index(w); }
    }
}

// hproj[r][j] = sum_c hidden[r][c] * W[j][c]: one wave per output, f32
// accumulation; lane l takes 8 consecutive columns per 512, with the loads
// of up to four such groups in flight at once (H is a multiple of 256)
__device__ __forceinline__ void hproj_wave(const float *hidden, int H, const uint16_t *w, int rank, int rows, float *out,
                                           int wave) {
    const int lane = threadIdx.x & 63;
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
__global__ __launch_bounds__(256) void hidden_proj(const float *hidden, int H, const uint16_t *w, int rank, int rows,
                                                   float *out) {
    hproj_wave(hidden, H, w, rank, rows, out, blockIdx.x * 4 + (threadIdx.x >> 6));
}

// Merge of a row's nl sorted lists (one per first-stage chunk: that
// chunk's q best, row stride ld) into the row's k best, in order.  The four
// waves copy the lists to LDS as keys, list c at c * k, then wave 0 merges
// them: lane j holds the heads of lists j + 64 u.  A chunk may hold more
// than q of the row's k best: when a list of q runs out, the wave extracts
// that chunk's k best from the logits into the list's LDS row (its first q
// are the same entries), and the merge goes on.
constexpr int MERGE_THREADS = 256;
static_assert(MERGE_THREADS == 256, "projection blocks are four waves");
struct HProjArgs {
    const float *hidden;
    int H;
    const uint16_t *w;
    int rank, rows;
    float *out;
};
constexpr int MERGE_SMAX = 512;        // candidates the ranking route takes (more: the sequential merge)
template <int LMAX, int VPL>
__global__ __launch_bounds__(MERGE_THREADS) void topk_merge(const float *in_v, const int32_t *in_i, int nl, int q, int k,
                                                            long long ld, const float *logits, long long lld, int vocab,
                                                            float *out_v, int32_t *out_i, int rows, HProjArgs hp) {
    // blocks past the rows run the rank-r projection, four output waves each
    if ((int)blockIdx.x >= rows) {
        hproj_wave(hp.hidden, hp.H, hp.w, hp.rank, hp.rows, hp.out, ((int)blockIdx.x - rows) * 4 + (threadIdx.x >> 6));
        return;
    }
    extern __shared__ Key lst[];                             // [nl][k]
    __shared__ Key surv[MERGE_SMAX], thr;
    __shared__ int srank[MERGE_SMAX], ns, fb;
    __shared__ unsigned char slast[MERGE_SMAX];
    const int lane = threadIdx.x, row = blockIdx.x;
    const float *sv = in_v + (size_t)row * ld;
    const int32_t *si = in_i + (size_t)row * ld;
    float *ov = out_v + (size_t)row * k;
    int32_t *oi = out_i + (size_t)row * k;
    const int ne = nl * q;
    if (threadIdx.x == 0) { ns = 0; fb = 0; }
#pragma unroll 4
    for (int e = threadIdx.x; e < ne; e += MERGE_THREADS) {
        const int c = e / q;
        lst[c * k + (e - c * q)] = sel_key(sv[e], si[e]);
    }
    __syncthreads();
    if (nl >= k) {
        // Ranking route.  The k-th best list head L bounds the row's k-th
        // best from below (k real keys are >= L), so the k best are among
        // the candidates >= L: rank those among themselves by counting.  If
        // a list's last kept entry (position q - 1 < k - 1) ranks among the
        // k best, its chunk may hold more of them: the sequential merge
        // below, which refills such lists, decides the row instead.
        for (int t = threadIdx.x; t < nl; t += MERGE_THREADS) {
            const Key hk = lst[t * k];
            int rk = 0;
            for (int c = 0; c < nl; ++c) rk += lst[c * k] > hk ? 1 : 0;
            if (rk == k - 1) thr = hk;                      // heads are distinct real keys: exactly one
        }
        __syncthreads();
        const Key L = thr;
        for (int e = threadIdx.x; e < ne; e += MERGE_THREADS) {
            const int c = e / q, j = e - c * q;
            const Key x = lst[c * k + j];
            if (x >= L) {
                const int sl = atomicAdd(&ns, 1);
                if (sl < MERGE_SMAX) {
                    surv[sl] = x;
                    slast[sl] = j == q - 1 && q < k;
                }
            }
        }
        __syncthreads();
        const int S = ns;
        if (S <= MERGE_SMAX) {
            for (int t = threadIdx.x; t < S; t += MERGE_THREADS) {
                const Key x = surv[t];
                int rk = 0;
                for (int u = 0; u < S; ++u) rk += surv[u] > x ? 1 : 0;
                srank[t] = rk;
                if (rk < k && slast[t]) fb = 1;
            }
            __syncthreads();
            if (!fb) {
                for (int t = threadIdx.x; t < S; t += MERGE_THREADS)
                    if (srank[t] < k) { ov[srank[t]] = key_value(surv[t]); oi[srank[t]] = key_index(surv[t]); }
                return;
            }
        }
    }
    if (threadIdx.x >= 64) return;
    Key h[LMAX];
    int pos[LMAX], len[LMAX];
#pragma unroll
    for (int u = 0; u < LMAX; ++u) {
        const int li = lane + 64 * u;
        const bool ok = li < nl;
        const Key e = lst[ok ? li * k : 0];
        h[u] = ok ? e : taken_key();
        pos[u] = ok ? 0 : k;
        len[u] = ok ? q : k;
    }
    const float *lrow = logits + (size_t)row * lld;
    for (int r = 0; r < k; ++r) {
        Key b = h[0];
        int bu = 0;
#pragma unroll
        for (int u = 1; u < LMAX; ++u)
            if (h[u] > b) { b = h[u]; bu = u; }
        const Key w = wave_best(b);
        if (lane == 0) { ov[r] = key_value(w); oi[r] = key_index(w); }
        // the owner of the winning head moves to that list's next entry (a
        // "taken" entry past a list of k).  Several lanes match only when the
        // winner is such an entry, and then every head left is one too.
        bool need = false;
        int nli = 0;
        if (b == w) {
#pragma unroll
            for (int u = 0; u < LMAX; ++u)
                if (u == bu) {
                    const int nx = ++pos[u];
                    need = nx == len[u] && len[u] < k;
                    nli = lane + 64 * u;
                    const Key e = lst[nx < len[u] ? nli * k + nx : 0];
                    h[u] = nx < len[u] ? e : taken_key();
                }
        }
        // lists of q that ran out: the whole wave refills each from its chunk
        unsigned long long m = __ballot(need);
        while (m) {
            const int L = __builtin_ctzll(m);
            m &= m - 1;
            const int li = __builtin_amdgcn_readlane(nli, L);
            const int lo = li * TOPK_CHUNK;
            Key x[VPL];
            load_sorted(x, lrow, nullptr, lo, min(vocab, lo + TOPK_CHUNK));
            for (int t = 0; t < k; ++t) {
                const Key y = take_best(x);
                if (lane == 0) lst[li * k + t] = y;
            }
            __builtin_amdgcn_wave_barrier();
            if (lane == L) {
#pragma unroll
                for (int u = 0; u < LMAX; ++u)
                    if (u == bu) {
                        len[u] = k;
                        h[u] = lst[li * k + pos[u]];
                    }
            }
        }
    }
}

}  // namespace

int topk_chunks(int vocab) { return (vocab + TOPK_CHUNK - 1) / TOPK_CHUNK; }

size_t topk_scratch_entries(int rows, int vocab, int k) {
    // the first stage's candidates, then the second stage's, side by side
    const size_t n1 = (size_t)topk_chunks(vocab) * k;
    return (size_t)rows * (n1 + (size_t)topk_chunks((int)n1) * k);
}

hipError_t topk_rows(const float *logits, long long ld, int rows, int vocab, int k, float *part_v, int32_t *part_i,
                     float *vals, int32_t *idx, const float *hidden, int H, const void *w, int rank, float *hout,
                     hipStream_t s) {
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
    if (nc1 > 1 && nc1 <= TOPK_MERGE_LISTS && (size_t)nc1 * k * sizeof(unsigned long long) <= TOPK_MERGE_LDS) {
        // first stage (each chunk's q best), then the merge of its sorted lists
        const int q = std::min(k, TOPK_QUOTA);
        hipLaunchKernelGGL(topk_wave<TOPK_CHUNK / 64>, dim3(nc1, rows), dim3(64), 0, s, logits, (const int32_t *)nullptr,
                           vocab, ld, TOPK_CHUNK, q, part_v, part_i, nc1 * q);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        const HProjArgs ha{hidden, H, (const uint16_t *)w, rank, rows, hout};
        const int pblocks = (rows * rank + 3) / 4;
        hipLaunchKernelGGL((topk_merge<TOPK_MERGE_LISTS / 64, TOPK_CHUNK / 64>), dim3(rows + pblocks), dim3(MERGE_THREADS),
                           (size_t)nc1 * k * sizeof(unsigned long long), s, part_v, part_i, nc1, q, k, (long long)nc1 * q,
                           logits, ld, vocab, vals, idx, rows, ha);
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
        if (e != hipSuccess) return e;
        if (last) return hidden_projection(hidden, H, w, rank, rows, hout, s);
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
