// Kernels of the batched multi-sequence round: S independent sequences, each
// with its own draft KV cache ([atlas dflash_head] "DflashProposerState":
// per-sequence drafter state), run one drafting round together, so that each
// projection streams its weights once for all S * b block rows.
//
// The projections are the split-K skinny GEMM (gemm.hip) over the stacked
// rows, and the norms are the row RMSNorm (norm_rope.hip).  This file holds
// the per-sequence steps between them ([DflashDraft] "forward_round"):
//   batch_qk_rope  q/k head RMSNorm + NeoX rope (f64 angles) x mscale; q
//                  (also x log2(e)/sqrt(d)) goes to a bf16 MFMA operand
//                  buffer, the block's k and v to the sequence's cache at
//                  rows [len, len + b) (transient, never committed);
//   batch_attn     non-causal attention of the G q heads of one kv head over
//                  one key split of one sequence (the window's ctx keys and
//                  the block keys alike come from the cache).  The key
//                  blocks are staged through LDS, 64 keys at a time, by all
//                  eight waves; wave v computes q head v with MFMA 16x16x32
//                  bf16 (S^T = K Q^T, online softmax, O^T += V^T P^T) and
//                  writes the split's partial (m, l, O).  Each wave's
//                  dependent chain (reads, MFMAs, softmax) is what bounds
//                  it, so the kernel is held to 128 VGPRs and two
//                  workgroups share a compute unit;
//   batch_merge    the splits' log-sum-exp merge into the attention output;
//   d2_dyn/d2_conv the DFlash2 conv wrap: the dynamic coefficients of a
//                  sublayer's normed input, its prepare conv, and its finish
//                  conv added into the residual stream.
#include "batch.h"
#include "common.h"

namespace dfl {
namespace {

// q / k / v of one stacked row: one wave per (row, head); lane j < d/2 holds
// the rope pair (j, j + d/2)
__global__ __launch_bounds__(256) void batch_qk_rope(BatchArgs a) {
    const int s = blockIdx.x / 16, r = blockIdx.x % 16;
    const int head = blockIdx.y * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int nq = a.nq, nkv = a.nkv, d = a.d, half = d >> 1;
    if (head >= nq + 2 * nkv) return;
    const bool act = lane < half;
    if (head < nq) {
        const int h = head / a.G, j = head - h * a.G;
        uint16_t *dst = a.q + ((((size_t)s * nkv + h) * a.G + j) * 16 + r) * d;
        if (r >= a.b) {                                   // padding rows of the MFMA tile
            if (act) { dst[lane] = 0; dst[lane + half] = 0; }
            return;
        }
    } else if (r >= a.b) {
        return;
    }
    const float *row = a.qkv + (size_t)(s * a.b + r) * a.qkv_ld;
    const BatchSeq &sq = a.seq[s];
    double sv = 0.0, cv = 1.0;
    if (act) sincos((double)a.pos[s * a.b + r] * a.inv_freq[lane], &sv, &cv);
    const float c = (float)cv, sn = (float)sv;
    if (head < nq + nkv) {                                // q or k head: RMSNorm, rope, scale
        const bool isq = head < nq;
        const float *src = row + (isq ? head * d : a.qd + (head - nq) * d);
        const float x0 = act ? src[lane] : 0.f, x1 = act ? src[lane + half] : 0.f;
        const float inv = 1.f / sqrtf(wave_sum(x0 * x0 + x1 * x1) / (float)d + a.eps);
        if (!act) return;
        const float *g = isq ? a.g_q : a.g_k;
        const float y0 = g[lane] * (x0 * inv), y1 = g[lane + half] * (x1 * inv);
        const float sc = isq ? a.mscale * a.qscale : a.mscale;
        const float o0 = (y0 * c - y1 * sn) * sc, o1 = (y1 * c + y0 * sn) * sc;
        if (isq) {
            const int h = head / a.G, j = head - h * a.G;
            uint16_t *dst = a.q + ((((size_t)s * nkv + h) * a.G + j) * 16 + r) * d;
            dst[lane] = (uint16_t)f32_to_bf16_bits(o0);
            dst[lane + half] = (uint16_t)f32_to_bf16_bits(o1);
        } else {
            const int h = head - nq, kr = sq.len + r;
            char *kl = sq.kv.k + (size_t)a.layer * sq.kv.lstride;
            const int pg = kv_page(sq.kv, kr);
            *reinterpret_cast<uint16_t *>(kl + kv_k_off(sq.kv, pg, nkv, h, kr, d, lane)) = (uint16_t)f32_to_bf16_bits(o0);
            *reinterpret_cast<uint16_t *>(kl + kv_k_off(sq.kv, pg, nkv, h, kr, d, lane + half)) =
                (uint16_t)f32_to_bf16_bits(o1);
        }
    } else if (act) {                                     // v head: raw, transposed store
        const int h = head - nq - nkv, kr = sq.len + r;
        const float *src = row + a.qd + a.kvd + h * d;
        char *vl = sq.kv.v + (size_t)a.layer * sq.kv.lstride;
        const int pg = kv_page(sq.kv, kr);
        *reinterpret_cast<uint16_t *>(vl + kv_v_off(sq.kv, pg, nkv, h, kr, d, lane)) = (uint16_t)f32_to_bf16_bits(src[lane]);
        *reinterpret_cast<uint16_t *>(vl + kv_v_off(sq.kv, pg, nkv, h, kr, d, lane + half)) =
            (uint16_t)f32_to_bf16_bits(src[lane + half]);
    }
}

// Key staging: a 32-key block is NPART parts of 64 lanes x 16 bytes, in the
// order the MFMAs read them: K parts (key tile kt, d chunk c), then V^T
// parts (d tile t).  Within K tile kt, MFMA row n16 holds key
// 8 (n16 / 4) + 4 kt + n16 % 4 of the block, so after S^T = K Q^T the lane
// (query n16, group g) holds the scores of keys 8g .. 8g + 7: exactly the
// P^T operand it needs for O^T += V^T P^T.
template <int D> struct BA {
    static constexpr int NC = D / 32;                  // 32-wide d chunks (8 bf16 per lane)
    static constexpr int NDT = D / 16;                 // 16-wide d tiles of V^T
    static constexpr int NPART = 2 * NC + NDT;
    static constexpr int NB = BATCH_CHUNK_KEYS / 32;   // blocks per staged chunk
    static constexpr int PIECES = NB * NPART * 64;     // 16-byte pieces per chunk
    static constexpr int PER_THREAD = PIECES / BATCH_ATTN_THREADS;
    static_assert(PIECES % BATCH_ATTN_THREADS == 0, "pieces split evenly over the threads");
};

template <int D>
__global__ __launch_bounds__(BATCH_ATTN_THREADS, 2) void batch_attn(BatchArgs a) {
    using T = BA<D>;
    constexpr int NC = T::NC, NDT = T::NDT, NPART = T::NPART, NB = T::NB;
    __shared__ u32x4 stage[NB * NPART * 64];
    const int split = blockIdx.x, h = blockIdx.y, s = blockIdx.z;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n16 = lane & 15, g = lane >> 4;
    const BatchSeq &sq = a.seq[s];
    const int nkeys = sq.len + a.b;                   // window's ctx keys + the block's keys
    const int a0 = sq.win_lo & ~31;
    const int k_lo = a0 + split * a.kps;
    const int k_hi = min(nkeys, k_lo + a.kps);
    const char *kl = sq.kv.k + (size_t)a.layer * sq.kv.lstride;
    const char *vl = sq.kv.v + (size_t)a.layer * sq.kv.lstride;
    const int nkv = a.nkv;
    const bool comp = wave < a.G;

    // this wave's q head: rows n16, d chunks c (B operand of S^T = K Q^T)
    u32x4 qf[NC];
    {
        const uint16_t *qsrc = a.q + ((((size_t)s * nkv + h) * a.G + (comp ? wave : 0)) * 16 + n16) * D + 8 * g;
#pragma unroll
        for (int c = 0; c < NC; ++c) qf[c] = *reinterpret_cast<const u32x4 *>(qsrc + 32 * c);
    }
    float m = -1e30f, l = 0.f;
    f32x4 o[NDT];
#pragma unroll
    for (int t = 0; t < NDT; ++t) o[t] = f32x4{0.f, 0.f, 0.f, 0.f};

    // global address of piece i of the chunk starting at key k0 (every address
    // stays inside the sequence's rows [a0, roundup(nkeys, 8)))
    auto piece_ptr = [&](int i, int k0) -> const u32x4 * {
        const int part = i / 64, pl = i & 63, pn = pl & 15, pg = pl >> 4;
        const int blk = part / NPART, q = part - blk * NPART;
        const int kb = k0 + 32 * blk;
        if (q < 2 * NC) {
            const int kt = q / NC, c = q - kt * NC;
            int key = kb + 8 * (pn >> 2) + 4 * kt + (pn & 3);
            key = min(key, nkeys - 1);
            return reinterpret_cast<const u32x4 *>(kl + kv_k_off(sq.kv, kv_page(sq.kv, key), nkv, h, key, D, 32 * c + 8 * pg));
        }
        const int t = q - 2 * NC;
        int key = kb + 8 * pg;
        key = min(key, (nkeys - 1) & ~7);
        return reinterpret_cast<const u32x4 *>(vl + kv_v_off(sq.kv, kv_page(sq.kv, key), nkv, h, key, D, 16 * t + pn));
    };

    u32x4 reg[T::PER_THREAD];
    const int nchunk = k_hi > k_lo ? (k_hi - k_lo + 32 * NB - 1) / (32 * NB) : 0;
    if (nchunk > 0) {
#pragma unroll
        for (int i = 0; i < T::PER_THREAD; ++i) reg[i] = *piece_ptr(tid + i * BATCH_ATTN_THREADS, k_lo);
    }
    for (int ch = 0; ch < nchunk; ++ch) {
        const int k0 = k_lo + ch * 32 * NB;
        __syncthreads();                               // the previous chunk's LDS reads are done
#pragma unroll
        for (int i = 0; i < T::PER_THREAD; ++i) stage[tid + i * BATCH_ATTN_THREADS] = reg[i];
        __syncthreads();
        if (ch + 1 < nchunk) {                         // next chunk's loads overlap this chunk's math
#pragma unroll
            for (int i = 0; i < T::PER_THREAD; ++i) reg[i] = *piece_ptr(tid + i * BATCH_ATTN_THREADS, k0 + 32 * NB);
        }
        if (!comp) continue;
#pragma unroll
        for (int blk = 0; blk < NB; ++blk) {
            const int kb = k0 + 32 * blk;
            if (kb >= k_hi) break;
            const u32x4 *bp = stage + blk * NPART * 64 + lane;
            f32x4 sc4[2];
#pragma unroll
            for (int kt = 0; kt < 2; ++kt) {
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int c = 0; c < NC; ++c)
                    acc = mfma_bf16(__builtin_bit_cast(bf16x8, bp[(kt * NC + c) * 64]), __builtin_bit_cast(bf16x8, qf[c]), acc);
                sc4[kt] = acc;
            }
            // lane (n16, g) holds keys kb + 8g + i, i = 0..7, of query n16
            float sc[8];
            float bmax = -INFINITY;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int key = kb + 8 * g + i;
                const bool ok = key >= sq.win_lo && key < k_hi;
                sc[i] = ok ? sc4[i >> 2][i & 3] : -INFINITY;
                bmax = fmaxf(bmax, sc[i]);
            }
            bmax = group4_max(bmax);
            const float m_new = fmaxf(m, bmax);
            const float corr = __builtin_amdgcn_exp2f(m - m_new);
            float psum = 0.f;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                sc[i] = __builtin_amdgcn_exp2f(sc[i] - m_new);
                psum += sc[i];
            }
            l = l * corr + group4_sum(psum);
            m = m_new;
            const bf16x8 pb = to_bf16x8(sc);
#pragma unroll
            for (int t = 0; t < NDT; ++t) {
                u32x4 vv = bp[(2 * NC + t) * 64];
                // zero the values of keys outside the split (their rows may hold anything)
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    const int key = kb + 8 * g + 2 * w;
                    const uint32_t lo = key >= sq.win_lo && key < k_hi ? 0x0000FFFFu : 0u;
                    const uint32_t hi = key + 1 >= sq.win_lo && key + 1 < k_hi ? 0xFFFF0000u : 0u;
                    vv[w] &= lo | hi;
                }
                o[t] = mfma_bf16(__builtin_bit_cast(bf16x8, vv), pb, o[t] * corr);
            }
        }
    }
    if (!comp) return;
    // partials: O^T tile t holds d = 16t + 4g + j of query n16
    const size_t item = (((size_t)s * nkv + h) * a.nsplit + split) * a.G + wave;
    float *po = a.po + (item * 16 + n16) * D;
#pragma unroll
    for (int t = 0; t < NDT; ++t) *reinterpret_cast<f32x4 *>(po + 16 * t + 4 * g) = o[t];
    if (g == 0) *reinterpret_cast<float2 *>(a.pml + (item * 16 + n16) * 2) = make_float2(m, l);
}

// one wave per (stacked row, q head): O = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s.
// Lane i reads split i's (m, l) (nsplit <= 64), so M and L take one load
// round trip and two wave reductions; the partial O rows are then read 8
// splits at a time, all loads of a group issued before the first use.
__global__ __launch_bounds__(256) void batch_merge(BatchArgs a) {
    const int unit = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int rows = a.S * a.b;
    if (unit >= rows * a.nq) return;
    const int row = unit / a.nq, hq = unit - row * a.nq;
    const int s = row / a.b, r = row - s * a.b;
    const int h = hq / a.G, j = hq - h * a.G, d = a.d, ns = a.nsplit;
    const size_t item0 = (((size_t)s * a.nkv + h) * ns) * a.G + j;     // split sp: item0 + sp * G
    float2 ml = make_float2(-1e30f, 0.f);
    if (lane < ns) ml = *reinterpret_cast<const float2 *>(a.pml + ((item0 + (size_t)lane * a.G) * 16 + r) * 2);
    const float M = wave_max(ml.x);
    const float w = lane < ns ? __builtin_amdgcn_exp2f(ml.x - M) : 0.f;
    const float L = wave_sum(w * ml.y);
    const float *po = a.po + (item0 * 16 + r) * d + lane;
    const size_t sstride = (size_t)a.G * 16 * d;                       // floats between consecutive splits
    const bool two = d > 64;
    float acc0 = 0.f, acc1 = 0.f;
    constexpr int U = 8;
    for (int sp0 = 0; sp0 < ns; sp0 += U) {
        float v0[U], v1[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int sp = min(sp0 + u, ns - 1);
            v0[u] = po[(size_t)sp * sstride];
            v1[u] = two ? po[(size_t)sp * sstride + 64] : 0.f;
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            // the split index is the same on every lane: a scalar read of lane sp
            const float ws = sp0 + u < ns ? __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), sp0 + u)) : 0.f;
            acc0 += ws * v0[u];
            acc1 += ws * v1[u];
        }
    }
    float *dst = a.attn + (size_t)row * a.qd + (size_t)hq * d;
    const float il = 1.f / L;
    dst[lane] = acc0 * il;
    if (two) dst[lane + 64] = acc1 * il;
}

// ---- DFlash2 grouped dynamic causal conv ([memra dflash module] "Dflash2Conv";
// [DflashDraft] "d2_conv_prepare", "d2_conv_finish") --------------------------

// D[row][j] = (xn[row] . W_dyn[j]) * scale[j]: one wave per (row, j); the
// 4G coefficients of a row are laid out [half][group][tap]
template <int WT>
__global__ __launch_bounds__(256) void d2_dyn(const float *xn, int H, const void *w, const float *scale, int nj, int rows,
                                              float *D) {
    const int unit = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
    if (unit >= rows * nj) return;
    const int row = unit / nj, j = unit - row * nj;
    const float *x = xn + (size_t)row * H;
    float acc = 0.f;
    for (int c = lane; c < H; c += 64) {
        float wv;
        if constexpr (WT == WT_BF16) wv = bf16_bits_to_f32(reinterpret_cast<const uint16_t *>(w)[(size_t)j * H + c]);
        else if constexpr (WT == WT_FP8) wv = __builtin_amdgcn_cvt_f32_fp8((uint32_t)reinterpret_cast<const uint8_t *>(w)[(size_t)j * H + c], 0);
        else wv = reinterpret_cast<const float *>(w)[(size_t)j * H + c];
        acc += x[c] * wv;
    }
    acc = wave_sum(acc);
    if (lane == 0) D[(size_t)row * nj + j] = acc * (WT == WT_FP8 ? scale[j] : 1.f);
}

// Two-tap causal conv over each sequence's block rows (row 0's predecessor
// is zero), coefficients base[c][tap] + D[row][half][g(c)][tap] with
// g(c) = floor(c G / H); tap 0 multiplies row r - 1, tap 1 row r.  Writes
// the result, or adds it to dst (the finish conv into the residual).
__global__ __launch_bounds__(256) void d2_conv(const float *src, const float *D, int half, const float *base, int H, int G,
                                               int b, int rows, float *dst, int accumulate) {
    const int row = blockIdx.y, c = blockIdx.x * 256 + threadIdx.x;
    if (row >= rows || c >= H) return;
    const int r = row % b, g = (int)(((long long)c * G) / H);
    const float *Dr = D + (size_t)row * 4 * G + (size_t)(half * G + g) * 2;
    const float *bh = base + (size_t)half * H * 2 + (size_t)c * 2;
    const float cur = src[(size_t)row * H + c];
    const float prev = r > 0 ? src[(size_t)(row - 1) * H + c] : 0.f;
    const float y = (bh[0] + Dr[0]) * prev + (bh[1] + Dr[1]) * cur;
    float *o = dst + (size_t)row * H + c;
    *o = accumulate ? *o + y : y;
}

}  // namespace

hipError_t d2_dyn_launch(const float *xn, int H, const void *w, const float *scale, int wt, int nj, int rows, float *D,
                         hipStream_t s) {
    const dim3 grid((rows * nj + 3) / 4), block(256);
    if (wt == WT_BF16) hipLaunchKernelGGL(d2_dyn<WT_BF16>, grid, block, 0, s, xn, H, w, scale, nj, rows, D);
    else if (wt == WT_FP8) hipLaunchKernelGGL(d2_dyn<WT_FP8>, grid, block, 0, s, xn, H, w, scale, nj, rows, D);
    else hipLaunchKernelGGL(d2_dyn<WT_F32>, grid, block, 0, s, xn, H, w, scale, nj, rows, D);
    return hipGetLastError();
}

hipError_t d2_conv_launch(const float *src, const float *D, int half, const float *base, int H, int G, int b, int rows,
                          float *dst, bool accumulate, hipStream_t s) {
    hipLaunchKernelGGL(d2_conv, dim3((H + 255) / 256, rows), dim3(256), 0, s, src, D, half, base, H, G, b, rows, dst,
                       accumulate ? 1 : 0);
    return hipGetLastError();
}

hipError_t batch_qk_rope_launch(const BatchArgs &a, hipStream_t s) {
    hipLaunchKernelGGL(batch_qk_rope, dim3(a.S * 16, (a.nq + 2 * a.nkv + 3) / 4), dim3(256), 0, s, a);
    return hipGetLastError();
}

hipError_t batch_attn_launch(const BatchArgs &a, hipStream_t s) {
    const dim3 grid(a.nsplit, a.nkv, a.S), block(BATCH_ATTN_THREADS);
    if (a.d == 128) hipLaunchKernelGGL(batch_attn<128>, grid, block, 0, s, a);
    else if (a.d == 64) hipLaunchKernelGGL(batch_attn<64>, grid, block, 0, s, a);
    else return hipErrorInvalidValue;
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(batch_merge, dim3((a.S * a.b * a.nq + 3) / 4), dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace dfl
