// Non-causal grouped-query attention of the block queries over the draft KV
// cache ([DflashDraft] "forward_round": block K/V sit at rows
// [len, len + b) and attention is full over all len + b keys; "forward":
// full non-causal attention, no mask, no window).
//
// Per kv head h, the queries are the b block rows x the G = nq / nkv q heads
// that read h (q head hq reads kv head floor(hq / G)).  Query index
// qi = r * G + (hq - h * G).  They are padded to 16-query tiles.
//
// Split over keys (flash-decode style):
// * Workgroup (split s, kv head h) runs over keys [s * kps, (s+1) * kps) in
//   blocks of 32, with an online softmax.  It writes unnormalised partials
//   (m, l, O) per query.  A merge kernel combines the splits in order.
// * Scores come from S^T = K . Q^T, so each lane owns one query (l % 16) and
//   8 keys.  Both MFMA tiles of a block map MFMA row i to key
//   8 * (i / 4) + 4t + (i % 4).  Lane group g then holds keys 8g .. 8g+7,
//   which is exactly the B operand of the next product.
// * O^T = V^T . P^T, with V stored transposed in the cache ([d][cap]), so the
//   A operand is 8 contiguous keys.  The output tile has the same query per
//   lane as the scores.  Hence the running max, running sum and rescale are
//   lane-local, and only the row max/sum need the 4-lane-group shuffles.
// * bf16 cache: Q and P go through bf16 MFMA 16x16x32.  f32 cache: MFMA
//   16x16x4 f32.
#include "common.h"
#include "kernels.h"

namespace dfl {

template <bool F32, int D>
struct KVFrag;

// one 16-key MFMA tile row's K data for d-step s: bf16 -> 8 values (16 B)
template <int D>
struct KVFrag<false, D> {
    static constexpr int DSTEP = 32;          // d per MFMA (16x16x32)
    static constexpr int NDS = D / DSTEP;
};
template <int D>
struct KVFrag<true, D> {
    static constexpr int DSTEP = 16;          // d per 4 MFMAs (16x16x4, float4 per lane)
    static constexpr int NDS = D / DSTEP;
};

template <bool F32, int D, int TPW>
__global__ __launch_bounds__(256) void attn_kernel(AttnArgs a) {
    using FR = KVFrag<F32, D>;
    constexpr int NDS = FR::NDS;
    constexpr int NDT = D / 16;               // d tiles of the output
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 4, r16 = lane & 15;
    const int split = blockIdx.x, h = blockIdx.y;
    const int G = a.nq / a.nkv;
    const int nqh = a.b * G;                  // real queries of this kv head
    const int qtiles = a.qpad / 16;

    const int kbeg = split * a.kps;
    const int kend = min(kbeg + a.kps, a.n_keys);

    const size_t kv_head = (size_t)h * a.cap * D;   // same element offset for K [cap][d] and V [d][cap]

    for (int tb = 0; tb < TPW; ++tb) {
        const int qt = wave + 4 * tb;
        if (qt >= qtiles) break;
        // ---- this lane's query (B operand of S^T): Q[qi][d] ----
        const int qi = qt * 16 + r16;
        const bool qvalid = qi < nqh;
        const float *qrow = a.q + (size_t)((qvalid ? qi / G : 0) * a.nq + h * G + (qvalid ? qi % G : 0)) * D;

        bf16x8 qb[F32 ? 1 : NDS];
        float4 qf[F32 ? NDS : 1];
        if constexpr (!F32) {
#pragma unroll
            for (int s = 0; s < NDS; ++s) {
                float x[8];
                float4 p0 = qvalid ? ld_f4(qrow + 32 * s + 8 * g) : make_float4(0, 0, 0, 0);
                float4 p1 = qvalid ? ld_f4(qrow + 32 * s + 8 * g + 4) : make_float4(0, 0, 0, 0);
                x[0] = p0.x; x[1] = p0.y; x[2] = p0.z; x[3] = p0.w; x[4] = p1.x; x[5] = p1.y; x[6] = p1.z; x[7] = p1.w;
                qb[s] = to_bf16x8(x);
            }
        } else {
#pragma unroll
            for (int s = 0; s < NDS; ++s) qf[s] = qvalid ? ld_f4(qrow + 16 * s + 4 * g) : make_float4(0, 0, 0, 0);
        }

        float m_run = -1e30f, l_run = 0.f;
        f32x4 o[NDT];
#pragma unroll
        for (int t = 0; t < NDT; ++t) o[t] = f32x4{0.f, 0.f, 0.f, 0.f};

        for (int k0 = kbeg; k0 < kend; k0 += 32) {
            // ---- S^T for 32 keys: two 16-key tiles ----
            f32x4 st[2];
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                st[t] = f32x4{0.f, 0.f, 0.f, 0.f};
                const int key = k0 + 8 * (r16 >> 2) + 4 * t + (r16 & 3);   // MFMA row r16 of tile t
                if constexpr (!F32) {
                    const uint16_t *kr = reinterpret_cast<const uint16_t *>(a.kc) + kv_head + (size_t)key * D;
#pragma unroll
                    for (int s = 0; s < NDS; ++s) {
                        u32x4 kv = *reinterpret_cast<const u32x4 *>(kr + 32 * s + 8 * g);
                        st[t] = mfma_bf16(__builtin_bit_cast(bf16x8, kv), qb[s], st[t]);
                    }
                } else {
                    const float *kr = reinterpret_cast<const float *>(a.kc) + kv_head + (size_t)key * D;
#pragma unroll
                    for (int s = 0; s < NDS; ++s) {
                        float4 kv = ld_f4(kr + 16 * s + 4 * g);
                        st[t] = mfma_f32(kv.x, qf[s].x, st[t]);
                        st[t] = mfma_f32(kv.y, qf[s].y, st[t]);
                        st[t] = mfma_f32(kv.z, qf[s].z, st[t]);
                        st[t] = mfma_f32(kv.w, qf[s].w, st[t]);
                    }
                }
            }
            // lane (query r16, group g) holds keys k0 + 8g + 4t + j
            float sc[8];
            float bmax = -INFINITY;
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int key = k0 + 8 * g + 4 * t + j;
                    float v = st[t][j] * a.scale_log2;
                    v = key < kend ? v : -INFINITY;
                    sc[4 * t + j] = v;
                    bmax = fmaxf(bmax, v);
                }
            bmax = group4_max(bmax);
            const float m_new = fmaxf(m_run, bmax);
            const float corr = exp2f(m_run - m_new);
            float psum = 0.f;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                sc[i] = exp2f(sc[i] - m_new);
                psum += sc[i];
            }
            psum = group4_sum(psum);
            l_run = l_run * corr + psum;
            m_run = m_new;
#pragma unroll
            for (int t = 0; t < NDT; ++t) o[t] *= corr;

            // ---- O^T += V^T . P^T ----
            const bool full = (k0 + 32 <= kend);
            if constexpr (!F32) {
                const bf16x8 pb = to_bf16x8(sc);
#pragma unroll
                for (int t = 0; t < NDT; ++t) {
                    const uint16_t *vr = reinterpret_cast<const uint16_t *>(a.vc) + kv_head +
                                         (size_t)(16 * t + r16) * a.cap + k0 + 8 * g;
                    u32x4 vv = *reinterpret_cast<const u32x4 *>(vr);
                    if (!full) {
                        // keys past the end hold stale data: zero them so 0 * NaN cannot occur
#pragma unroll
                        for (int w = 0; w < 4; ++w) {
                            const int kk = k0 + 8 * g + 2 * w;
                            uint32_t m = (kk < kend ? 0x0000FFFFu : 0u) | (kk + 1 < kend ? 0xFFFF0000u : 0u);
                            vv[w] &= m;
                        }
                    }
                    o[t] = mfma_bf16(__builtin_bit_cast(bf16x8, vv), pb, o[t]);
                }
            } else {
#pragma unroll
                for (int t = 0; t < NDT; ++t) {
                    const float *vr = reinterpret_cast<const float *>(a.vc) + kv_head +
                                      (size_t)(16 * t + r16) * a.cap + k0 + 8 * g;
                    float4 v0 = ld_f4(vr), v1 = ld_f4(vr + 4);
                    float vk[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        if (!full && k0 + 8 * g + i >= kend) vk[i] = 0.f;
                        o[t] = mfma_f32(vk[i], sc[i], o[t]);
                    }
                }
            }
        }

        // ---- partials: lane holds O^T[d = 16t + 4g + j][query r16] ----
        if (qi < a.qpad) {
            const size_t pq = ((size_t)h * a.nsplit + split) * a.qpad + qi;
            if (g == 0) {
                a.part_ml[pq * 2 + 0] = m_run;
                a.part_ml[pq * 2 + 1] = l_run;
            }
#pragma unroll
            for (int t = 0; t < NDT; ++t)
                *reinterpret_cast<f32x4 *>(a.part_o + pq * D + 16 * t + 4 * g) = o[t];
        }
    }
}

// Merge the splits of one (kv head, query): O = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s.
__global__ __launch_bounds__(128) void attn_merge_kernel(AttnArgs a) {
    const int qi = blockIdx.x, h = blockIdx.y, dd = threadIdx.x;
    const int G = a.nq / a.nkv;
    if (qi >= a.b * G || dd >= a.d) return;
    const size_t base = (size_t)h * a.nsplit * a.qpad + qi;
    float M = -1e30f;
    for (int s = 0; s < a.nsplit; ++s) M = fmaxf(M, a.part_ml[(base + (size_t)s * a.qpad) * 2]);
    float L = 0.f, acc = 0.f;
    for (int s = 0; s < a.nsplit; ++s) {
        const size_t pq = base + (size_t)s * a.qpad;
        const float w = exp2f(a.part_ml[pq * 2] - M);
        L += w * a.part_ml[pq * 2 + 1];
        acc += w * a.part_o[pq * a.d + dd];
    }
    const int r = qi / G, hq = h * G + qi % G;
    a.out[((size_t)r * a.nq + hq) * a.d + dd] = acc / L;
}

void attn_plan(AttnArgs &a, int max_splits) {
    const int G = a.nq / a.nkv;
    a.qpad = (a.b * G + 15) / 16 * 16;
    // aim for ~256 workgroups, at least 64 keys per split
    int want = 256 / a.nkv;
    if (want < 1) want = 1;
    int ns = (a.n_keys + 63) / 64;
    if (ns > want) ns = want;
    if (ns > max_splits) ns = max_splits;
    if (ns < 1) ns = 1;
    int kps = (a.n_keys + ns - 1) / ns;
    kps = (kps + 31) / 32 * 32;
    a.kps = kps;
    a.nsplit = (a.n_keys + kps - 1) / kps;
}

template <bool F32, int D>
static void launch_attn(const AttnArgs &a, hipStream_t s) {
    const int qtiles = a.qpad / 16;
    dim3 grid(a.nsplit, a.nkv), block(256);
    if (qtiles <= 4) hipLaunchKernelGGL((attn_kernel<F32, D, 1>), grid, block, 0, s, a);
    else if (qtiles <= 8) hipLaunchKernelGGL((attn_kernel<F32, D, 2>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((attn_kernel<F32, D, 4>), grid, block, 0, s, a);
}

hipError_t attention(const AttnArgs &a, hipStream_t s) {
    if (a.kv_f32) {
        if (a.d == 64) launch_attn<true, 64>(a, s);
        else launch_attn<true, 128>(a, s);
    } else {
        if (a.d == 64) launch_attn<false, 64>(a, s);
        else launch_attn<false, 128>(a, s);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(attn_merge_kernel, dim3(a.qpad, a.nkv), dim3(a.d), 0, s, a);
    return hipGetLastError();
}

}  // namespace dfl
