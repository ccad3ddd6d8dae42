// Skinny GEMM for the drafter's projections:  Y[M, N] (epi)= A[M, K] . W[N, K]^T
//
// A: f32 activations (M = 16 block rows on the round path; ctx rows on the
//    ingest / first-light path).
// W: f32, bf16 or fp8 e4m3fn weights in torch Linear layout [N, K], streamed
//    from HBM once per call.  This stream is the dominant cost of a round.
//
// Work item = (MT 16-row tiles) x (64 output columns) x (one K split).
// * A workgroup of 4 waves takes one item.  Wave w owns the 16 columns
//   [16w, 16w + 16) of the group (with SwiGLU, also the matching 16 up
//   columns).
// * Per K chunk, every thread first issues its activation loads, then every
//   wave all of its weight loads.  Each lane loads one 16-byte piece per
//   step and weight row: bf16 8 values (K step 32), fp8 16 codes (K step
//   64), f32 4 values (K step 16).
// * While the weight loads are in flight, the workgroup stages the
//   activations in LDS once, in MFMA fragment order.  bf16/fp8 weights use the activations split into bf16
//   hi + lo parts (two MFMAs 16x16x32 per step, ~16-bit activation
//   precision).  f32 weights use MFMA 16x16x4 f32 on the f32 values.
// * The MFMAs then read A from LDS (one 16-byte read per fragment) and W
//   from registers.
// * Split-K: each workgroup stores its partial tiles with device-coherent
//   stores, then bumps a per-column-group counter.  The last workgroup to
//   arrive sums the partials in split order and applies the epilogue.  The
//   result is therefore independent of scheduling.  Only workgroup-scope
//   fences are used (no L2 writeback / invalidate).
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace dfl {

template <int WT> struct WCfg;
// KS: K per 16-byte weight load; FR: 16-byte A fragments per step and m-tile
template <> struct WCfg<WT_BF16> { static constexpr int KS = 32, ES = 2, FR = 2; };
template <> struct WCfg<WT_FP8>  { static constexpr int KS = 64, ES = 1, FR = 4; };
template <> struct WCfg<WT_F32>  { static constexpr int KS = 16, ES = 4, FR = 1; };

__device__ __forceinline__ float silu(float x) { return x / (1.f + __expf(-x)); }

// Device-coherent 16-byte store / load of split-K partials (SC1: written
// through to memory, read past the XCD's L2), through a buffer resource whose
// base is uniform over the wave; the byte offset is per lane.  A lane's four
// partial sums are one 16-byte access, so a wave writes and reads 1 KB runs
// (scattered 4-byte write-through stores cost far more per byte).
constexpr int CPOL_SC1 = 16;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t part_rsrc(const float *base) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(base), 0, 0x7fffffff, 0x00020000);
}
__device__ __forceinline__ void st_coherent16(float *base, uint32_t off, f32x4 v) {
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), part_rsrc(base), off, 0, CPOL_SC1);
}
__device__ __forceinline__ f32x4 ld_coherent16(const float *base, uint32_t off) {
    return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(part_rsrc(base), off, 0, CPOL_SC1));
}

// Stage A[m0 .. m0+16*MT)[k0 .. k0 + NSTEP*KS) into LDS fragments, in two
// halves: load_a issues every load of the chunk at once (addresses clamped
// into range, so the values stay in registers), put_a converts them and
// writes the fragments; the caller issues the weight loads in between.
// Layout: lds[((mt * NSTEP + s) * FR + f) * 64 + lane] (16 bytes each).
template <int WT, int MT, int NSTEP> struct AStage {
    static constexpr int GROUPS = NSTEP * WCfg<WT>::KS / 8;   // 8-float groups per row
    static constexpr int TOTAL = MT * 16 * GROUPS;
    static constexpr int IT = (TOTAL + 255) / 256;            // groups per thread
    float4 v[IT][2];
};

template <int WT, int MT, int NSTEP>
__device__ __forceinline__ void load_a(AStage<WT, MT, NSTEP> &st, const GemmArgs &p, int m0, int k0, int kvalid) {
    using S = AStage<WT, MT, NSTEP>;
#pragma unroll
    for (int it = 0; it < S::IT; ++it) {
        const int idx = min((int)threadIdx.x + 256 * it, S::TOTAL - 1);
        const int rowl = idx / S::GROUPS, j = idx - rowl * S::GROUPS;
        const int row = min(m0 + rowl, p.M - 1), kk = min(8 * j, kvalid - 8);
        const float *src = p.A + (size_t)row * p.lda + k0 + kk;
        st.v[it][0] = ld_f4(src);
        st.v[it][1] = ld_f4(src + 4);
    }
}

// PL: activation planes (2: hi + lo, 1: bf16 rounding only); FRP fragments
// per step and m-tile in LDS
template <int WT, int PL> struct Planes {
    static constexpr int FRP = (WT == WT_F32 || PL == 2) ? WCfg<WT>::FR : WCfg<WT>::FR / 2;
};

template <int WT, int MT, int NSTEP, int PL>
__device__ __forceinline__ void put_a(u32x4 *lds, const AStage<WT, MT, NSTEP> &st, const GemmArgs &p, int m0, int kvalid) {
    using S = AStage<WT, MT, NSTEP>;
#pragma unroll
    for (int it = 0; it < S::IT; ++it) {
        const int idx = (int)threadIdx.x + 256 * it;
        if (idx >= S::TOTAL) break;
        const int rowl = idx / S::GROUPS, j = idx - rowl * S::GROUPS;   // row in item, 8-float group
        const bool ok = m0 + rowl < p.M && 8 * j < kvalid;
        const float4 a = st.v[it][0], b = st.v[it][1];
        float x[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
        for (int i = 0; i < 8; ++i) x[i] = ok ? x[i] : 0.f;
        const int mt = rowl >> 4, r16 = rowl & 15;
        if constexpr (WT == WT_F32) {
            // step s covers 16 K: lane group g holds K 4g..4g+3 -> two fragments per 8 floats
            const int s = j >> 1, g0 = (j & 1) * 2;
            u32x4 f0 = {__float_as_uint(x[0]), __float_as_uint(x[1]), __float_as_uint(x[2]), __float_as_uint(x[3])};
            u32x4 f1 = {__float_as_uint(x[4]), __float_as_uint(x[5]), __float_as_uint(x[6]), __float_as_uint(x[7])};
            lds[(mt * NSTEP + s) * 64 + g0 * 16 + r16] = f0;
            lds[(mt * NSTEP + s) * 64 + (g0 + 1) * 16 + r16] = f1;
        } else {
            int s, f, g;
            if constexpr (WT == WT_BF16) { s = j >> 2; g = j & 3; f = 0; }
            else { s = j >> 3; const int jj = j & 7; g = jj >> 1; f = (jj & 1) * 2; }  // fp8: lane group g holds 16 K
            const int lane = g * 16 + r16;
            if constexpr (PL == 1) {
                lds[((mt * NSTEP + s) * Planes<WT, PL>::FRP + f / 2) * 64 + lane] = __builtin_bit_cast(u32x4, to_bf16x8(x));
            } else {
                bf16x8 hi, lo;
                split_bf16x8(x, hi, lo);
                lds[((mt * NSTEP + s) * WCfg<WT>::FR + f) * 64 + lane] = __builtin_bit_cast(u32x4, hi);
                lds[((mt * NSTEP + s) * WCfg<WT>::FR + f + 1) * 64 + lane] = __builtin_bit_cast(u32x4, lo);
            }
        }
    }
}

template <int WT, int PL>
__device__ __forceinline__ void mac_step(f32x4 &acc, const u32x4 &wv, const u32x4 *af) {
    if constexpr (WT == WT_BF16) {
        const bf16x8 b = __builtin_bit_cast(bf16x8, wv);
        acc = mfma_bf16(__builtin_bit_cast(bf16x8, af[0]), b, acc);
        if constexpr (PL == 2) acc = mfma_bf16(__builtin_bit_cast(bf16x8, af[64]), b, acc);
    } else if constexpr (WT == WT_FP8) {
        const bf16x8 b0 = fp8x8_to_bf16x8(wv.x, wv.y), b1 = fp8x8_to_bf16x8(wv.z, wv.w);
        if constexpr (PL == 2) {
            acc = mfma_bf16(__builtin_bit_cast(bf16x8, af[0]), b0, acc);
            acc = mfma_bf16(__builtin_bit_cast(bf16x8, af[64]), b0, acc);
            acc = mfma_bf16(__builtin_bit_cast(bf16x8, af[128]), b1, acc);
            acc = mfma_bf16(__builtin_bit_cast(bf16x8, af[192]), b1, acc);
        } else {
            acc = mfma_bf16(__builtin_bit_cast(bf16x8, af[0]), b0, acc);
            acc = mfma_bf16(__builtin_bit_cast(bf16x8, af[64]), b1, acc);
        }
    } else {
        const u32x4 a = af[0];
        acc = mfma_f32(__uint_as_float(a.x), __uint_as_float(wv.x), acc);
        acc = mfma_f32(__uint_as_float(a.y), __uint_as_float(wv.y), acc);
        acc = mfma_f32(__uint_as_float(a.z), __uint_as_float(wv.z), acc);
        acc = mfma_f32(__uint_as_float(a.w), __uint_as_float(wv.w), acc);
    }
}

template <int WT, int MT, int EPI, int NSTEP, int PL>
__global__ __launch_bounds__(256) void gemm_kernel(GemmArgs p) {
    constexpr int KS = WCfg<WT>::KS, ES = WCfg<WT>::ES, FR = Planes<WT, PL>::FRP;
    constexpr int NACC = (EPI == EPI_SWIGLU) ? 2 : 1;
    constexpr int KCH = NSTEP * KS;                      // K per staged chunk
    __shared__ u32x4 lds[2][MT * NSTEP * FR * 64];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 4, r16 = lane & 15;
    const int group = blockIdx.x / p.ksplit, split = blockIdx.x - group * p.ksplit;
    const int mgroup = blockIdx.y;
    const int m0 = mgroup * MT * 16;
    const int n0 = group * 64 + wave * 16;               // this wave's first output column

    // weight segment of this column group (groups never straddle segments)
    const char *wbase[NACC];
    const float *wscale[NACC];
    int ncol = n0;                                       // column inside the segment
    if constexpr (EPI == EPI_SWIGLU) {
        wbase[0] = (const char *)p.seg[0].w; wscale[0] = p.seg[0].scale;
        wbase[1] = (const char *)p.seg[1].w; wscale[1] = p.seg[1].scale;
    } else {
        // walked with the group's first column, which is uniform over the
        // workgroup, so the segment table is read with scalar loads
        int gcol = group * 64, s = 0;
        while (s + 1 < p.nseg && gcol >= p.seg[s].n) { gcol -= p.seg[s].n; ++s; }
        ncol = gcol + wave * 16;
        wbase[0] = (const char *)p.seg[s].w; wscale[0] = p.seg[s].scale;
    }
    const size_t K = p.K;
    const int kbeg = split * p.kchunk;
    const int kend = min(kbeg + p.kchunk, p.K);

    f32x4 acc[MT][NACC];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int a = 0; a < NACC; ++a) acc[mt][a] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int lane_koff = g * (KS / 4);                  // this lane's K offset inside a step
    // The chunks of this split are software-pipelined: chunk c + 1's
    // activation and weight loads are issued before chunk c's MFMAs, into the
    // other of two register buffers (weights) and LDS buffers (activation
    // fragments).  One barrier per chunk: put_a of chunk c writes LDS buffer
    // c & 1, last read by the MFMAs of chunk c - 2, which every wave finished
    // before the barrier of chunk c - 1.
    AStage<WT, MT, NSTEP> ast;
    u32x4 wv[2][NSTEP][NACC];
    auto load_w = [&](u32x4 (&w)[NSTEP][NACC], int k0, int nst) {
#pragma unroll
        for (int a = 0; a < NACC; ++a) {
            const char *wr = wbase[a] + ((size_t)(ncol + r16) * K + k0 + lane_koff) * ES;
            // unconditional (steps past the chunk reload its last one), so the
            // compiler counts them and waits for the activations alone first
#pragma unroll
            for (int s = 0; s < NSTEP; ++s) w[s][a] = ld_stream16(wr + (size_t)min(s, nst - 1) * KS * ES);
        }
    };
    auto chunk = [&](auto bufc, int k0) -> bool {
        constexpr int B = decltype(bufc)::value;
        const int kvalid = min(KCH, kend - k0);           // a multiple of KS
        const int nst = kvalid / KS;
        put_a<WT, MT, NSTEP, PL>(lds[B], ast, p, m0, kvalid);
        const int k1 = k0 + KCH;
        const bool more = k1 < kend;
        if (more) {
            load_a<WT, MT, NSTEP>(ast, p, m0, k1, min(KCH, kend - k1));
            asm volatile("" ::: "memory");               // activation loads ahead of the weights'
            load_w(wv[B ^ 1], k1, min(KCH, kend - k1) / KS);
        }
        __syncthreads();
#pragma unroll
        for (int s = 0; s < NSTEP; ++s)
            if (s < nst)
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                const u32x4 *af = lds[B] + ((mt * NSTEP + s) * FR) * 64 + lane;
#pragma unroll
                for (int a = 0; a < NACC; ++a) mac_step<WT, PL>(acc[mt][a], wv[B][s][a], af);
            }
        return more;
    };
    if (kbeg < kend) {
        load_a<WT, MT, NSTEP>(ast, p, m0, kbeg, min(KCH, kend - kbeg));
        asm volatile("" ::: "memory");
        load_w(wv[0], kbeg, min(KCH, kend - kbeg) / KS);
        for (int k0 = kbeg;; k0 += 2 * KCH) {
            if (!chunk(std::integral_constant<int, 0>{}, k0)) break;
            if (!chunk(std::integral_constant<int, 1>{}, k0 + KCH)) break;
        }
    }

    // ---- split-K: the last workgroup of the column group reduces in split order ----
    // partial layout per (item, split): [mt][a][wave][256]
    constexpr int PER = MT * NACC * 4 * 256;
    if (p.ksplit > 1) {
        const int item = mgroup * p.ngroups + group;
        float *part = p.part + (size_t)item * p.ksplit * PER;
        float *mine = part + (size_t)split * PER;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int a = 0; a < NACC; ++a)
                st_coherent16(mine, (uint32_t)((((mt * NACC + a) * 4 + wave) * 256 + lane * 4) * 4), acc[mt][a]);
        // every partial store must have completed before this workgroup is counted
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        __shared__ int is_last;
        if (tid == 0) {
            unsigned prev = __hip_atomic_fetch_add(p.cnt + item, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            is_last = (prev == (unsigned)(p.ksplit - 1));
        }
        __syncthreads();
        if (!is_last) return;
        // Sum the partials in split order.  All loads of a group of up to
        // MAXS splits are issued before the first add.
        constexpr int MAXS = 16;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int a = 0; a < NACC; ++a) {
                f32x4 v = f32x4{0.f, 0.f, 0.f, 0.f};
                const uint32_t q0 = (uint32_t)((((mt * NACC + a) * 4 + wave) * 256 + lane * 4) * 4);
                for (int s0 = 0; s0 < p.ksplit; s0 += MAXS) {
                    f32x4 pv[MAXS];
#pragma unroll
                    for (int s = 0; s < MAXS; ++s)
                        if (s0 + s < p.ksplit) pv[s] = ld_coherent16(part, q0 + (uint32_t)((s0 + s) * PER * 4));
#pragma unroll
                    for (int s = 0; s < MAXS; ++s)
                        if (s0 + s < p.ksplit) v += pv[s];
                }
                acc[mt][a] = v;
            }
        if (tid == 0) __hip_atomic_store(p.cnt + item, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }

    // ---- epilogue: lane holds rows 4g + j, column r16 of each 16x16 tile ----
    const int col = n0 + r16, ccol = ncol + r16;
    float sc[NACC];
#pragma unroll
    for (int a = 0; a < NACC; ++a) sc[a] = (WT == WT_FP8) ? wscale[a][ccol] : 1.f;
    float res[MT][4];
    if constexpr (EPI == EPI_ADD) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int row = m0 + mt * 16 + 4 * g + j;
                res[mt][j] = row < p.M ? p.Y[(size_t)row * p.ldy + col] : 0.f;
            }
    }
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int row = m0 + mt * 16 + 4 * g + j;
            if (row >= p.M) continue;
            float *y = p.Y + (size_t)row * p.ldy + col;
            if constexpr (EPI == EPI_SWIGLU) {
                *y = silu(acc[mt][0][j] * sc[0]) * (acc[mt][1][j] * sc[1]);
            } else if constexpr (EPI == EPI_ADD) {
                *y = res[mt][j] + acc[mt][0][j] * sc[0];
            } else {
                *y = acc[mt][0][j] * sc[0];
            }
        }
}

// ---------------------------------------------------------------------------
// host side: plan and launch
// ---------------------------------------------------------------------------
static int ks_of(int wt) { return wt == WT_BF16 ? 32 : wt == WT_FP8 ? 64 : 16; }

// steps per staged chunk for a given instantiation
static int nstep_of(int wt, int mt, int epi) {
    if (mt > 1) return wt == WT_FP8 ? 2 : 4;
    if (wt == WT_FP8) return epi == EPI_SWIGLU ? 2 : 4;
    return epi == EPI_SWIGLU ? 4 : 8;
}

int gemm_plan(GemmArgs &a) {
    const int nacc = a.epi == EPI_SWIGLU ? 2 : 1;
    int ncols = 0;
    if (a.epi == EPI_SWIGLU) ncols = a.seg[0].n;
    else for (int s = 0; s < a.nseg; ++s) ncols += a.seg[s].n;
    a.ngroups = ncols / 64;
    a.mt = a.M <= 16 ? 1 : a.M <= 32 ? 2 : 4;
    a.mgroups = (a.M + 16 * a.mt - 1) / (16 * a.mt);
    const int kch = nstep_of(a.wtype, a.mt, a.epi) * ks_of(a.wtype);
    const int nchunks = (a.K + kch - 1) / kch;
    const int base = a.ngroups * a.mgroups;
    // K split: the one that minimises (workgroups per CU, rounded up) x
    // (chunks per split + 2), the 2 standing for a split's first round trip
    // and its reduction; ties go to fewer workgroups.  With whole chunks per
    // split this lands on multiples of 256 workgroups where the shape allows.
    const size_t per = (size_t)a.mt * nacc * 4 * 256;
    int ksplit = 1;
    long long best = -1;
    for (int ks = 1; ks <= nchunks; ++ks) {
        const int cp = (nchunks + ks - 1) / ks, ks2 = (nchunks + cp - 1) / cp;
        if (ks2 != ks) continue;
        if (ks > 1 && ((size_t)base * ks * per > GEMM_PART_FLOATS || base > GEMM_MAX_COUNTERS)) break;
        const long long wg = (long long)base * ks, per_cu = (wg + GEMM_CUS - 1) / GEMM_CUS;
        const long long cost = per_cu * (cp + 2);
        if (best < 0 || cost < best) { best = cost; ksplit = ks; }
    }
    const int chunks_per = (nchunks + ksplit - 1) / ksplit;
    a.kchunk = chunks_per * kch;
    a.ksplit = (a.K + a.kchunk - 1) / a.kchunk;
    return base * a.ksplit;
}

template <int WT, int EPI, int PL>
static void launch_wt_epi_pl(const GemmArgs &a, hipStream_t s) {
    dim3 grid(a.ngroups * a.ksplit, a.mgroups), block(256);
    constexpr bool SW = EPI == EPI_SWIGLU;
    constexpr int N1 = WT == WT_FP8 ? (SW ? 2 : 4) : (SW ? 4 : 8);
    constexpr int N4 = WT == WT_FP8 ? 2 : 4;
    switch (a.mt) {
        case 1: hipLaunchKernelGGL((gemm_kernel<WT, 1, EPI, N1, PL>), grid, block, 0, s, a); break;
        case 2: hipLaunchKernelGGL((gemm_kernel<WT, 2, EPI, N4, PL>), grid, block, 0, s, a); break;
        default: hipLaunchKernelGGL((gemm_kernel<WT, 4, EPI, N4, PL>), grid, block, 0, s, a); break;
    }
}
template <int WT, int EPI>
static void launch_wt_epi(const GemmArgs &a, hipStream_t s) {
    if (WT != WT_F32 && a.planes == 1) launch_wt_epi_pl<WT, EPI, 1>(a, s);
    else launch_wt_epi_pl<WT, EPI, 2>(a, s);
}

template <int WT>
static void launch_wt(const GemmArgs &a, hipStream_t s) {
    switch (a.epi) {
        case EPI_STORE: launch_wt_epi<WT, EPI_STORE>(a, s); break;
        case EPI_ADD: launch_wt_epi<WT, EPI_ADD>(a, s); break;
        default: launch_wt_epi<WT, EPI_SWIGLU>(a, s); break;
    }
}

hipError_t gemm(GemmArgs a, float *part, unsigned *cnt, hipStream_t s) {
    if (a.M <= 0) return hipSuccess;
    if (gemm_tall_ok(a)) return gemm_tall(a, cnt, s);
    gemm_plan(a);
    a.part = part;
    a.cnt = cnt;
    switch (a.wtype) {
        case WT_BF16: launch_wt<WT_BF16>(a, s); break;
        case WT_FP8: launch_wt<WT_FP8>(a, s); break;
        default: launch_wt<WT_F32>(a, s); break;
    }
    return hipGetLastError();
}

}  // namespace dfl
