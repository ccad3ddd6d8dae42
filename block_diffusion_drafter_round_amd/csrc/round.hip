// Persistent forward_round kernel: one launch runs every layer of a drafting
// round ([DflashDraft] "forward_round": only the b block rows are projected
// per layer, block K/V land at cache rows [len, len + b), attention is full
// and non-causal over all len + b keys; [atlas dflash_head] overview:
// pre-norm Qwen3 layers, GQA).
//
// Launch shape: one workgroup of 8 waves per CU.  The work of each layer is
// a sequence of phases separated by grid barriers:
//   1 qkv GEMM     stream-K partials of X(*)g_in . [Wq;Wk;Wv]^T
//   2 qkv reduce   sum partials, times the input-norm scale 1/rms(X),
//                  q/k head RMSNorm, NeoX rope (f64 angles), times mscale;
//                  q -> Q, block k/v -> cache rows len + r
//   3 attention    (kv head, key split) items: online softmax, partial (m,l,O)
//   4 merge        combine the key splits -> O
//   5 o GEMM       stream-K partials of O . Wo^T
//   6 o reduce     X += sum of partials; per 128-column slice sum of squares
//   7 gate|up GEMM stream-K partials of X(*)g_post . [Wg;Wu]^T
//   8 SwiGLU       Z = silu(s*g) * (s*u), s = 1/rms(X)
//   9 down GEMM    stream-K partials of Z . Wd^T
//  10 down reduce  X += sum of partials; slice sums of squares
// and finally out = g_norm * X / rms(X).
//
// Each RMSNorm is split the same way.  The gain multiplies the GEMM input
// while it is staged.  The 1/rms row scale multiplies the GEMM output in the
// reduce phase.  The row sums of squares come from the phase that last wrote
// X.
//
// GEMMs (stream-K).  The (128-column group, K step) units of a GEMM are cut
// into equal contiguous ranges, one per workgroup.  Every workgroup thus
// streams the same number of weight bytes.  Wave w owns columns
// [16w, 16w + 16) of each group.  A range may span several groups; each
// group it touches yields one partial tile ("slot").  The reduce phase sums
// the slots of a group in workgroup order, so results do not depend on
// scheduling.
//
// Weight prefetch.  After a GEMM phase (after attention, for o_proj), each
// workgroup issues the loads of its range of the next GEMM into registers.
// These loads depend on no activation, so HBM keeps streaming through the
// following light phases and barriers.
//
// Coherence.  Data that one workgroup writes and another reads during the
// launch (partials, X, Q, O, Z, attention partials, the block K/V rows) is
// written with device-coherent stores and read with device-coherent loads
// (sc1).  No L2 writeback or invalidate is needed.  Weights and the
// committed cache rows are only read.
//
// Grid barrier.  Each workgroup bumps a counter for its XCD slot
// (blockIdx % 8).  The last arrival of a slot bumps a global counter.  The
// last global arrival publishes a new generation to one flag per slot, and
// the waiting workgroups poll the flag of their own slot.  The counters are
// never reset: after g barriers over the workspace's lifetime a slot counter
// holds g * (workgroups in the slot) and the global one g * (slots), mod 2^32,
// so each arrival learns from the returned value whether it is the last.
// The spin is bounded: on expiry the kernel sets an error word and every
// workgroup exits.
#include "common.h"
#include "round.h"

namespace dfl {

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------------------
// device-coherent memory ops (sc1)
// ---------------------------------------------------------------------------
// Vector loads go through buffer instructions with the sc1 cache policy, so
// the compiler tracks them and inserts the waits before their uses.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t cbuf(const void *base) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, 0x7fffffff, 0x00020000);
}
constexpr int CPOL_SC1 = 16;
__device__ __forceinline__ u32x4 ldc4(const void *base, uint32_t byte_off) {
    return __builtin_amdgcn_raw_buffer_load_b128(cbuf(base), byte_off, 0, CPOL_SC1);
}
__device__ __forceinline__ u32x2 ldc2(const void *base, uint32_t byte_off) {
    return __builtin_amdgcn_raw_buffer_load_b64(cbuf(base), byte_off, 0, CPOL_SC1);
}
__device__ __forceinline__ void stc4(void *base, uint32_t byte_off, u32x4 v) {
    __builtin_amdgcn_raw_buffer_store_b128(v, cbuf(base), byte_off, 0, CPOL_SC1);
}
__device__ __forceinline__ void stc2f(float *base, size_t elem, float x0, float x1) {
    const u32x2 v = {__float_as_uint(x0), __float_as_uint(x1)};
    __builtin_amdgcn_raw_buffer_store_b64(v, cbuf(base), (uint32_t)(elem * 4), 0, CPOL_SC1);
}
__device__ __forceinline__ void vm_wait() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
__device__ __forceinline__ float ldc(const float *p) {
    return __hip_atomic_load(const_cast<float *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void stc(float *p, float v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void stc_u16(uint16_t *p, uint16_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ unsigned ldc_u(unsigned *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void stc_u(unsigned *p, unsigned v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ unsigned add_u(unsigned *p, unsigned v) {
    return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float f_of(uint32_t u) { return __uint_as_float(u); }

// the kernel's own arguments, read in place (address space 4: scalar loads)
typedef const __attribute__((address_space(4))) RoundArgs KArgs;
typedef const __attribute__((address_space(4))) double KDouble;
__device__ __forceinline__ KArgs *kargs() { return (KArgs *)__builtin_amdgcn_kernarg_segment_ptr(); }

// A copy of the launch scalars, reloaded per phase through an opaque pointer
// so that the compiler cannot keep them alive across phases.
template <class T>
__device__ __forceinline__ T *opaque(T *p) {
    asm volatile("" : "+s"(p));
    return p;
}
__device__ __forceinline__ RoundScalars kscalars() {
    static_assert(sizeof(RoundScalars) % 4 == 0, "word copy");
    constexpr int NW = sizeof(RoundScalars) / 4;
    const __attribute__((address_space(4))) uint32_t *src =
        (const __attribute__((address_space(4))) uint32_t *)opaque(kargs());
    uint32_t w[NW];
#pragma unroll
    for (int i = 0; i < NW; ++i) w[i] = src[i];
    RoundScalars r;
    __builtin_memcpy(&r, w, sizeof r);
    return r;
}

typedef const __attribute__((address_space(4))) MatRef KMat;
__device__ __forceinline__ MatRef kmat(KMat &m) { return MatRef{m.w, m.s, m.n, 0}; }
__device__ __forceinline__ LayerRefs klayer(int l) {
    KArgs *ka = opaque(kargs());
    LayerRefs L;
    L.q = kmat(ka->L[l].q); L.k = kmat(ka->L[l].k); L.v = kmat(ka->L[l].v); L.o = kmat(ka->L[l].o);
    L.g = kmat(ka->L[l].g); L.u = kmat(ka->L[l].u); L.d = kmat(ka->L[l].d);
    L.g_in = ka->L[l].g_in; L.g_post = ka->L[l].g_post; L.g_q = ka->L[l].g_q; L.g_k = ka->L[l].g_k;
    L.aw = kmat(ka->L[l].aw); L.mw = kmat(ka->L[l].mw); L.abase = ka->L[l].abase; L.mbase = ka->L[l].mbase;
    return L;
}

// ---------------------------------------------------------------------------
// grid barrier
// ---------------------------------------------------------------------------
// Returns false if the barrier timed out; the caller then leaves the kernel.
__device__ __forceinline__ bool grid_sync(unsigned *st, unsigned &gen) {
    __shared__ int ok;
    vm_wait();                                  // this workgroup's coherent stores are complete
    __syncthreads();
    if (threadIdx.x == 0) {
        const unsigned nwg = gridDim.x;
        const unsigned nx = nwg < 8 ? nwg : 8;
        const unsigned x = blockIdx.x & 7;
        const unsigned per_x = (nwg - x + 7) / 8;
        const unsigned target = gen + 1;
        unsigned *xc = st + BAR_XCNT + x * 32, *gc = st + BAR_GCNT, *gf = st + BAR_GEN + x * 32;
        const unsigned prev = add_u(xc, 1u);
        if (prev + 1 == target * per_x) {
            const unsigned g = add_u(gc, 1u);
            if (g + 1 == target * nx)
                for (unsigned k = 0; k < nx; ++k) stc_u(st + BAR_GEN + k * 32, target);
        }
        int spins = 0, good = 1;
        while (ldc_u(gf) != target) {
            if (++spins > (1 << 22) || ldc_u(st + BAR_ERR) != 0) {
                good = 0;
                stc_u(st + BAR_ERR, 1u);
                break;
            }
            __builtin_amdgcn_s_sleep(1);
        }
        ok = good;
    }
    __syncthreads();
    gen += 1;
    return ok != 0;
}

// Phase trace: workgroup 0 stamps the 100 MHz wall clock after each barrier.
__device__ __forceinline__ void trace_mark(unsigned long long *tr, int &k) {
    if (tr && blockIdx.x == 0 && threadIdx.x == 0 && k < RND_TRACE_WORDS) tr[k] = wall_clock64();
    ++k;
}

// ---------------------------------------------------------------------------
// stream-K GEMM phase
// ---------------------------------------------------------------------------
template <int WT> struct KT;
// KS: K per unit (one 16-byte weight load per lane); FR: 16-byte activation
// fragments per unit; LDS holds 32 fragment units of 1 KiB.
template <int WT> struct KT;
template <> struct KT<WT_BF16> { static constexpr int KS = 32, ES = 2, FR = 2; };
template <> struct KT<WT_FP8>  { static constexpr int KS = 64, ES = 1, FR = 4; };
template <> struct KT<WT_F32>  { static constexpr int KS = 16, ES = 4, FR = 1; };
// units per chunk: 16 prefetch registers (u32x4) per lane, 32 KiB of LDS
template <int WT, bool DUAL>
constexpr int maxu() { return (DUAL ? 8 : 16) < 32 / KT<WT>::FR ? (DUAL ? 8 : 16) : 32 / KT<WT>::FR; }

struct Prefetch {
    u32x4 w[16];
};

struct GemmIO {
    GemmPlanDev p;
    MatRef s0, s1, s2;       // segments side by side (DUAL: s0 gate, s1 up); unused ones have n = 0
    const float *A;          // [rows][K], read coherently
    const float *gain;       // [K] multiplies A while staging, or nullptr
    int rows;
    float *part;             // partial slots [NWG][MAXSLOT][16][PW]
    // DFlash2 prepare conv applied while staging (G > 0, K = hidden): the
    // staged row r is (base[c,0] + D[r,g(c),0]) xn[r-1] + (base[c,1] + D[r,g(c),1]) xn[r]
    // with xn[r] = A[r] * gain * rinv[r] and xn[-1] = 0.
    int G;
    const float *cD;         // coefficients [16][4G], half 0 used here
    const float *cbase;      // static taps [2][K][2], half 0 used here
    const float *crinv;      // [16]
};

__device__ __forceinline__ void unit_range(const GemmPlanDev &p, int &u0, int &n) {
    u0 = blockIdx.x * p.upw;
    const int u1 = min(u0 + p.upw, p.total);
    n = max(0, u1 - u0);
}

// Issue the weight loads of units [u0, u0 + n) (n <= MAXU) for this wave's 16 columns.
template <int WT, bool DUAL>
__device__ __forceinline__ void gemm_issue(const GemmIO &io, int u0, int n, Prefetch &pf) {
    constexpr int KS = KT<WT>::KS, ES = KT<WT>::ES, MAXU = maxu<WT, DUAL>();
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int g = lane >> 4, r16 = lane & 15;
#pragma unroll
    for (int i = 0; i < MAXU; ++i) {
        if (i < n) {
            const int unit = u0 + i;
            const int grp = unit / io.p.steps, st = unit - grp * io.p.steps;
            int col = grp * 128 + wave * 16 + r16;
            const size_t koff = ((size_t)st * KS + g * (KS / 4)) * ES;
            if constexpr (DUAL) {
                pf.w[2 * i] = ld_stream16((const char *)io.s0.w + (size_t)col * io.p.K * ES + koff);
                pf.w[2 * i + 1] = ld_stream16((const char *)io.s1.w + (size_t)col * io.p.K * ES + koff);
            } else {
                const void *wb = io.s0.w;
                if (col >= io.s0.n) {
                    col -= io.s0.n;
                    wb = io.s1.w;
                    if (col >= io.s1.n) { col -= io.s1.n; wb = io.s2.w; }
                }
                pf.w[i] = ld_stream16((const char *)wb + (size_t)col * io.p.K * ES + koff);
            }
        }
    }
}

template <int WT, bool DUAL>
__device__ __forceinline__ void gemm_issue_first(const GemmIO &io, Prefetch &pf) {
    int u0, n;
    unit_range(io.p, u0, n);
    gemm_issue<WT, DUAL>(io, u0, min(n, maxu<WT, DUAL>()), pf);
}

// acc = W_frag . A_frag^T: the weights are the A operand (MFMA row = output
// column n), the activations the B operand (MFMA column = row m).  Lane
// (r16, g) then holds output columns 4g..4g+3 of row r16, contiguous in a
// row-major [m][n] tile.
template <int WT>
__device__ __forceinline__ void mac_unit(f32x4 &acc, const u32x4 &wv, const u32x4 *af) {
    if constexpr (WT == WT_BF16) {
        const bf16x8 b = __builtin_bit_cast(bf16x8, wv);
        acc = mfma_bf16(b, __builtin_bit_cast(bf16x8, af[0]), acc);
        acc = mfma_bf16(b, __builtin_bit_cast(bf16x8, af[64]), acc);
    } else if constexpr (WT == WT_FP8) {
        const bf16x8 b0 = fp8x8_to_bf16x8(wv.x, wv.y), b1 = fp8x8_to_bf16x8(wv.z, wv.w);
        acc = mfma_bf16(b0, __builtin_bit_cast(bf16x8, af[0]), acc);
        acc = mfma_bf16(b0, __builtin_bit_cast(bf16x8, af[64]), acc);
        acc = mfma_bf16(b1, __builtin_bit_cast(bf16x8, af[128]), acc);
        acc = mfma_bf16(b1, __builtin_bit_cast(bf16x8, af[192]), acc);
    } else {
        const u32x4 a = af[0];
        acc = mfma_f32(f_of(wv.x), f_of(a.x), acc);
        acc = mfma_f32(f_of(wv.y), f_of(a.y), acc);
        acc = mfma_f32(f_of(wv.z), f_of(a.z), acc);
        acc = mfma_f32(f_of(wv.w), f_of(a.w), acc);
    }
}

// Stage A[0..16)[K range of units u0 .. u0+n) (times the gain) into LDS
// fragments: fragment (unit i, f, lane) at lds[(i * FR + f) * 64 + lane].
// At most 2 groups of 8 floats per thread (n <= MAXU), loaded before use.
template <int WT>
__device__ __forceinline__ void stage_units(const GemmIO &io, int u0, int n, u32x4 *lds) {
    constexpr int KS = KT<WT>::KS, FR = KT<WT>::FR;
    constexpr int G8 = KS / 8;                          // 8-float groups per row and unit
    const int total = n * 16 * G8;                      // <= 2 * RND_THREADS
    u32x4 v[2][2], vp[2][2];
    int kk[2], ii[2], rr[2], jj[2];
    bool live[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        const int idx = threadIdx.x + t * RND_THREADS;
        live[t] = idx < total;
        const int i = idx / (16 * G8), rem = idx - i * 16 * G8;
        const int row = rem / G8, j = rem - row * G8;
        const int unit = u0 + i;
        const int st = unit - (unit / io.p.steps) * io.p.steps;
        ii[t] = i; rr[t] = row; jj[t] = j;
        kk[t] = st * KS + 8 * j;
        if (live[t] && row < io.rows) {
            const uint32_t off = (uint32_t)(((size_t)row * io.p.K + kk[t]) * 4);
            v[t][0] = ldc4(io.A, off);
            v[t][1] = ldc4(io.A, off + 16);
            if (io.G && row > 0) {
                vp[t][0] = ldc4(io.A, off - (uint32_t)io.p.K * 4);
                vp[t][1] = ldc4(io.A, off - (uint32_t)io.p.K * 4 + 16);
            }
        }
    }
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        if (!live[t]) continue;
        const int i = ii[t], row = rr[t], j = jj[t];
        float x[8];
        if (row < io.rows) {
            x[0] = f_of(v[t][0].x); x[1] = f_of(v[t][0].y); x[2] = f_of(v[t][0].z); x[3] = f_of(v[t][0].w);
            x[4] = f_of(v[t][1].x); x[5] = f_of(v[t][1].y); x[6] = f_of(v[t][1].z); x[7] = f_of(v[t][1].w);
            if (io.gain) {
                const float4 g0 = ld_f4(io.gain + kk[t]), g1 = ld_f4(io.gain + kk[t] + 4);
                x[0] *= g0.x; x[1] *= g0.y; x[2] *= g0.z; x[3] *= g0.w;
                x[4] *= g1.x; x[5] *= g1.y; x[6] *= g1.z; x[7] *= g1.w;
                if (io.G) {
                    // 8 consecutive channels share one group (K / G is a multiple of 8)
                    const int grp = kk[t] * io.G / io.p.K;
                    const float rr_ = ldc(io.crinv + row), rp = row > 0 ? ldc(io.crinv + row - 1) : 0.f;
                    const float d0 = ldc(io.cD + row * 4 * io.G + 2 * grp), d1 = ldc(io.cD + row * 4 * io.G + 2 * grp + 1);
                    float xp[8];
                    if (row > 0) {
                        xp[0] = f_of(vp[t][0].x); xp[1] = f_of(vp[t][0].y); xp[2] = f_of(vp[t][0].z); xp[3] = f_of(vp[t][0].w);
                        xp[4] = f_of(vp[t][1].x); xp[5] = f_of(vp[t][1].y); xp[6] = f_of(vp[t][1].z); xp[7] = f_of(vp[t][1].w);
                    } else {
#pragma unroll
                        for (int q = 0; q < 8; ++q) xp[q] = 0.f;
                    }
                    const float gq[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
#pragma unroll
                    for (int q = 0; q < 8; q += 2) {
                        const float4 b = ld_f4(io.cbase + (size_t)(kk[t] + q) * 2);   // taps of channels c, c+1
                        const float p0 = xp[q] * gq[q] * rp, p1 = xp[q + 1] * gq[q + 1] * rp;
                        x[q] = (b.x + d0) * p0 + (b.y + d1) * (x[q] * rr_);
                        x[q + 1] = (b.z + d0) * p1 + (b.w + d1) * (x[q + 1] * rr_);
                    }
                }
            }
        } else {
#pragma unroll
            for (int q = 0; q < 8; ++q) x[q] = 0.f;
        }
        if constexpr (WT == WT_F32) {
            const int g0 = 2 * j;   // lane groups 2j, 2j+1 hold K 8j..8j+3 and 8j+4..8j+7
            lds[i * 64 + g0 * 16 + row] = u32x4{__float_as_uint(x[0]), __float_as_uint(x[1]), __float_as_uint(x[2]), __float_as_uint(x[3])};
            lds[i * 64 + (g0 + 1) * 16 + row] = u32x4{__float_as_uint(x[4]), __float_as_uint(x[5]), __float_as_uint(x[6]), __float_as_uint(x[7])};
        } else {
            bf16x8 hi, lo;
            split_bf16x8(x, hi, lo);
            int g, f;
            if constexpr (WT == WT_BF16) { g = j; f = 0; }
            else { g = j >> 1; f = (j & 1) * 2; }       // fp8: lane group g holds 16 K
            const int ln = g * 16 + row;
            lds[(i * FR + f) * 64 + ln] = __builtin_bit_cast(u32x4, hi);
            lds[(i * FR + f + 1) * 64 + ln] = __builtin_bit_cast(u32x4, lo);
        }
    }
}

// Run this workgroup's stream-K range; pf holds the loads of its first MAXU units.
template <int WT, bool DUAL>
__device__ __forceinline__ void gemm_run(const GemmIO &io, Prefetch &pf, u32x4 *lds) {
    constexpr int MAXU = maxu<WT, DUAL>();
    constexpr int NM = DUAL ? 2 : 1;
    constexpr int PW = DUAL ? 256 : 128;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int g = lane >> 4, r16 = lane & 15;
    int u0, n;
    unit_range(io.p, u0, n);
    if (n <= 0) return;
    const int first_grp = u0 / io.p.steps;
    f32x4 acc[NM];
#pragma unroll
    for (int m = 0; m < NM; ++m) acc[m] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int c0 = 0; c0 < n; c0 += MAXU) {
        const int cn = min(MAXU, n - c0);
        if (c0 > 0) gemm_issue<WT, DUAL>(io, u0 + c0, cn, pf);
        __syncthreads();                                 // LDS free
        stage_units<WT>(io, u0 + c0, cn, lds);
        __syncthreads();
#pragma unroll
        for (int i = 0; i < MAXU; ++i) {
            if (i < cn) {
                const int unit = u0 + c0 + i;
                const u32x4 *af = lds + (i * KT<WT>::FR) * 64 + lane;
#pragma unroll
                for (int m = 0; m < NM; ++m) mac_unit<WT>(acc[m], pf.w[i * NM + m], af);
                const bool seg_end = (c0 + i == n - 1) || ((unit + 1) % io.p.steps == 0);
                if (seg_end) {
                    const int grp = unit / io.p.steps;
                    const size_t tile = (size_t)(blockIdx.x * MAXSLOT + (grp - first_grp)) * 16 * PW;
#pragma unroll
                    for (int m = 0; m < NM; ++m)
                        stc4(io.part, (uint32_t)((tile + (size_t)r16 * PW + m * 128 + wave * 16 + 4 * g) * 4),
                             __builtin_bit_cast(u32x4, acc[m]));
#pragma unroll
                    for (int m = 0; m < NM; ++m) acc[m] = f32x4{0.f, 0.f, 0.f, 0.f};
                }
            }
        }
    }
}

// Sum, in workgroup order, of the partial slots of group grp at (row, cols c, c+1).
__device__ __forceinline__ float2 sum_slots2(const GemmPlanDev &p, const float *part, int grp, int row, int c, int PW) {
    const int w0 = (grp * p.steps) / p.upw, w1 = ((grp + 1) * p.steps - 1) / p.upw;
    float2 s = make_float2(0.f, 0.f);
    for (int wb = w0; wb <= w1; wb += 8) {
        u32x2 v[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            const int w = wb + q;
            if (w <= w1) {
                const int slot = grp - (w * p.upw) / p.steps;
                v[q] = ldc2(part, (uint32_t)((((size_t)(w * MAXSLOT + slot) * 16 + row) * PW + c) * 4));
            }
        }
#pragma unroll
        for (int q = 0; q < 8; ++q)
            if (wb + q <= w1) { s.x += f_of(v[q].x); s.y += f_of(v[q].y); }
    }
    return s;
}

// 1/rms of row r of X from the slice sums of squares
__device__ __forceinline__ float inv_rms_row(const RoundScalars &a, int r) {
    const int lane = threadIdx.x & 63;
    const int ns = a.H / 128;
    float s = 0.f;
    for (int q = lane; q < ns; q += 64) s += ldc(a.ssq + q * 16 + r);
    s = wave_sum(s);
    return 1.f / sqrtf(s / (float)a.H + a.eps);
}

__device__ __forceinline__ float col_scale(const MatRef &m, int col) { return m.s ? m.s[col] : 1.f; }

// ---------------------------------------------------------------------------
// light phases (wave-level items)
// ---------------------------------------------------------------------------
__device__ __forceinline__ int gwave() { return blockIdx.x * (RND_THREADS / 64) + (threadIdx.x >> 6); }
__device__ __forceinline__ int nwaves() { return gridDim.x * (RND_THREADS / 64); }

// X = noise, slice sums of squares (first launch of a call)
__device__ __forceinline__ void init_phase(const RoundScalars &a) {
    const int lane = threadIdx.x & 63, ng = a.H / 128;
    for (int it = gwave(); it < ng * a.b; it += nwaves()) {
        const int grp = it % ng, r = it / ng, c = grp * 128 + 2 * lane;
        const float2 x = *reinterpret_cast<const float2 *>(a.noise + (size_t)r * a.H + c);
        stc2f(a.X, (size_t)r * a.H + c, x.x, x.y);
        const float ss = wave_sum(x.x * x.x + x.y * x.y);
        if (lane == 0) stc(a.ssq + grp * 16 + r, ss);
    }
}

// X += y (+ fp8 column scale); slice sums of squares.  y is the sum of the
// partials, or with a DFlash2 wrap (cD != nullptr) the finish conv of it:
// y'[r,c] = (base1[c,0] + D[r,1,g(c),0]) y[r-1,c] + (base1[c,1] + D[r,1,g(c),1]) y[r,c].
__device__ __forceinline__ void residual_phase(const RoundScalars &a, const GemmPlanDev &p, const MatRef &m,
                                               const float *cD = nullptr, const float *base1 = nullptr) {
    const int lane = threadIdx.x & 63, ng = a.H / 128;
    for (int it = gwave(); it < ng * a.b; it += nwaves()) {
        const int grp = it % ng, r = it / ng, cl = 2 * lane, c = grp * 128 + cl;
        float2 s = sum_slots2(p, a.part, grp, r, cl, 128);
        const u32x2 xo = ldc2(a.X, (uint32_t)(((size_t)r * a.H + c) * 4));
        float y0 = s.x * col_scale(m, c), y1 = s.y * col_scale(m, c + 1);
        if (cD) {
            float2 sp = make_float2(0.f, 0.f);
            if (r > 0) sp = sum_slots2(p, a.part, grp, r - 1, cl, 128);
            const float p0 = sp.x * col_scale(m, c), p1 = sp.y * col_scale(m, c + 1);
            const int gi = c * a.d2 / a.H;
            const float d0 = ldc(cD + r * 4 * a.d2 + 2 * (a.d2 + gi)), d1 = ldc(cD + r * 4 * a.d2 + 2 * (a.d2 + gi) + 1);
            const float4 bb = ld_f4(base1 + (size_t)c * 2);
            y0 = (bb.x + d0) * p0 + (bb.y + d1) * y0;
            y1 = (bb.z + d0) * p1 + (bb.w + d1) * y1;
        }
        const float x0 = f_of(xo.x) + y0, x1 = f_of(xo.y) + y1;
        stc2f(a.X, (size_t)r * a.H + c, x0, x1);
        const float ss = wave_sum(x0 * x0 + x1 * x1);
        if (lane == 0) stc(a.ssq + grp * 16 + r, ss);
    }
}

__device__ __forceinline__ float silu(float x) { return x / (1.f + __expf(-x)); }

// four consecutive weights of one row, widened to f32
template <int WT>
__device__ __forceinline__ float4 ld_w4(const void *w, size_t idx) {
    if constexpr (WT == WT_F32) {
        return ld_f4(reinterpret_cast<const float *>(w) + idx);
    } else if constexpr (WT == WT_BF16) {
        const uint2 u = *reinterpret_cast<const uint2 *>(reinterpret_cast<const uint16_t *>(w) + idx);
        return make_float4(__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xFFFF0000u),
                           __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xFFFF0000u));
    } else {
        const uint32_t u = *reinterpret_cast<const uint32_t *>(reinterpret_cast<const uint8_t *>(w) + idx);
        const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8(u, false), hi = __builtin_amdgcn_cvt_pk_f32_fp8(u, true);
        return make_float4(lo[0], lo[1], hi[0], hi[1]);
    }
}

// DFlash2 coefficients of a sublayer: D[r][j] = rinv[r] * s_j * sum_c X[r,c] g[c] W[j,c]
// (the projection of the normalised rows, j over [half][group][tap]), and
// rinv[r] = 1/rms(X[r]).  One wave per (row, 8 consecutive j).
template <int WT>
__device__ __forceinline__ void d2_phase(const RoundScalars &a, const MatRef &w, const float *gain, float *Dout) {
    const int lane = threadIdx.x & 63;
    const int nj = 4 * a.d2, njb = nj / 8;
    for (int it = gwave(); it < a.b * njb; it += nwaves()) {
        const int r = it / njb, j0 = (it - r * njb) * 8;
        float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        for (int c = lane * 4; c < a.H; c += 256) {
            const u32x4 xv = ldc4(a.X, (uint32_t)(((size_t)r * a.H + c) * 4));
            const float4 g = ld_f4(gain + c);
            const float x0 = f_of(xv.x) * g.x, x1 = f_of(xv.y) * g.y, x2 = f_of(xv.z) * g.z, x3 = f_of(xv.w) * g.w;
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                const float4 wv = ld_w4<WT>(w.w, (size_t)(j0 + q) * a.H + c);
                acc[q] += x0 * wv.x + x1 * wv.y + x2 * wv.z + x3 * wv.w;
            }
        }
        const float rs = inv_rms_row(a, r);
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            const float v = wave_sum(acc[q]);
            if (lane == q) stc(Dout + r * nj + j0 + q, v * rs * (w.s ? w.s[j0 + q] : 1.f));
        }
        if (j0 == 0 && lane == 0) stc(a.d2_rinv + r, rs);
    }
}

// Z = silu(s * gate) * (s * up), s = 1/rms(X) (the post-attention norm's row scale)
__device__ __forceinline__ void swiglu_phase(const RoundScalars &a, const LayerRefs &L) {
    const int lane = threadIdx.x & 63, ng = a.I / 128;
    for (int it = gwave(); it < ng * a.b; it += nwaves()) {
        const int grp = it % ng, r = it / ng, cl = 2 * lane, c = grp * 128 + cl;
        const float rs = a.d2 ? 1.f : inv_rms_row(a, r);      // the conv staging already normalised the rows
        const float2 gs = sum_slots2(a.p_gu, a.part, grp, r, cl, 256);
        const float2 us = sum_slots2(a.p_gu, a.part, grp, r, 128 + cl, 256);
        const float g0 = gs.x * rs * col_scale(L.g, c), g1 = gs.y * rs * col_scale(L.g, c + 1);
        const float u0 = us.x * rs * col_scale(L.u, c), u1 = us.y * rs * col_scale(L.u, c + 1);
        stc2f(a.Z, (size_t)r * a.I + c, silu(g0) * u0, silu(g1) * u1);
    }
}

// out = g_norm * X / rms(X)
__device__ __forceinline__ void final_phase(const RoundScalars &a) {
    const int lane = threadIdx.x & 63, ng = a.H / 128;
    for (int it = gwave(); it < ng * a.b; it += nwaves()) {
        const int grp = it % ng, r = it / ng, c = grp * 128 + 2 * lane;
        const float rs = inv_rms_row(a, r);
        const u32x2 x = ldc2(a.X, (uint32_t)(((size_t)r * a.H + c) * 4));
        const float2 gg = *reinterpret_cast<const float2 *>(a.g_norm + c);
        *reinterpret_cast<float2 *>(a.out + (size_t)r * a.H + c) = make_float2(gg.x * (f_of(x.x) * rs), gg.y * (f_of(x.y) * rs));
    }
}

// qkv reduce: input-norm row scale, q/k head RMSNorm + rope (+ mscale), stores.
// The per-matrix pointers come in as separate values: selecting among members
// of a layer struct at run time would put the struct in scratch memory.
template <bool KVF32, int D>
__device__ __forceinline__ void qkv_phase(const RoundScalars &a, const float *sq, const float *sk, const float *sv,
                                          const float *g_q, const float *g_k, KDouble *inv_freq, char *kc, char *vc) {
    constexpr int HALF = D / 2;
    const int lane = threadIdx.x & 63;
    const int nh = a.nq + 2 * a.nkv;
    const bool act = lane < HALF;
    const int j = act ? lane : 0;
    for (int it = gwave(); it < nh * a.b; it += nwaves()) {
        const int h = it % nh, r = it / nh;
        const int kind = h < a.nq ? 0 : h < a.nq + a.nkv ? 1 : 2;        // q / k / v
        const int hh = kind == 0 ? h : kind == 1 ? h - a.nq : h - a.nq - a.nkv;
        const int col0 = kind == 0 ? hh * D : kind == 1 ? a.qd + hh * D : a.qd + a.kvd + hh * D;
        const int grp = col0 / 128, cin = col0 % 128;
        const float rs = a.d2 ? 1.f : inv_rms_row(a, r);      // the conv staging already normalised the rows
        // partials for columns (j, j + HALF) of the head
        const int w0 = (grp * a.p_qkv.steps) / a.p_qkv.upw, w1 = ((grp + 1) * a.p_qkv.steps - 1) / a.p_qkv.upw;
        float x0 = 0.f, x1 = 0.f;
        for (int wb = w0; wb <= w1; wb += 8) {
            float v0[8], v1[8];
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                const int w = wb + q;
                if (w <= w1) {
                    const int slot = grp - (w * a.p_qkv.upw) / a.p_qkv.steps;
                    const float *src = a.part + ((size_t)(w * MAXSLOT + slot) * 16 + r) * 128 + cin;
                    v0[q] = ldc(src + j);
                    v1[q] = ldc(src + j + HALF);
                }
            }
#pragma unroll
            for (int q = 0; q < 8; ++q)
                if (wb + q <= w1) { x0 += v0[q]; x1 += v1[q]; }
        }
        const float *msc = kind == 0 ? sq : kind == 1 ? sk : sv;   // fp8 row scales, or null
        x0 *= rs * (msc ? msc[hh * D + j] : 1.f);
        x1 *= rs * (msc ? msc[hh * D + j + HALF] : 1.f);
        if (!act) { x0 = 0.f; x1 = 0.f; }
        const size_t crow = (size_t)(a.len + r);
        if (kind == 2) {
            if (act) {
                const size_t i0 = ((size_t)hh * D + j) * a.cap + crow, i1 = ((size_t)hh * D + j + HALF) * a.cap + crow;
                if constexpr (KVF32) {
                    stc(reinterpret_cast<float *>(vc) + i0, x0);
                    stc(reinterpret_cast<float *>(vc) + i1, x1);
                } else {
                    stc_u16(reinterpret_cast<uint16_t *>(vc) + i0, (uint16_t)f32_to_bf16_bits(x0));
                    stc_u16(reinterpret_cast<uint16_t *>(vc) + i1, (uint16_t)f32_to_bf16_bits(x1));
                }
            }
            continue;
        }
        const float ss = wave_sum(x0 * x0 + x1 * x1);
        const float inv = 1.f / sqrtf(ss / (float)D + a.eps);
        const float *gain = kind == 0 ? g_q : g_k;
        if (act) {
            const float y0 = gain[j] * (x0 * inv), y1 = gain[j + HALF] * (x1 * inv);
            double sv, cv;
            sincos((double)a.pos[r] * inv_freq[j], &sv, &cv);
            const float c = (float)cv, s = (float)sv;
            const float o0 = (y0 * c - y1 * s) * a.mscale, o1 = (y1 * c + y0 * s) * a.mscale;
            if (kind == 0) {
                float *q = a.Q + ((size_t)r * a.nq + hh) * D;
                stc(q + j, o0);
                stc(q + j + HALF, o1);
            } else {
                const size_t base = ((size_t)hh * a.cap + crow) * D;
                if constexpr (KVF32) {
                    stc(reinterpret_cast<float *>(kc) + base + j, o0);
                    stc(reinterpret_cast<float *>(kc) + base + j + HALF, o1);
                } else {
                    stc_u16(reinterpret_cast<uint16_t *>(kc) + base + j, (uint16_t)f32_to_bf16_bits(o0));
                    stc_u16(reinterpret_cast<uint16_t *>(kc) + base + j + HALF, (uint16_t)f32_to_bf16_bits(o1));
                }
            }
        }
    }
}

// ---------------------------------------------------------------------------
// attention: item (kv head h, key split s); wave w takes query tiles w, w + 8.
// The workgroup stages K and V^T of each 32-key block in LDS (one
// device-coherent 16-byte load per thread and tensor, double-buffered), and
// all waves read their MFMA fragments from there.
// S^T = K.Q^T puts one query per lane (l % 16) and keys 8g..8g+7 per lane
// group; O^T = V^T.P^T keeps the same query per lane, so the online softmax
// is lane-local apart from the 4-group row max / sum.
// ---------------------------------------------------------------------------
template <bool F32, int D>
struct AttnLds {
    static constexpr int ES = F32 ? 4 : 2;
    static constexpr int KC = D * ES / 16;          // 16-byte chunks per key row
    static constexpr int VC = 32 * ES / 16;         // 16-byte chunks per V^T row of a block
    static constexpr int KW = KC + 1, VW = VC + 1;  // padded row widths
    static constexpr int STAGE = 32 * KW + D * VW;  // u32x4 per staged block
};

template <bool F32, int D>
__device__ __forceinline__ void attn_phase(const RoundScalars &a, const char *kc, const char *vc, u32x4 *lds) {
    using AL = AttnLds<F32, D>;
    constexpr int ES = AL::ES, KC = AL::KC, VC = AL::VC, KW = AL::KW, VW = AL::VW;
    constexpr int NDS = F32 ? D / 16 : D / 32;       // MFMA d-steps per score tile
    constexpr int NDT = D / 16;                      // output d-tiles
    constexpr int TQ = 1;                            // query tiles per wave and pass
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 4, r16 = lane & 15;
    const int G = a.nq / a.nkv, nqh = a.b * G, qtiles = a.qpad / 16;
    const int n_keys = a.len + a.b;
    const int items = a.nkv * a.attn_nsplit;
    const int npass = (qtiles + 7) / 8;              // more than 8 query tiles: a second pass over the keys
    for (int item = blockIdx.x; item < items * npass; item += gridDim.x) {
        const int pass = item / items, it0 = item - pass * items;
        const int h = it0 / a.attn_nsplit, split = it0 - h * a.attn_nsplit;
        const int kbeg = split * a.attn_kps, kend = min(kbeg + a.attn_kps, n_keys);
        const int nblk = (kend - kbeg + 31) / 32;
        // this thread's share of a staged block: one K chunk and one V^T chunk
        const bool kact = tid < 32 * KC, vact = tid < D * VC;
        const int kkey = tid / KC, kcol = tid - kkey * KC;
        const int vrow = tid / VC, vcol = tid - vrow * VC;
        auto kof = [&](int k0) { return (uint32_t)((((size_t)h * a.cap + k0 + kkey) * D) * ES + kcol * 16); };
        auto vof = [&](int k0) { return (uint32_t)((((size_t)h * D + vrow) * a.cap + k0) * ES + vcol * 16); };
        u32x4 kr = {0, 0, 0, 0}, vr = {0, 0, 0, 0};
        if (kact) kr = ldc4(kc, kof(kbeg));
        if (vact) vr = ldc4(vc, vof(kbeg));
        __syncthreads();                            // LDS free (previous phase / item)
        if (kact) lds[kkey * KW + kcol] = kr;
        if (vact) lds[32 * KW + vrow * VW + vcol] = vr;

        // query fragments (B operand of S^T) and running state per query tile
        bf16x8 qb[TQ][F32 ? 1 : NDS];
        float4 qf[TQ][F32 ? NDS : 1];
        float m_run[TQ], l_run[TQ];
        f32x4 o[TQ][NDT];
#pragma unroll
        for (int tq = 0; tq < TQ; ++tq) {
            const int qt = wave + 8 * (tq + pass);
            const int qi = qt * 16 + r16;
            const bool qvalid = qt < qtiles && qi < nqh;
            const uint32_t qoff = (uint32_t)(((size_t)(qvalid ? qi / G : 0) * a.nq + h * G + (qvalid ? qi % G : 0)) * D * 4);
#pragma unroll
            for (int s = 0; s < NDS; ++s) {
                if constexpr (!F32) {
                    const u32x4 p0 = ldc4(a.Q, qoff + (32 * s + 8 * g) * 4), p1 = ldc4(a.Q, qoff + (32 * s + 8 * g + 4) * 4);
                    float x[8] = {f_of(p0.x), f_of(p0.y), f_of(p0.z), f_of(p0.w), f_of(p1.x), f_of(p1.y), f_of(p1.z), f_of(p1.w)};
                    if (!qvalid)
#pragma unroll
                        for (int q = 0; q < 8; ++q) x[q] = 0.f;
                    qb[tq][s] = to_bf16x8(x);
                } else {
                    const u32x4 p0 = ldc4(a.Q, qoff + (16 * s + 4 * g) * 4);
                    qf[tq][s] = qvalid ? make_float4(f_of(p0.x), f_of(p0.y), f_of(p0.z), f_of(p0.w)) : make_float4(0, 0, 0, 0);
                }
            }
            m_run[tq] = -1e30f;
            l_run[tq] = 0.f;
#pragma unroll
            for (int t = 0; t < NDT; ++t) o[tq][t] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
        __syncthreads();

        for (int bi = 0; bi < nblk; ++bi) {
            const int k0 = kbeg + 32 * bi;
            const u32x4 *Kl = lds + (bi & 1) * AL::STAGE;
            const u32x4 *Vl = Kl + 32 * KW;
            // next block's loads overlap this block's math
            if (bi + 1 < nblk) {
                if (kact) kr = ldc4(kc, kof(k0 + 32));
                if (vact) vr = ldc4(vc, vof(k0 + 32));
            }
            const bool full = k0 + 32 <= kend;
#pragma unroll
            for (int tq = 0; tq < TQ; ++tq) {
                if (wave + 8 * (tq + pass) >= qtiles) continue;
                f32x4 st[2];
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    st[t] = f32x4{0.f, 0.f, 0.f, 0.f};
                    const int key = 8 * (r16 >> 2) + 4 * t + (r16 & 3);     // MFMA row r16 of tile t
#pragma unroll
                    for (int s = 0; s < NDS; ++s) {
                        const u32x4 kf = Kl[key * KW + 4 * s + g];
                        if constexpr (!F32) {
                            st[t] = mfma_bf16(__builtin_bit_cast(bf16x8, kf), qb[tq][s], st[t]);
                        } else {
                            st[t] = mfma_f32(f_of(kf.x), qf[tq][s].x, st[t]);
                            st[t] = mfma_f32(f_of(kf.y), qf[tq][s].y, st[t]);
                            st[t] = mfma_f32(f_of(kf.z), qf[tq][s].z, st[t]);
                            st[t] = mfma_f32(f_of(kf.w), qf[tq][s].w, st[t]);
                        }
                    }
                }
                // lane (query r16, group g) holds keys k0 + 8g + 4t + j
                float sc[8];
                float bmax = -INFINITY;
#pragma unroll
                for (int t = 0; t < 2; ++t)
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj) {
                        float v = st[t][jj] * a.scale_log2;
                        v = k0 + 8 * g + 4 * t + jj < kend ? v : -INFINITY;
                        sc[4 * t + jj] = v;
                        bmax = fmaxf(bmax, v);
                    }
                bmax = group4_max(bmax);
                const float m_new = fmaxf(m_run[tq], bmax);
                const float corr = __builtin_amdgcn_exp2f(m_run[tq] - m_new);
                float psum = 0.f;
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    sc[i] = __builtin_amdgcn_exp2f(sc[i] - m_new);
                    psum += sc[i];
                }
                psum = group4_sum(psum);
                l_run[tq] = l_run[tq] * corr + psum;
                m_run[tq] = m_new;
#pragma unroll
                for (int t = 0; t < NDT; ++t) o[tq][t] *= corr;
                if constexpr (!F32) {
                    const bf16x8 pb = to_bf16x8(sc);
#pragma unroll
                    for (int t = 0; t < NDT; ++t) {
                        u32x4 vv = Vl[(16 * t + r16) * VW + g];
                        if (!full) {
#pragma unroll
                            for (int w = 0; w < 4; ++w) {
                                const int kk = k0 + 8 * g + 2 * w;
                                const uint32_t msk = (kk < kend ? 0x0000FFFFu : 0u) | (kk + 1 < kend ? 0xFFFF0000u : 0u);
                                vv[w] &= msk;
                            }
                        }
                        o[tq][t] = mfma_bf16(__builtin_bit_cast(bf16x8, vv), pb, o[tq][t]);
                    }
                } else {
#pragma unroll
                    for (int t = 0; t < NDT; ++t) {
                        const u32x4 v0 = Vl[(16 * t + r16) * VW + 2 * g], v1 = Vl[(16 * t + r16) * VW + 2 * g + 1];
                        float vk[8] = {f_of(v0.x), f_of(v0.y), f_of(v0.z), f_of(v0.w), f_of(v1.x), f_of(v1.y), f_of(v1.z), f_of(v1.w)};
#pragma unroll
                        for (int i = 0; i < 8; ++i) {
                            if (!full && k0 + 8 * g + i >= kend) vk[i] = 0.f;
                            o[tq][t] = mfma_f32(vk[i], sc[i], o[tq][t]);
                        }
                    }
                }
            }
            if (bi + 1 < nblk) {
                u32x4 *Kn = lds + ((bi + 1) & 1) * AL::STAGE;
                if (kact) Kn[kkey * KW + kcol] = kr;
                if (vact) Kn[32 * KW + vrow * VW + vcol] = vr;
            }
            __syncthreads();
        }
        // partials: lane holds O^T[d = 16t + 4g + j][query r16]
#pragma unroll
        for (int tq = 0; tq < TQ; ++tq) {
            const int qt = wave + 8 * (tq + pass);
            if (qt >= qtiles) continue;
            const size_t pq = ((size_t)h * a.attn_nsplit + split) * a.qpad + qt * 16 + r16;
            if (g == 0) {
                stc(a.attn_ml + pq * 2 + 0, m_run[tq]);
                stc(a.attn_ml + pq * 2 + 1, l_run[tq]);
            }
#pragma unroll
            for (int t = 0; t < NDT; ++t)
                stc4(a.attn_o, (uint32_t)((pq * D + 16 * t + 4 * g) * 4), __builtin_bit_cast(u32x4, o[tq][t]));
        }
    }
}

// merge the key splits of (kv head, query): O = sum_s 2^(m_s-M) O_s / sum_s 2^(m_s-M) l_s
template <int D>
__device__ __forceinline__ void merge_phase(const RoundScalars &a) {
    const int lane = threadIdx.x & 63;
    const int G = a.nq / a.nkv, nqh = a.b * G, ns = a.attn_nsplit;
    for (int it = gwave(); it < a.nkv * nqh; it += nwaves()) {
        const int h = it / nqh, qi = it - h * nqh;
        const size_t base = (size_t)h * ns * a.qpad + qi;
        float m = -1e30f, l = 0.f;
        if (lane < ns) {
            m = ldc(a.attn_ml + (base + (size_t)lane * a.qpad) * 2);
            l = ldc(a.attn_ml + (base + (size_t)lane * a.qpad) * 2 + 1);
        }
        float M = m;
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) M = fmaxf(M, __shfl_xor(M, o, 64));
        const float w = lane < ns ? __builtin_amdgcn_exp2f(m - M) : 0.f;
        const float L = wave_sum(w * l);
        float acc0 = 0.f, acc1 = 0.f;
        constexpr int MB = 16;
        for (int sb = 0; sb < ns; sb += MB) {
            float v0[MB], v1[MB];
#pragma unroll
            for (int q = 0; q < MB; ++q) {
                if (sb + q < ns) {
                    const float *src = a.attn_o + (base + (size_t)(sb + q) * a.qpad) * D;
                    v0[q] = ldc(src + lane);
                    v1[q] = D > 64 ? ldc(src + 64 + lane) : 0.f;
                }
            }
#pragma unroll
            for (int q = 0; q < MB; ++q)
                if (sb + q < ns) {
                    const float wq = __shfl(w, sb + q, 64);
                    acc0 += wq * v0[q];
                    acc1 += wq * v1[q];
                }
        }
        const int r = qi / G, hq = h * G + qi % G;
        float *dst = a.O + ((size_t)r * a.nq + hq) * D;
        stc(dst + lane, acc0 / L);
        if (D > 64) stc(dst + 64 + lane, acc1 / L);
    }
}

// ---------------------------------------------------------------------------
// the kernel
// ---------------------------------------------------------------------------
template <int WT, bool KVF32, int D>
__global__ __launch_bounds__(RND_THREADS, 1) void round_kernel(RoundArgs) {
    // GEMM activation fragments (32 KiB) / attention K, V^T blocks (2 stages)
    constexpr int LDS_U4 = 2 * AttnLds<KVF32, D>::STAGE > 2048 ? 2 * AttnLds<KVF32, D>::STAGE : 2048;
    __shared__ u32x4 lds[LDS_U4];
    Prefetch pf;
    unsigned *bar;
    unsigned long long *tr;
    unsigned gen;
    int nl, first, last, tk = 0;
    {
        const RoundScalars a = kscalars();
        bar = a.bar;
        tr = a.trace;
        nl = a.nl; first = a.first; last = a.last;
        gen = ldc_u(a.bar + BAR_GEN + (blockIdx.x & 7) * 32);
    }
    const MatRef none{nullptr, nullptr, 0, 0};
    // one GEMM's operands, built from fresh copies of the scalars
    auto io_make = [&](int which, int l) {
        const RoundScalars a = kscalars();
        const LayerRefs L = klayer(l);
        GemmIO io;
        io.rows = a.b; io.part = a.part;
        io.G = 0; io.cD = nullptr; io.cbase = nullptr; io.crinv = a.d2_rinv;
        if (which == 0) { io.p = a.p_qkv; io.s0 = L.q; io.s1 = L.k; io.s2 = L.v; io.A = a.X; io.gain = L.g_in; }
        else if (which == 1) { io.p = a.p_o; io.s0 = L.o; io.s1 = none; io.s2 = none; io.A = a.O; io.gain = nullptr; }
        else if (which == 2) { io.p = a.p_gu; io.s0 = L.g; io.s1 = L.u; io.s2 = none; io.A = a.X; io.gain = L.g_post; }
        else { io.p = a.p_d; io.s0 = L.d; io.s1 = none; io.s2 = none; io.A = a.Z; io.gain = nullptr; }
        if (a.d2 && which == 0) { io.G = a.d2; io.cD = a.d2_Da; io.cbase = L.abase; }
        if (a.d2 && which == 2) { io.G = a.d2; io.cD = a.d2_Dm; io.cbase = L.mbase; }
        return io;
    };

    trace_mark(tr, tk);
    if (nl > 0) gemm_issue_first<WT, false>(io_make(0, 0), pf);
    if (first) {
        init_phase(kscalars());
        if (!grid_sync(bar, gen)) return;
        trace_mark(tr, tk);
    }
    const int d2 = kscalars().d2;
    for (int l = 0; l < nl; ++l) {
        if (d2) {                                   // DFlash2: attention prepare coefficients
            const RoundScalars a = kscalars();
            const LayerRefs L = klayer(l);
            d2_phase<WT>(a, L.aw, L.g_in, a.d2_Da);
            if (!grid_sync(bar, gen)) return;
            trace_mark(tr, tk);
        }
        gemm_run<WT, false>(io_make(0, l), pf, lds);
        if (!grid_sync(bar, gen)) return;
        trace_mark(tr, tk);
        {
            const RoundScalars a = kscalars();
            const LayerRefs L = klayer(l);
            qkv_phase<KVF32, D>(a, L.q.s, L.k.s, L.v.s, L.g_q, L.g_k, opaque(kargs())->inv_freq,
                                a.kc + (size_t)l * a.kv_lstride, a.vc + (size_t)l * a.kv_lstride);
        }
        if (!grid_sync(bar, gen)) return;
        trace_mark(tr, tk);
        {
            const RoundScalars a = kscalars();
            attn_phase<KVF32, D>(a, a.kc + (size_t)l * a.kv_lstride, a.vc + (size_t)l * a.kv_lstride, lds);
        }
        gemm_issue_first<WT, false>(io_make(1, l), pf);
        if (!grid_sync(bar, gen)) return;
        trace_mark(tr, tk);
        merge_phase<D>(kscalars());
        if (!grid_sync(bar, gen)) return;
        trace_mark(tr, tk);
        gemm_run<WT, false>(io_make(1, l), pf, lds);
        gemm_issue_first<WT, true>(io_make(2, l), pf);
        if (!grid_sync(bar, gen)) return;
        trace_mark(tr, tk);
        {
            const RoundScalars a = kscalars();
            const LayerRefs L = klayer(l);
            if (a.d2) residual_phase(a, a.p_o, L.o, a.d2_Da, L.abase + 2 * (size_t)a.H);
            else residual_phase(a, a.p_o, L.o);
        }
        if (!grid_sync(bar, gen)) return;
        trace_mark(tr, tk);
        if (d2) {                                   // DFlash2: MLP prepare coefficients
            const RoundScalars a = kscalars();
            const LayerRefs L = klayer(l);
            d2_phase<WT>(a, L.mw, L.g_post, a.d2_Dm);
            if (!grid_sync(bar, gen)) return;
            trace_mark(tr, tk);
        }
        gemm_run<WT, true>(io_make(2, l), pf, lds);
        gemm_issue_first<WT, false>(io_make(3, l), pf);
        if (!grid_sync(bar, gen)) return;
        trace_mark(tr, tk);
        swiglu_phase(kscalars(), klayer(l));
        if (!grid_sync(bar, gen)) return;
        trace_mark(tr, tk);
        gemm_run<WT, false>(io_make(3, l), pf, lds);
        if (l + 1 < nl) gemm_issue_first<WT, false>(io_make(0, l + 1), pf);
        if (!grid_sync(bar, gen)) return;
        trace_mark(tr, tk);
        {
            const RoundScalars a = kscalars();
            const LayerRefs L = klayer(l);
            if (a.d2) residual_phase(a, a.p_d, L.d, a.d2_Dm, L.mbase + 2 * (size_t)a.H);
            else residual_phase(a, a.p_d, L.d);
        }
        if (!grid_sync(bar, gen)) return;
        trace_mark(tr, tk);
    }
    if (last) final_phase(kscalars());
    __syncthreads();
    trace_mark(tr, tk);
}

template <int WT, bool KVF32>
static void launch_d(const RoundArgs &a, int nwg, hipStream_t s) {
    if (a.s.d == 64) hipLaunchKernelGGL((round_kernel<WT, KVF32, 64>), dim3(nwg), dim3(RND_THREADS), 0, s, a);
    else if constexpr (!KVF32) hipLaunchKernelGGL((round_kernel<WT, KVF32, 128>), dim3(nwg), dim3(RND_THREADS), 0, s, a);
}

hipError_t round_launch(const RoundArgs &a, int nwg, hipStream_t s) {
    switch (a.s.wt) {
        case WT_F32: launch_d<WT_F32, true>(a, nwg, s); break;
        case WT_BF16: launch_d<WT_BF16, false>(a, nwg, s); break;
        default: launch_d<WT_FP8, false>(a, nwg, s); break;
    }
    return hipGetLastError();
}

}  // namespace dfl
