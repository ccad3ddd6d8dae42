// Tiled GEMM for tall activations:  Y[M, N] = A[M, K] . W[N, K]^T
// with A in f32, W in bf16 (torch Linear layout), M >= 256: the ctx_features
// fc and the ingest k|v projections of a long context (first light, prefill).
//
// * Workgroup tile 128 rows x 128 columns, eight waves; wave w computes rows
//   [16 w, 16 w + 16) of the tile against all 128 columns: 8 MFMA 16x16x32
//   tiles.  Like the skinny kernel, the activations enter the MFMA as bf16
//   hi + lo parts (two MFMAs per tile and k step, ~16-bit activation
//   precision); the split is made in registers, right before the MFMAs.
// * K runs in stages of 64.  Each wave loads the A fragments of its own rows
//   straight into registers (lane (r, g): row r, k 8g .. 8g + 7 of each k
//   step of 32, two 16-byte loads), since no other wave reads them, and two
//   of the stage's sixteen W fragments (column tile, k step; lane (c, g):
//   8 k values of column c), which it writes to a double-buffered LDS tile
//   that all eight waves read.  Loads run two stages ahead through a
//   three-stage register ring; one workgroup barrier per stage.
// * Two waves per SIMD: what bounds this kernel is latency (the LDS round
//   trip, the hi / lo split and the barrier of every stage), and the second
//   wave hides part of it.  With one wave per SIMD (four waves of 32 rows)
//   the same tile took 175 us for the 1024-row fc, with eight 157 us.
// * A 128-column tile reads each A row (f32) once for twice the columns of
//   a 64-column one.  When the tiles do not fill the device, K is split in
//   two halves; the half that finishes first stores its partial into the
//   tile's own place in Y (write-through), the other adds it to its own and
//   stores the result.  Two-term f32 sums do not depend on the order, so the
//   result is the same whichever half arrives first.
// * Tiles are spread so that the workgroups of one XCD share column tiles
//   (their W stays in that XCD's L2) and sweep every row tile.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace dfl {
namespace {

constexpr int TM = 128, TN = 128, TK = 64;         // tile rows, columns, k per stage
constexpr int CT = TN / 16, KSTEP = TK / 32;
constexpr int NW = 8;                              // waves per workgroup
constexpr int RT = TM / 16 / NW;                   // 16-row tiles per wave
constexpr int WF = CT * KSTEP / NW;                // W fragments (column tile, k step) each wave loads per stage
static_assert(RT * NW * 16 == TM && WF * NW == CT * KSTEP, "tile split over the waves");

struct Stage {
    u32x4 a[KSTEP][RT][2];   // [k step][row tile][half]: 8 f32 of one row
    u32x4 w[WF];             // this wave's W fragments, 8 bf16 of one column
};

// Device-coherent 16-byte store / load (SC1: written through to memory,
// read past the XCD's L2) for the split halves' partial sums.
constexpr int CPOL_SC1 = 16;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t y_rsrc(const float *base) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(base), 0, 0x7fffffff, 0x00020000);
}

__global__ __launch_bounds__(64 * NW) void gemm_tall_kernel(GemmArgs p, int nrt, int nct, int nsplit) {
    __shared__ u32x4 wl[2][CT * KSTEP * 64];
    __shared__ unsigned role, seen;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int r16 = lane & 15, g = lane >> 4;

    // work item of this workgroup (tile, K half): consecutive workgroups go
    // to different XCDs (round robin over 8), so item i runs on XCD
    // i / (items / 8) when the item count is a multiple of 8; the tiles of
    // one XCD are column-major
    const int ntile = nrt * nct, nitem = ntile * nsplit;
    int it = blockIdx.x;
    if (nitem % 8 == 0) it = (blockIdx.x % 8) * (nitem / 8) + blockIdx.x / 8;
    const int t = it % ntile, half = it / ntile;
    const int rt0 = t % nrt, ct0 = t / nrt;
    const int m0 = rt0 * TM, n0 = ct0 * TN;
    const int kc = p.K / nsplit, kbeg = half * kc;

    // weight segment holding columns [n0, n0 + 128) (segments are multiples of 128 wide)
    int scol = n0, s = 0;
    while (s + 1 < p.nseg && scol >= p.seg[s].n) { scol -= p.seg[s].n; ++s; }
    const char *wseg = (const char *)p.seg[s].w;
    const size_t K = p.K;

    // this lane's sources: A rows of its wave's two row tiles (clamped into
    // range; rows past M are never stored), W rows of the column tiles this
    // wave loads
    const int w0 = m0 + 16 * RT * wave;            // first row of this wave
    const float *arow[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) arow[rt] = p.A + (size_t)min(w0 + 16 * rt + r16, p.M - 1) * p.lda + kbeg + 8 * g;
    // W fragment f = WF wave + i of a stage: column tile f / KSTEP, k step f % KSTEP
    const char *wrow[WF];
#pragma unroll
    for (int i = 0; i < WF; ++i) {
        const int f = WF * wave + i;
        wrow[i] = wseg + ((size_t)(scol + 16 * (f / KSTEP) + r16) * K + kbeg + 32 * (f % KSTEP) + 8 * g) * 2;
    }

    auto load = [&](Stage &x, int st) {
        const int k0 = st * TK;
#pragma unroll
        for (int ks = 0; ks < KSTEP; ++ks) {
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
                const float *src = arow[rt] + k0 + 32 * ks;
                x.a[ks][rt][0] = *reinterpret_cast<const u32x4 *>(src);
                x.a[ks][rt][1] = *reinterpret_cast<const u32x4 *>(src + 4);
            }
        }
#pragma unroll
        for (int i = 0; i < WF; ++i) x.w[i] = *reinterpret_cast<const u32x4 *>(wrow[i] + (size_t)k0 * 2);
    };

    f32x4 acc[RT][CT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) acc[rt][ct] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int nst = kc / TK;
    constexpr int NR = 3;                          // register ring stages (loads NR - 1 stages ahead)
    Stage ring[NR];
    // Every stage issues the same loads (the last stages reload the final
    // one), so the compiler's load counting is the same on every path and
    // each stage waits for its own loads only.
#pragma unroll
    for (int i = 0; i + 1 < NR; ++i) load(ring[i], min(i, nst - 1));
    // stage st: its W tile to LDS buffer st & 1 (last read in stage st - 2,
    // which every wave finished before the barrier of stage st - 1), the
    // barrier, stage st + NR - 1's loads into the registers stage st - 1
    // used, then the MFMAs
    auto step = [&](auto bufc, int st) {
        constexpr int B = decltype(bufc)::value;
        Stage &x = ring[B];
        u32x4 *wb = wl[st & 1];
#pragma unroll
        for (int i = 0; i < WF; ++i) wb[(WF * wave + i) * 64 + lane] = x.w[i];
        __syncthreads();
        // issued here, ahead of the stage's LDS reads and MFMAs (the
        // scheduler would otherwise sink them below the MFMAs)
        __builtin_amdgcn_sched_barrier(0);
        load(ring[(B + NR - 1) % NR], min(st + NR - 1, nst - 1));
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int ks = 0; ks < KSTEP; ++ks) {
            u32x4 fw[CT];
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) fw[ct] = wb[(ct * KSTEP + ks) * 64 + lane];
            bf16x8 ah[RT], al[RT];
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
                const u32x4 x0 = x.a[ks][rt][0], x1 = x.a[ks][rt][1];
                const float v[8] = {__uint_as_float(x0.x), __uint_as_float(x0.y), __uint_as_float(x0.z), __uint_as_float(x0.w),
                                    __uint_as_float(x1.x), __uint_as_float(x1.y), __uint_as_float(x1.z), __uint_as_float(x1.w)};
                split_bf16x8(v, ah[rt], al[rt]);
            }
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) {
                const bf16x8 b = __builtin_bit_cast(bf16x8, fw[ct]);
#pragma unroll
                for (int rt = 0; rt < RT; ++rt) {
                    acc[rt][ct] = mfma_bf16(ah[rt], b, acc[rt][ct]);
                    acc[rt][ct] = mfma_bf16(al[rt], b, acc[rt][ct]);
                }
            }
        }
    };
    // the loop body is branch-free (for the load counting), the last
    // stages (fewer than NR) follow it
    int st = 0;
    for (; st + NR <= nst; st += NR) {
        step(std::integral_constant<int, 0>{}, st);
        if constexpr (NR > 1) step(std::integral_constant<int, 1 % NR>{}, st + 1);
        if constexpr (NR > 2) step(std::integral_constant<int, 2 % NR>{}, st + 2);
    }
    if (st < nst) step(std::integral_constant<int, 0>{}, st);
    if constexpr (NR > 2) {
        if (st + 1 < nst) step(std::integral_constant<int, 1 % NR>{}, st + 1);
    }

    if (nsplit > 1) {
        // K halves: the first to arrive leaves its partial in Y, the second
        // adds it.  Lane (r16, g) holds rows 4g .. 4g + 3 of column r16 of a
        // 16 x 16 tile; those four sums travel as one 16-byte piece, placed
        // in the same four rows of Y: row 4g + r16 % 4, columns
        // 4 (r16 / 4) .. + 3.  M is a multiple of 4 here, so a group of
        // four rows is either wholly inside or wholly past M.
        unsigned *cnt = p.cnt + 2 * t;
        auto piece = [&](int rt, int ct) -> uint32_t {
            const int row = w0 + 16 * rt + 4 * g + (r16 & 3);
            return (uint32_t)(((size_t)row * p.ldy + n0 + 16 * ct + 4 * (r16 >> 2)) * 4);
        };
        bool rows_in[RT];
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) rows_in[rt] = w0 + 16 * rt + 4 * g < p.M;
        if (threadIdx.x == 0) role = __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __syncthreads();
        if (role == 0) {
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                for (int ct = 0; ct < CT; ++ct)
                    if (rows_in[rt])
                        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, acc[rt][ct]), y_rsrc(p.Y), piece(rt, ct), 0, CPOL_SC1);
            // every partial store must have completed before the flag is raised
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            __syncthreads();
            if (threadIdx.x == 0) __hip_atomic_store(cnt + 1, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            return;
        }
        // the other half has arrived and is storing (it never waits), so
        // this wait ends; the bound only guards against a broken invariant
        if (threadIdx.x == 0) {
            int spins = 0;
            while (__hip_atomic_load(cnt + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == 0u && ++spins < (1 << 24))
                __builtin_amdgcn_s_sleep(2);
            seen = spins < (1 << 24) ? 1u : 0u;
        }
        __syncthreads();
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int ct = 0; ct < CT; ++ct)
                if (rows_in[rt]) {
                    const f32x4 o = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(y_rsrc(p.Y), piece(rt, ct), 0, CPOL_SC1));
                    acc[rt][ct] = seen ? acc[rt][ct] + o : f32x4{__builtin_nanf(""), __builtin_nanf(""), __builtin_nanf(""), __builtin_nanf("")};
                }
        if (threadIdx.x == 0) {
            __hip_atomic_store(cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(cnt + 1, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }

    // epilogue: lane holds rows 4g + j, column r16 of each 16x16 tile
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int row = w0 + 16 * rt + 4 * g + j;
            if (row >= p.M) continue;
            float *y = p.Y + (size_t)row * p.ldy + n0 + r16;
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) y[16 * ct] = acc[rt][ct][j];
        }
}

// K halves when the tiles alone do not fill the device (and the split
// bookkeeping applies: M a multiple of 4, both halves whole stages)
int tall_split(const GemmArgs &a, int ntile) {
    return ntile < GEMM_CUS && a.M % 4 == 0 && a.K % (2 * TK) == 0 && 2 * ntile <= GEMM_MAX_COUNTERS &&
                   (long long)a.M * a.ldy * 4 < 0x7fffffffLL
               ? 2
               : 1;
}

}  // namespace

// Taken only when the work items fill the device (one per compute unit or
// more): with fewer, the skinny kernel's K split spreads the work better
// (measured on the 1024-row k|v projection at 128 tiles of 128 x 64: 39 us
// here, 30 us there).
bool gemm_tall_ok(const GemmArgs &a) {
    if (a.wtype != WT_BF16 || a.M < 256 || a.epi != EPI_STORE || a.K % TK != 0 || a.K <= 0) return false;
    int ncols = 0;
    for (int s = 0; s < a.nseg; ++s) {
        if (a.seg[s].n <= 0 || a.seg[s].n % TN != 0) return false;
        ncols += a.seg[s].n;
    }
    const long long ntile = (long long)((a.M + TM - 1) / TM) * (ncols / TN);
    if (ntile > (1 << 20)) return false;
    return ntile * tall_split(a, (int)ntile) >= GEMM_CUS;
}

hipError_t gemm_tall(const GemmArgs &a, unsigned *cnt, hipStream_t s) {
    int ncols = 0;
    for (int i = 0; i < a.nseg; ++i) ncols += a.seg[i].n;
    const int nrt = (a.M + TM - 1) / TM, nct = ncols / TN, ns = tall_split(a, nrt * nct);
    GemmArgs g = a;
    g.cnt = cnt;
    hipLaunchKernelGGL(gemm_tall_kernel, dim3(nrt * nct * ns), dim3(64 * NW), 0, s, g, nrt, nct, ns);
    return hipGetLastError();
}

}  // namespace dfl
