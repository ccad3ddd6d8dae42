// Tiled GEMM for tall activations:  Y[M, N] = A[M, K] . W[N, K]^T
// with A in f32, W in bf16 (torch Linear layout), M >= 256: the ctx_features
// fc and the ingest k|v projections of a long context (first light, prefill).
//
// * Workgroup tile 128 rows x 64 columns, four waves; wave w computes rows
//   [32 w, 32 w + 32) of the tile against all 64 columns: 2 x 4 MFMA
//   16x16x32 tiles.  Like the skinny kernel, the activations enter the MFMA
//   as bf16 hi + lo parts (two MFMAs per tile and k step, ~16-bit activation
//   precision); the split is made when a lane reads its fragment from LDS.
// * K runs in stages of 64.  Each wave loads the A fragments of its own rows
//   straight into registers (lane (r, g): row r, k 8g .. 8g + 7 of each k
//   step of 32, two 16-byte loads), since no other wave reads them, and the
//   W fragments of one column tile (lane (c, g): 8 k values of column c),
//   which it writes to a double-buffered LDS tile that all four waves read.
//   Loads run two stages ahead through a three-stage register ring; one
//   workgroup barrier per stage.
// * Tiles are spread so that the workgroups of one XCD share column tiles
//   (their W stays in that XCD's L2) and sweep every row tile.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace dfl {
namespace {

constexpr int TM = 128, TN = 64, TK = 64;          // tile rows, columns, k per stage
constexpr int CT = TN / 16, KSTEP = TK / 32;

struct Stage {
    u32x4 a[KSTEP][2][2];    // [k step][row tile][half]: 8 f32 of one row
    u32x4 w[KSTEP];          // this wave's column tile, 8 bf16 of one column
};

__global__ __launch_bounds__(256) void gemm_tall_kernel(GemmArgs p, int nrt, int nct) {
    __shared__ u32x4 wl[2][CT * KSTEP * 64];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int r16 = lane & 15, g = lane >> 4;

    // tile of this workgroup: consecutive workgroups go to different XCDs
    // (round robin over 8), so tile t runs on XCD t / (tiles / 8) when the
    // tile count is a multiple of 8; the tiles of one XCD are column-major
    const int ntile = nrt * nct;
    int t = blockIdx.x;
    if (ntile % 8 == 0) t = (blockIdx.x % 8) * (ntile / 8) + blockIdx.x / 8;
    const int rt0 = t % nrt, ct0 = t / nrt;
    const int m0 = rt0 * TM, n0 = ct0 * TN;

    // weight segment holding columns [n0, n0 + 64) (segments are multiples of 64 wide)
    int scol = n0, s = 0;
    while (s + 1 < p.nseg && scol >= p.seg[s].n) { scol -= p.seg[s].n; ++s; }
    const char *wseg = (const char *)p.seg[s].w;
    const size_t K = p.K;

    // this lane's sources: A rows of its wave's two row tiles (clamped into
    // range; rows past M are never stored), W row of the column tile this
    // wave loads
    const float *arow[2];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) arow[rt] = p.A + (size_t)min(m0 + 32 * wave + 16 * rt + r16, p.M - 1) * p.lda + 8 * g;
    const char *wrow = wseg + ((size_t)(scol + 16 * wave + r16) * K + 8 * g) * 2;

    auto load = [&](Stage &x, int st) {
        const int k0 = st * TK;
#pragma unroll
        for (int ks = 0; ks < KSTEP; ++ks) {
#pragma unroll
            for (int rt = 0; rt < 2; ++rt) {
                const float *src = arow[rt] + k0 + 32 * ks;
                x.a[ks][rt][0] = *reinterpret_cast<const u32x4 *>(src);
                x.a[ks][rt][1] = *reinterpret_cast<const u32x4 *>(src + 4);
            }
            x.w[ks] = *reinterpret_cast<const u32x4 *>(wrow + (size_t)(k0 + 32 * ks) * 2);
        }
    };

    f32x4 acc[2][CT];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) acc[rt][ct] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int nst = p.K / TK;
    Stage ring[3];
    // Every stage issues the same ten loads (the last two stages reload the
    // final one), so the compiler's load counting is the same on every path
    // and each stage waits for its own loads only.
    load(ring[0], 0);
    load(ring[1], min(1, nst - 1));
    // stage st: its W tile to LDS buffer st & 1 (last read in stage st - 2,
    // which every wave finished before the barrier of stage st - 1), the
    // barrier, stage st + 2's loads into the registers stage st - 1 used,
    // then the MFMAs
    auto step = [&](auto bufc, int st) {
        constexpr int B = decltype(bufc)::value;
        Stage &x = ring[B];
        u32x4 *wb = wl[st & 1];
#pragma unroll
        for (int ks = 0; ks < KSTEP; ++ks) wb[(wave * KSTEP + ks) * 64 + lane] = x.w[ks];
        __syncthreads();
        // issued here, ahead of the stage's LDS reads and MFMAs (the
        // scheduler would otherwise sink them below the MFMAs)
        __builtin_amdgcn_sched_barrier(0);
        load(ring[(B + 2) % 3], min(st + 2, nst - 1));
        __builtin_amdgcn_sched_barrier(0);
        u32x4 fw[KSTEP][CT];
#pragma unroll
        for (int ks = 0; ks < KSTEP; ++ks)
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) fw[ks][ct] = wb[(ct * KSTEP + ks) * 64 + lane];
#pragma unroll
        for (int ks = 0; ks < KSTEP; ++ks) {
            bf16x8 ah[2], al[2];
#pragma unroll
            for (int rt = 0; rt < 2; ++rt) {
                const u32x4 x0 = x.a[ks][rt][0], x1 = x.a[ks][rt][1];
                const float v[8] = {__uint_as_float(x0.x), __uint_as_float(x0.y), __uint_as_float(x0.z), __uint_as_float(x0.w),
                                    __uint_as_float(x1.x), __uint_as_float(x1.y), __uint_as_float(x1.z), __uint_as_float(x1.w)};
                split_bf16x8(v, ah[rt], al[rt]);
            }
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) {
                const bf16x8 b = __builtin_bit_cast(bf16x8, fw[ks][ct]);
#pragma unroll
                for (int rt = 0; rt < 2; ++rt) {
                    acc[rt][ct] = mfma_bf16(ah[rt], b, acc[rt][ct]);
                    acc[rt][ct] = mfma_bf16(al[rt], b, acc[rt][ct]);
                }
            }
        }
    };
    // the loop body is branch-free (for the load counting), the last one or
    // two stages follow it
    int st = 0;
    for (; st + 3 <= nst; st += 3) {
        step(std::integral_constant<int, 0>{}, st);
        step(std::integral_constant<int, 1>{}, st + 1);
        step(std::integral_constant<int, 2>{}, st + 2);
    }
    if (st < nst) step(std::integral_constant<int, 0>{}, st);
    if (st + 1 < nst) step(std::integral_constant<int, 1>{}, st + 1);

    // epilogue: lane holds rows 4g + j, column r16 of each 16x16 tile
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int row = m0 + 32 * wave + 16 * rt + 4 * g + j;
            if (row >= p.M) continue;
            float *y = p.Y + (size_t)row * p.ldy + n0 + r16;
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) y[16 * ct] = acc[rt][ct][j];
        }
}

}  // namespace

// Taken only when the tiles fill the device (one per compute unit or more):
// with fewer, the skinny kernel's K split spreads the work better (measured
// on the 1024-row k|v projection, 128 tiles: 39 us here, 30 us there).
bool gemm_tall_ok(const GemmArgs &a) {
    if (a.wtype != WT_BF16 || a.M < 256 || a.epi != EPI_STORE || a.K % TK != 0 || a.K <= 0) return false;
    int ncols = 0;
    for (int s = 0; s < a.nseg; ++s) {
        if (a.seg[s].n <= 0 || a.seg[s].n % TN != 0) return false;
        ncols += a.seg[s].n;
    }
    return (long long)((a.M + TM - 1) / TM) * (ncols / TN) >= GEMM_CUS;
}

hipError_t gemm_tall(const GemmArgs &a, hipStream_t s) {
    int ncols = 0;
    for (int i = 0; i < a.nseg; ++i) ncols += a.seg[i].n;
    const int nrt = (a.M + TM - 1) / TM, nct = ncols / TN;
    hipLaunchKernelGGL(gemm_tall_kernel, dim3(nrt * nct), dim3(256), 0, s, a, nrt, nct);
    return hipGetLastError();
}

}  // namespace dfl
