// Row RMSNorm, and the q/k head norm + NeoX rope + KV stores.
//
// RMSNorm ([DflashDraft] "ctx_features": hidden_norm; the layer norms and the
// final norm): y = g * x / sqrt(mean(x^2) + eps).  One workgroup per row.
//
// K head norm + rope ([memra dflash module] "DflashKv": cached K is
// normed+roped, V raw; [DflashDraft] "rope_yarn": rope_neox_ff with
// per-dimension inverse frequencies, then the q/k scale mscale).
// * One workgroup per (row, layer), so one launch covers every layer whose
//   k|v projections one GEMM produced side by side, and the rows of up to
//   ROPE_MAX_SEQ sequences (consecutive blocks of seq_rows rows), each into
//   its own cache.  It first builds the
//   row's cos/sin table.  The angle pos * inv_freq[j] and its sin/cos are
//   evaluated in f64, so long positions keep full accuracy.
// * Each wave then takes heads in turn.  Lane j < d/2 holds the rope pair
//   (j, j + d/2) of one head: one wave-wide sum of squares gives the head's
//   RMS, and the rotation is lane-local.
// * k and v go to the layer's cache at rows row0 + r (kvview.h: K
//   [page][nkv][P][d], V transposed [page][nkv][d][P]; a contiguous cache
//   is one page of P = capacity rows).
#include "common.h"
#include "kernels.h"

namespace dfl {

__global__ __launch_bounds__(256) void rmsnorm_kernel(const float *__restrict__ x, int ldx,
                                                      const float *__restrict__ g, float *y, int ldy,
                                                      float *xcopy, int H, float eps) {
    const int r = blockIdx.x, tid = threadIdx.x;
    const float *xr = x + (size_t)r * ldx;
    float ss = 0.f;
    for (int c = tid * 4; c < H; c += 256 * 4) {
        float4 v = ld_f4(xr + c);
        ss += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
    }
    ss = wave_sum(ss);
    __shared__ float part[4];
    if ((tid & 63) == 0) part[tid >> 6] = ss;
    __syncthreads();
    const float tot = (part[0] + part[1]) + (part[2] + part[3]);
    const float inv = 1.f / sqrtf(tot / (float)H + eps);
    float *yr = y + (size_t)r * ldy;
    for (int c = tid * 4; c < H; c += 256 * 4) {
        float4 v = ld_f4(xr + c), gg = ld_f4(g + c);
        if (xcopy) *reinterpret_cast<float4 *>(xcopy + (size_t)r * H + c) = v;
        float4 o = make_float4(gg.x * (v.x * inv), gg.y * (v.y * inv), gg.z * (v.z * inv), gg.w * (v.w * inv));
        *reinterpret_cast<float4 *>(yr + c) = o;
    }
}

hipError_t rmsnorm(const float *x, int ldx, const float *g, float *y, int ldy, float *xcopy, int rows, int H,
                   float eps, hipStream_t s) {
    if (rows <= 0) return hipSuccess;
    hipLaunchKernelGGL(rmsnorm_kernel, dim3(rows), dim3(256), 0, s, x, ldx, g, y, ldy, xcopy, H, eps);
    return hipGetLastError();
}

__device__ __forceinline__ void store_kv(char *p, float v, int kv_f32) {
    if (kv_f32) *reinterpret_cast<float *>(p) = v;
    else *reinterpret_cast<uint16_t *>(p) = (uint16_t)f32_to_bf16_bits(v);
}

__global__ __launch_bounds__(256) void kv_norm_rope_kernel(RopeArgs a) {
    const int r = blockIdx.x, l = blockIdx.y, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int half = a.d >> 1;
    __shared__ float cs[MAX_HALF_DIM], sn[MAX_HALF_DIM];
    if (tid < half) {
        double th = (double)a.pos[r] * a.inv_freq[tid];
        double sv, cv;
        sincos(th, &sv, &cv);
        cs[tid] = (float)cv;
        sn[tid] = (float)sv;
    }
    __syncthreads();

    const float *row = a.src + (size_t)r * a.ld + (size_t)l * a.lstride;
    const float *gain = a.g_k[l];
    const int seq = r / a.seq_rows;
    const KvView &kv = a.kv[seq];
    char *kc = kv.k + (size_t)(a.layer0 + l) * kv.lstride, *vc = kv.v + (size_t)(a.layer0 + l) * kv.lstride;
    const int kvd = a.nkv * a.d;
    const bool act = lane < half;
    const float c = act ? cs[lane] : 0.f, s = act ? sn[lane] : 0.f;
    const int crow = a.row0[seq] + r - seq * a.seq_rows;
    const int page = kv_page(kv, crow);

    for (int h = wave; h < 2 * a.nkv; h += 4) {
        if (h < a.nkv) {
            const float *src = row + h * a.d;
            const float x0 = act ? src[lane] : 0.f, x1 = act ? src[lane + half] : 0.f;
            const float ss = wave_sum(x0 * x0 + x1 * x1);
            const float inv = 1.f / sqrtf(ss / (float)a.d + a.eps);
            if (act) {
                const float y0 = gain[lane] * (x0 * inv), y1 = gain[lane + half] * (x1 * inv);
                const float o0 = (y0 * c - y1 * s) * a.mscale;
                const float o1 = (y1 * c + y0 * s) * a.mscale;
                store_kv(kc + kv_k_off(kv, page, a.nkv, h, crow, a.d, lane), o0, a.kv_f32);
                store_kv(kc + kv_k_off(kv, page, a.nkv, h, crow, a.d, lane + half), o1, a.kv_f32);
            }
        } else if (act) {
            const int hh = h - a.nkv;
            const float *src = row + kvd + hh * a.d;
            store_kv(vc + kv_v_off(kv, page, a.nkv, hh, crow, a.d, lane), src[lane], a.kv_f32);
            store_kv(vc + kv_v_off(kv, page, a.nkv, hh, crow, a.d, lane + half), src[lane + half], a.kv_f32);
        }
    }
}

hipError_t kv_norm_rope(const RopeArgs &a, hipStream_t s) {
    if (a.rows <= 0 || a.nl <= 0) return hipSuccess;
    if (a.nl > ROPE_MAX_LAYERS || a.d > 2 * MAX_HALF_DIM) return hipErrorInvalidValue;
    hipLaunchKernelGGL(kv_norm_rope_kernel, dim3(a.rows, a.nl), dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace dfl
