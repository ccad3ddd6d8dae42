// Streamed forward_round kernel for gfx950: every layer of a drafting round
// in one persistent launch ([DflashDraft] "forward_round": only the b block
// rows are projected per layer, block K/V land at cache rows [len, len + b),
// attention is full and non-causal over all len + b keys; [atlas dflash_head]
// overview: pre-norm Qwen3 layers with GQA and a SwiGLU MLP).
//
// One workgroup per CU: one loader wave, eight compute waves and one service
// wave (it computes the rows' 1/rms for the norm-consuming phases as soon as
// they open).
//
// Loader wave.  Weights and the committed K/V rows do not depend on the
// round's activations, so the loader streams them, in the exact order the
// compute waves use them, into a ring of LDS slots with direct-to-LDS loads
// (global_load_lds_dwordx4).  It keeps SR_DEPTH slots in flight, publishes a
// slot once its loads have landed, and reuses a slot once every compute wave
// has released it.  Its only memory operations are these loads, so its
// vector-memory counter tracks them exactly.  HBM keeps streaming while the
// compute waves wait for activations.
//
// Compute waves.  Each layer is a chain of phases.  A phase starts when every
// workgroup has signalled the previous one:
//   Q  q|k|v projection: columns split over workgroups, K split over waves
//   A  attention: (kv head, key split) items; q/k head RMSNorm + NeoX rope
//      in registers from gains and cos/sin staged in LDS; online softmax over
//      the ring's K/V blocks and (last split) the block's own K/V, staged in
//      LDS in the same round trip as q; partial (m, l, O) per split
//   M  merge of the splits -> O, written as o_proj input fragments
//   O  o_proj + residual -> post-attention-norm input fragments
//   G  gate|up + SwiGLU -> down input fragments
//   D  down + residual -> next layer's input fragments
// (with the DFlash2 wrap, a coefficient phase precedes Q and G).
// A workgroup owns the same hidden columns in O and D, so it keeps its slice
// of the residual stream X in LDS for the whole launch.
//
// Activations between phases are bf16 (f32 in the f32 arm) in MFMA fragment
// order, so a compute wave loads its K range with one coalesced 16-byte load
// per lane and k step.  RMSNorm is split: the producer applies the gain, the
// consumer the 1/rms row scale (from per-workgroup partial sums of squares)
// to its GEMM output.
//
// Synchronisation.  Inside a workgroup: LDS words only (no s_barrier; the
// loader never waits for compute waves except for free ring slots).  The last
// compute wave to finish a phase runs the epilogue, waits for its stores and
// bumps phase counter blockIdx % 64 (four workgroups share one, so the
// same-line atomics at a phase end stay short).  Wave 0 polls the 64
// counters, one per lane, with device-coherent loads and publishes the phase
// in LDS.  Each (layer, phase) output has its own workspace buffer, written with
// device-coherent (sc1) stores and first read after the counter says it is
// complete, so plain loads can use the L2 of each XCD.  Counters are never
// reset: the workspace's epoch word counts the phases of earlier launches.
// Every spin is bounded; on expiry the kernel sets the error word and all
// waves leave.
#include <type_traits>

#include "common.h"
#include "sround.h"

namespace dfl {
namespace {

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void lds_void;

// ---------------------------------------------------------------------------
// memory helpers
// ---------------------------------------------------------------------------
__device__ __forceinline__ __amdgpu_buffer_rsrc_t cbuf(const void *base) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, 0x7fffffff, 0x00020000);
}
constexpr int CPOL_SC1 = 16;
// device-coherent stores: written through to memory.  `base` must be
// uniform over the wave; the byte offset is per lane.
__device__ __forceinline__ void st16(void *base, size_t off, u32x4 v) {
    __builtin_amdgcn_raw_buffer_store_b128(v, cbuf(base), (uint32_t)off, 0, CPOL_SC1);
}
__device__ __forceinline__ void st8(void *base, size_t off, u32x2 v) {
    __builtin_amdgcn_raw_buffer_store_b64(v, cbuf(base), (uint32_t)off, 0, CPOL_SC1);
}
__device__ __forceinline__ void st4(void *base, size_t off, uint32_t v) {
    __builtin_amdgcn_raw_buffer_store_b32(v, cbuf(base), (uint32_t)off, 0, CPOL_SC1);
}
__device__ __forceinline__ void st2(void *base, size_t off, uint16_t v) {
    __builtin_amdgcn_raw_buffer_store_b16(v, cbuf(base), (uint32_t)off, 0, CPOL_SC1);
}
// s_waitcnt through the builtin, so the compiler's own counter tracking
// sees the wait (gfx9 encoding: vmcnt[3:0] | expcnt << 4 | lgkmcnt << 8 | vmcnt[5:4] << 14)
__device__ __forceinline__ void vm_wait() { __builtin_amdgcn_s_waitcnt(0x0F70); }     // vmcnt(0)
__device__ __forceinline__ unsigned ldc_u(unsigned *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void stc_u(unsigned *p, unsigned v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void add_u(unsigned *p, unsigned v) {
    __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// LDS words shared by the waves of the workgroup.  Loads return a
// wave-uniform value, so the spin loops around them branch on scalars.
__device__ __forceinline__ unsigned lds_ld(unsigned *p) {
    return __builtin_amdgcn_readfirstlane(__hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP));
}
__device__ __forceinline__ void lds_st(unsigned *p, unsigned v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
__device__ __forceinline__ unsigned lds_add(unsigned *p, unsigned v) {
    return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
__device__ __forceinline__ void cbar() { asm volatile("" ::: "memory"); }
// LDS word access for the loader wave.  Its direct-to-LDS loads are
// outstanding while it touches its counters; through the builtins the
// compiler would drain them (vmcnt(0)) before every such access, since it
// cannot tell the counters apart from the ring.  These never alias the ring.
__device__ __forceinline__ uint32_t lds_off(const void *p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void *)p;
}
__device__ __forceinline__ unsigned lds_ld_nodep(const unsigned *p) {
    unsigned v;
    asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(lds_off(p)) : "memory");
    return __builtin_amdgcn_readfirstlane(v);
}
__device__ __forceinline__ void lds_st_nodep(unsigned *p, unsigned v) {
    asm volatile("ds_write_b32 %0, %1" : : "v"(lds_off(p)), "v"(v) : "memory");
}
__device__ __forceinline__ float f_of(uint32_t u) { return __uint_as_float(u); }
__device__ __forceinline__ uint32_t bf2(float a, float b) { return bf16_pack(a, b); }

// Lane and wave index behind an opaque copy: values derived from them are
// recomputed inside each phase rather than hoisted out of the layer loop
// (which would keep them live, in registers, for the whole kernel).
__device__ __forceinline__ int lane_id() {
    int l = threadIdx.x & 63;
    asm volatile("" : "+v"(l));
    return l;
}
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

// The arguments are read in place from the kernel-argument segment.  Code
// outside the kernel function itself has no kernarg-segment pointer (that
// intrinsic yields null there), but it does receive the implicit-argument
// pointer, and the implicit arguments start right after the explicit ones.
typedef const __attribute__((address_space(4))) SrArgs KArgs;
static_assert(sizeof(SrArgs) % 8 == 0, "implicit arguments follow SrArgs directly");
__device__ __forceinline__ KArgs *ka() {
    return (KArgs *)((const __attribute__((address_space(4))) char *)__builtin_amdgcn_implicitarg_ptr() - sizeof(SrArgs));
}
#define SS (ka()->s)

constexpr int SPIN_LIMIT = 1 << 22;

// ---------------------------------------------------------------------------
// per-dtype constants
//   KW: K values per 16-byte weight load of one lane times the 4 lane groups
//   ES: bytes per weight, P: activation values per lane and k step,
//   AB: bytes per activation value, AFR: 16-byte activation pieces per step
// ---------------------------------------------------------------------------
template <int WT> struct TR;
template <> struct TR<WT_BF16> { static constexpr int KW = 32, ES = 2, P = 8, AB = 2, AFR = 1; };
template <> struct TR<WT_FP8>  { static constexpr int KW = 64, ES = 1, P = 16, AB = 2, AFR = 2; };
template <> struct TR<WT_F32>  { static constexpr int KW = 16, ES = 4, P = 4, AB = 4, AFR = 1; };

// element offset of activation (row r, column c) in fragment order: lane
// (r, g) of k step c / KW holds the P consecutive columns of group g
template <int WT>
__device__ __forceinline__ size_t frag_idx(int r, int c) {
    constexpr int KW = TR<WT>::KW, P = TR<WT>::P;
    const int ks = c / KW, rem = c - ks * KW, g = rem / P, j = rem - g * P;
    return ((size_t)(ks * 4 + g) * 16 + r) * P + j;
}

// store 4 consecutive activation values (c 4-aligned) as fragment elements
template <int WT>
__device__ __forceinline__ void put4(void *buf, int r, int c, float x0, float x1, float x2, float x3) {
    const size_t e = frag_idx<WT>(r, c);
    if constexpr (TR<WT>::AB == 4) st16(buf, e * 4, u32x4{__float_as_uint(x0), __float_as_uint(x1), __float_as_uint(x2), __float_as_uint(x3)});
    else st8(buf, e * 2, u32x2{bf2(x0, x1), bf2(x2, x3)});
}

// Two-plane bf16 activations (used with the DFlash2 wrap): the plane at buf
// holds bf16(x), the plane lo_off bytes further the rounding residual
// bf16(x - bf16(x)), so a GEMM over both planes sees x to about 16 bits.
__device__ __forceinline__ float bf_round(float x) { return __uint_as_float(bf16_pack(x, 0.f) << 16); }
template <int WT, bool HL>
__device__ __forceinline__ void put4x(void *buf, size_t lo_off, int r, int c, float x0, float x1, float x2, float x3) {
    if constexpr (HL) {
        static_assert(TR<WT>::AB == 2, "two planes hold bf16 activations");
        const uint32_t h01 = bf16_pack(x0, x1), h23 = bf16_pack(x2, x3);
        const size_t e = frag_idx<WT>(r, c);
        st8(buf, e * 2, u32x2{h01, h23});
        st8((char *)buf + lo_off, e * 2,
            u32x2{bf16_pack(x0 - __uint_as_float(h01 << 16), x1 - __uint_as_float(h01 & 0xFFFF0000u)),
                  bf16_pack(x2 - __uint_as_float(h23 << 16), x3 - __uint_as_float(h23 & 0xFFFF0000u))});
    } else {
        put4<WT>(buf, r, c, x0, x1, x2, x3);
    }
}

// ---------------------------------------------------------------------------
// LDS
// ---------------------------------------------------------------------------
static_assert(64 + SR_MAXCH <= 128, "aux holds 64 scales then the gains");
struct SrLds {
    u32x4 ring[SR_NSLOT][SR_CW][64];
    f32x4 red[SR_CW][SR_MAXT][64];
    float xown[16][SR_MAXCH];
    float rinv[16];
    float aux[128];            // epilogue constants of the phase: fp8 scales [tile][16], gains [64..)
    unsigned cons[SR_CW];      // slots each compute wave has released
    unsigned pub;              // slots the loader has published
    unsigned phase;            // global phases known complete
    unsigned rphase;           // phase whose row scales rinv holds (+1)
    unsigned done;             // compute-wave arrivals (8 per phase)
    unsigned stg;              // compute-wave arrivals at the attention staging (8 per layer)
    unsigned abort_;
    unsigned sink_;            // never read: keeps the service wave's L2 prefetch loads alive
};

// the workgroup's LDS (each kernel instance allocates its own copy)
__shared__ SrLds S;


// a bounded wait ran out: every wave leaves; the kernel's exit path records
// the error in the workspace

__device__ __forceinline__ void set_error(SrLds &S) { lds_st(&S.abort_, 1u); }

// Phase trace (workgroup 0, when enabled): stamp k of phase p at word 8p + k.
//   0 wave 0 sees the phase's inputs complete   1 wave 0 done with its share
//   2 epilogue done and signalled                3 loader issues the phase's first slot
//   4 loader has issued the phase's last slot
__device__ __forceinline__ void trace_at(unsigned p, int k) {
    if (blockIdx.x == 0 && (threadIdx.x & 63) == 0 && SS.trace && 8 * p + k < SR_TRACE) SS.trace[8 * p + k] = wall_clock64();
}

// ---------------------------------------------------------------------------
// phase list of a launch
// ---------------------------------------------------------------------------
enum Kind { K_INIT, K_DA, K_Q, K_A, K_M, K_O, K_DM, K_G, K_D };
__device__ __forceinline__ int npl() { return SS.d2 ? 8 : 6; }
__device__ __forceinline__ int kind_at(int i) {   // i-th phase of a layer
    if (SS.d2) {
        switch (i) {
            case 0: return K_DA; case 1: return K_Q; case 2: return K_A; case 3: return K_M;
            case 4: return K_O; case 5: return K_DM; case 6: return K_G; default: return K_D;
        }
    }
    switch (i) {
        case 0: return K_Q; case 1: return K_A; case 2: return K_M; case 3: return K_O; case 4: return K_G; default: return K_D;
    }
}
__device__ __forceinline__ char *layer_buf(int l) { return SS.lay + (size_t)l * SS.lay_stride; }

// ---------------------------------------------------------------------------
// GEMM tiles: output columns of this workgroup in pieces of <= 16
// ---------------------------------------------------------------------------
struct GT {
    const char *w;       // weight row of the tile's first column
    const float *sc;     // fp8 row scales of the tile's first column, or nullptr
    int n;               // columns (<= 16, multiple of 4)
    int col;             // first column within its matrix
    int seg;             // Q: 0 q, 1 k, 2 v;  G: 0 gate, 1 up
};

__device__ __forceinline__ SrMat kmat(const __attribute__((address_space(4))) SrMat &m) { return SrMat{m.w, m.s}; }

__device__ __forceinline__ int gemm_K(int kind) {
    return kind == K_O ? SS.qd : kind == K_D ? SS.I : SS.H;
}

// Tiles of a run of m columns (m a multiple of 4): 16-wide tiles, then the
// remainder as an 8-wide and/or a 4-wide tile, so every tile is 16, 8 or 4
// columns wide (a narrow tile packs 2 or 4 k steps into one ring part).
__device__ __forceinline__ int run_tiles(int m) {
    const int r = m & 15;
    return (m >> 4) + (r == 12 ? 2 : r ? 1 : 0);
}
// first column (relative to the run) and width of tile t of a run of m
__device__ __forceinline__ void run_tile(int m, int t, int &c, int &n) {
    const int full = m >> 4, r = m & 15;
    if (t < full) { c = 16 * t; n = 16; return; }
    c = 16 * full;
    if (r == 12) { if (t == full) n = 8; else { c += 8; n = 4; } }
    else n = r;
}

// number of tiles of this workgroup for a GEMM phase
__device__ __forceinline__ int gemm_nt(int kind) {
    const int w = blockIdx.x;
    switch (kind) {
        case K_Q: {
            const int c0 = w * SS.cq, c1 = c0 + SS.cq;
            const int a[3] = {0, SS.qd, SS.qd + SS.kvd}, e[3] = {SS.qd, SS.qd + SS.kvd, SS.qd + 2 * SS.kvd};
            int nt = 0;
#pragma unroll
            for (int s = 0; s < 3; ++s) {
                const int lo = max(c0, a[s]), hi = min(c1, e[s]);
                if (hi > lo) nt += run_tiles(hi - lo);
            }
            return nt;
        }
        case K_O: case K_D: return run_tiles(SS.ch);
        case K_G: return 2 * run_tiles(SS.ci);
        default: return 16 * w < 4 * SS.d2 ? run_tiles(min(16, 4 * SS.d2 - 16 * w)) : 0;     // K_DA, K_DM
    }
}

template <int WT>
__device__ __forceinline__ GT gemm_tile(int kind, int l, int t) {
    constexpr int ES = TR<WT>::ES;
    const int w = blockIdx.x;
    const int K = gemm_K(kind);
    GT r{nullptr, nullptr, 0, 0, 0};
    auto mk = [&](SrMat m, int col, int n, int seg) {
        r.w = (const char *)m.w + (size_t)col * K * ES;
        r.sc = m.s ? m.s + col : nullptr;
        r.n = n; r.col = col; r.seg = seg;
    };
    switch (kind) {
        case K_Q: {
            const int c0 = w * SS.cq, c1 = c0 + SS.cq;
            const int a[3] = {0, SS.qd, SS.qd + SS.kvd}, e[3] = {SS.qd, SS.qd + SS.kvd, SS.qd + 2 * SS.kvd};
            int base = 0;
#pragma unroll
            for (int s = 0; s < 3; ++s) {
                const int lo = max(c0, a[s]), hi = min(c1, e[s]);
                if (hi > lo) {
                    const int n = run_tiles(hi - lo);
                    if (t >= base && t < base + n) {
                        int c, nn;
                        run_tile(hi - lo, t - base, c, nn);
                        const SrMat m = s == 0 ? kmat(ka()->L[l].q) : s == 1 ? kmat(ka()->L[l].k) : kmat(ka()->L[l].v);
                        mk(m, lo - a[s] + c, nn, s);
                    }
                    base += n;
                }
            }
            break;
        }
        case K_O: case K_D: {
            int c, nn;
            run_tile(SS.ch, t, c, nn);
            mk(kind == K_O ? kmat(ka()->L[l].o) : kmat(ka()->L[l].d), w * SS.ch + c, nn, 0);
            break;
        }
        case K_G: {
            const int ntg = run_tiles(SS.ci);
            const int s = t < ntg ? 0 : 1;
            int c, nn;
            run_tile(SS.ci, t - s * ntg, c, nn);
            mk(s == 0 ? kmat(ka()->L[l].g) : kmat(ka()->L[l].u), w * SS.ci + c, nn, s);
            break;
        }
        default: {   // K_DA, K_DM
            int c, nn;
            run_tile(min(16, 4 * SS.d2 - 16 * w), t, c, nn);
            mk(kind == K_DA ? kmat(ka()->L[l].aw) : kmat(ka()->L[l].mw), 16 * w + c, nn, 0);
            break;
        }
    }
    return r;
}

// k steps of one GEMM pass per wave (activations of one pass are held in
// registers; the next pass's are loaded while this one runs) and the most
// passes built.  Each wave takes npass * NF consecutive k steps; steps past
// the end of K are dead (loader and compute waves agree on the count).
template <int WT> struct PassCfg { static constexpr int NF = WT == WT_FP8 ? 4 : 8; };
constexpr int SR_MAXPASS = 3;
template <int WT>
__device__ __forceinline__ int gemm_npass(int nst) {
    constexpr int NF = PassCfg<WT>::NF;
    const int nkw = (nst + SR_CW - 1) / SR_CW;
    return (nkw + NF - 1) / NF;
}

// attention item of this workgroup: kv head, key range, whether it holds the block
struct AItem {
    int h, k_lo, k_hi, last, nblk;
};
__device__ __forceinline__ bool attn_item(AItem &it) {
    const int item = blockIdx.x;
    if (item >= SS.nkv * SS.nsplit) return false;
    const int ns = SS.nsplit, nb = SS.nkb;
    it.h = item / ns;
    const int s = item - it.h * ns;
    // The last split attends the block's own keys (normed and roped in the
    // item itself), the others the cache's 32-key blocks, spread so that
    // their sizes differ by at most one.  With a single split it takes both.
    const int nc = ns > 1 ? ns - 1 : 1;
    if (s < nc) {
        const int b0 = nb - (nc - s) * nb / nc, b1 = nb - (nc - s - 1) * nb / nc;
        it.k_lo = 32 * b0;
        it.k_hi = min(SS.len, 32 * b1);
    } else {
        it.k_lo = it.k_hi = SS.len;
    }
    if (it.k_hi < it.k_lo) it.k_hi = it.k_lo;
    it.last = s == ns - 1;
    it.nblk = (it.k_hi - it.k_lo + 31) / 32;
    return true;
}

// K/V parts of one 32-key block: KP parts of K, then V^T parts (d tile t,
// half hv); eight parts fill one ring slot.
// The block's K rows are one contiguous run of the cache, so K part p is the
// contiguous 1 KB of keys p KPP .. p KPP + KPP - 1, with the 16-byte chunks of
// each row permuted: chunk cc of key k sits at chunk cc ^ kswz(k) of its row.
// An MFMA fragment read (16 keys, one chunk) then meets 16 distinct bank
// groups.
template <int WT, int D> struct AT {
    static constexpr bool F32 = WT == WT_F32;
    static constexpr int KVB = F32 ? 4 : 2;          // bytes per cached K/V value
    static constexpr int NC = D * KVB / 64;          // d chunks of 16 bytes per lane group
    static constexpr int KP = 2 * NC;
    static constexpr int RB = D * KVB;               // bytes per cached K row
    static constexpr int KPP = 1024 / RB, CPR = RB / 16;   // keys per K part, chunks per row
    static constexpr int VH = F32 ? 2 : 1;
    static constexpr int VP = (D / 16) * VH;
    static constexpr int SLOTS = (KP + VP) / 8;
    static constexpr int PQ = F32 ? 4 : 8;           // values per lane per d chunk
    static constexpr int NQV = D / 4;                // values per lane per head row
    static_assert(KPP * KP == 32 && (CPR == 8 || CPR == 16 || CPR == 32), "K part layout");
    // key k of a block (k = 8a + 4 kt + b): the fragment read of key tile kt
    // takes (a, b) over all 16 lanes, and (k % KPP) CPR + (cc ^ kswz) must
    // be distinct modulo 16 chunks
    __device__ static int kswz(int k) {
        const int a = (k >> 3) & 3, b = k & 3;
        return CPR == 8 ? (((b >> 1) & 1) | (a << 1)) : (b | (a << 2));
    }
};

// ---------------------------------------------------------------------------
// loader wave
// ---------------------------------------------------------------------------
struct Loader {
    unsigned seq;       // next slot to fill
    unsigned freed;     // slots known released by every compute wave
};

__device__ __forceinline__ bool loader_wait_free(SrLds &S, Loader &ld) {
    // slot seq reuses the storage of slot seq - NSLOT
    if (ld.seq < SR_NSLOT) return true;
    const unsigned need = ld.seq - SR_NSLOT + 1;
    int spins = 0;
    bool drained = false;
    while (ld.freed < need) {
        unsigned m = 0xffffffffu;
#pragma unroll
        for (int v = 0; v < SR_CW; ++v) m = min(m, lds_ld_nodep(&S.cons[v]));
        ld.freed = m;
        if (ld.freed >= need) break;
        if (!drained && ld.seq > SR_DEPTH) {
            // the ring is full and the compute waves are not consuming (they
            // wait for a phase): hand them every slot already issued
            drained = true;
            vm_wait();
            lds_st_nodep(&S.pub, ld.seq);
        }
        if (lds_ld_nodep(&S.abort_)) return false;
        if (++spins > SPIN_LIMIT) { lds_st_nodep(&S.abort_, 1u); return false; }
        __builtin_amdgcn_s_sleep(1);
    }
    return true;
}

// after the 8 loads of slot seq are issued: publish the slot SR_DEPTH behind
__device__ __forceinline__ void loader_commit(SrLds &S, Loader &ld) {
    ++ld.seq;
    if (ld.seq > SR_DEPTH) {
        static_assert(8 * SR_DEPTH == 24, "wait immediate");
        __builtin_amdgcn_s_waitcnt(0x4F78);                  // vmcnt(24): 8 * SR_DEPTH loads may stay in flight
        cbar();
        lds_st_nodep(&S.pub, ld.seq - SR_DEPTH);
    }
}

// Weight bytes are read once per launch: the non-temporal hint lets L2 evict
// them first, so the stream does not push out the code, the kernel arguments
// and the activations the workgroups share.
constexpr int CPOL_NT = 2;
__device__ __forceinline__ void dma16(const void *g, u32x4 *ldsdst) {
    __builtin_amdgcn_global_load_lds(g, (lds_void *)ldsdst, 16, 0, CPOL_NT);
}

// Slot layout of a group of 4 k steps: for each step, the tiles in order; a
// tile of width n takes one slot per 16 / n steps (its part holds that many
// steps).  off[t][j] is the slot (within the group) holding tile t's step j,
// cnt[j] the slots of steps 0..j.
struct Grp {
    int n[SR_MAXT], off[SR_MAXT][4], cnt[4], slots;
};
template <int WT>
__device__ __forceinline__ Grp grp_layout(int kind, int l, int nt) {
    // every field is wave-uniform and kept in scalar registers
    Grp G;
#pragma unroll
    for (int t = 0; t < SR_MAXT; ++t) G.n[t] = __builtin_amdgcn_readfirstlane(t < nt ? gemm_tile<WT>(kind, l, t).n : 16);
    // part of tile t that holds step j of a group: a new part every 16/n steps
    int c = 0, cur[SR_MAXT];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
#pragma unroll
        for (int t = 0; t < SR_MAXT; ++t) {
            const int m = G.n[t] == 16 ? 0 : G.n[t] == 8 ? 1 : 3;     // 16 / n - 1
            if (t < nt && (j & m) == 0) cur[t] = c++;
            G.off[t][j] = __builtin_amdgcn_readfirstlane(t < nt ? cur[t] : 0);
        }
        G.cnt[j] = __builtin_amdgcn_readfirstlane(c);
    }
    G.slots = __builtin_amdgcn_readfirstlane(c);
    return G;
}

// Packed weight stream.  The GEMM weights do not depend on the round, so
// they are rearranged once (sround_pack_kernel) into the exact order the
// loader wave moves them: per layer and GEMM phase, per workgroup, a run of
// ring slots, each slot SR_CW parts of 64 lanes x 16 bytes, contiguous.  The
// loader then streams 8 KiB runs; read in place, a part is 16 weight rows of
// 64 bytes each, which one wave moves at about half the contiguous rate.
// Slots per workgroup of one phase: groups of 4 k steps times one slot per 4
// of its columns (a 16-wide tile fills 4 slots per group, an 8-wide 2, a
// 4-wide 1); cols is the most columns any workgroup has in the phase.
__host__ __device__ inline long long pk_wg_slots(int wt, int K, int cols) {
    const int kw = wt == WT_BF16 ? 32 : wt == WT_FP8 ? 64 : 16;
    const int nf = wt == WT_FP8 ? 4 : 8;
    const int nkw = ((K / kw + SR_CW - 1) / SR_CW + nf - 1) / nf * nf;
    return (long long)(nkw / 4) * (cols / 4);
}
static_assert(TR<WT_BF16>::KW == 32 && TR<WT_FP8>::KW == 64 && TR<WT_F32>::KW == 16,
              "pk_wg_slots repeats the k values per 16-byte weight load for host-side sizing");
static_assert(PassCfg<WT_BF16>::NF == 8 && PassCfg<WT_FP8>::NF == 4 && PassCfg<WT_F32>::NF == 8,
              "pk_wg_slots repeats the k steps per pass for host-side sizing");
__host__ __device__ inline long long pk_wg_bytes(int wt, int kind, int H, int I, int qd, int cq, int ch, int ci) {
    const int K = kind == K_O ? qd : kind == K_D ? I : H;
    const int cols = kind == K_Q ? cq : (kind == K_O || kind == K_D) ? ch : kind == K_G ? 2 * ci : 16;
    return pk_wg_slots(wt, K, cols) * SR_SLOT;
}
// byte offset of a phase's runs in the layer's stream (phases in the order
// DA, Q, O, DM, G, D; DA and DM only with the DFlash2 wrap); any other kind
// gives the layer's total
__host__ __device__ inline long long pk_layer_off(int wt, int kind, int H, int I, int qd, int cq, int ch, int ci, int nwg, int d2) {
    long long off = 0;
    for (int i = 0; i < 6; ++i) {
        const int k = i == 0 ? K_DA : i == 1 ? K_Q : i == 2 ? K_O : i == 3 ? K_DM : i == 4 ? K_G : K_D;
        if (k == kind) return off;
        if (d2 == 0 && (k == K_DA || k == K_DM)) continue;
        off += (long long)nwg * pk_wg_bytes(wt, k, H, I, qd, cq, ch, ci);
    }
    return off;
}
// this workgroup's slot run of one GEMM phase of local layer l
template <int WT>
__device__ __forceinline__ char *pk_run(int kind, int l) {
    const long long off = pk_layer_off(WT, kind, SS.H, SS.I, SS.qd, SS.cq, SS.ch, SS.ci, SS.nwg, SS.d2) +
                          (long long)blockIdx.x * pk_wg_bytes(WT, kind, SS.H, SS.I, SS.qd, SS.cq, SS.ch, SS.ci);
    return ka()->L[l].pk + off;
}

// Writes this workgroup's slot run of one GEMM phase: slot by slot in the
// loader's order, part v of a slot holding what compute wave v consumes.
// Lane L of a part of tile t (width n) takes row L % n, lane group
// (L / n) % 4, of step L / (4 n) of the part's steps; steps past the end of
// K (dead steps) repeat step 0 and are never used.
template <int WT>
__device__ __forceinline__ void pack_gemm(int kind, int l) {
    constexpr int KW = TR<WT>::KW, ES = TR<WT>::ES, P = TR<WT>::P;
    const int lane = lane_id();
    const int nt = gemm_nt(kind);
    if (nt == 0) return;
    const int K = gemm_K(kind), nst = K / KW, nkw = gemm_npass<WT>(nst) * PassCfg<WT>::NF;
    const char *row[SR_MAXT];
    int sofs[SR_MAXT], spi[SR_MAXT];
#pragma unroll
    for (int t = 0; t < SR_MAXT; ++t) {
        row[t] = nullptr; sofs[t] = 0; spi[t] = 1;
        if (t < nt) {
            const GT tl = gemm_tile<WT>(kind, l, t);
            const int n = tl.n;
            row[t] = tl.w + (size_t)(lane & (n - 1)) * K * ES + (size_t)((lane / n) & 3) * P * ES;
            sofs[t] = lane / (4 * n);
            spi[t] = 16 / n;
        }
    }
    char *run = pk_run<WT>(kind, l);
    size_t si = 0;
    for (int j = 0; j < nkw; j += 4) {
        for (int j4 = 0; j4 < 4; ++j4) {
#pragma unroll
            for (int t = 0; t < SR_MAXT; ++t) {
                if (t < nt && (j4 & (spi[t] - 1)) == 0) {
                    u32x4 val[SR_CW];
#pragma unroll
                    for (int v = 0; v < SR_CW; ++v) {
                        int ks = v * nkw + j + j4 + sofs[t];
                        ks = ks < nst ? ks : 0;
                        val[v] = *reinterpret_cast<const u32x4 *>(row[t] + (size_t)ks * KW * ES);
                    }
#pragma unroll
                    for (int v = 0; v < SR_CW; ++v)
                        *reinterpret_cast<u32x4 *>(run + (si * SR_CW + v) * SR_PART + 16 * lane) = val[v];
                    ++si;
                }
            }
        }
    }
}

// Streams this workgroup's slot run of one GEMM phase into the ring: slot by
// slot, each lane moving 16 contiguous bytes per part.
template <int WT>
__device__ __forceinline__ bool load_gemm(SrLds &S, Loader &ld, int kind, int l) {
    const int nt = gemm_nt(kind);
    if (nt == 0) return true;
    const int nst = gemm_K(kind) / TR<WT>::KW, nkw = gemm_npass<WT>(nst) * PassCfg<WT>::NF;
    int cols = 0;
#pragma unroll
    for (int t = 0; t < SR_MAXT; ++t)
        if (t < nt) cols += gemm_tile<WT>(kind, l, t).n;
    const int nslot = __builtin_amdgcn_readfirstlane(nkw / 4 * (cols / 4));
    const char *src = pk_run<WT>(kind, l) + 16 * lane_id();
    for (int si = 0; si < nslot; ++si) {
        if (!loader_wait_free(S, ld)) return false;
        u32x4 *dst = &S.ring[ld.seq % SR_NSLOT][0][0];
#pragma unroll
        for (int v = 0; v < SR_CW; ++v) dma16(src + ((size_t)si * SR_CW + v) * SR_PART, dst + v * 64);
        loader_commit(S, ld);
    }
    return true;
}

template <int WT, int D>
__device__ __forceinline__ bool load_attn(SrLds &S, Loader &ld, int l) {
    using A = AT<WT, D>;
    AItem it;
    if (!attn_item(it)) return true;
    const int lane = lane_id(), n16 = lane & 15, g = lane >> 4;
    const char *kc = SS.kc + (size_t)l * SS.kv_lstride;
    const char *vc = SS.vc + (size_t)l * SS.kv_lstride;
    const int cap = SS.cap;
    for (int blk = 0; blk < it.nblk; ++blk) {
        const int k0 = it.k_lo + 32 * blk;
        for (int sl = 0; sl < A::SLOTS; ++sl) {
            if (!loader_wait_free(S, ld)) return false;
            u32x4 *dst = &S.ring[ld.seq % SR_NSLOT][0][0];
#pragma unroll
            for (int v = 0; v < SR_CW; ++v) {
                const int idx = sl * 8 + v;
                const char *src;
                if (idx < A::KP) {
                    // part idx, LDS chunk `lane`: row lane / CPR, chunk lane % CPR
                    const int kk = idx * A::KPP + lane / A::CPR;
                    const int cc = (lane % A::CPR) ^ A::kswz(kk);
                    int key = k0 + kk;
                    key = key < it.k_hi ? key : it.k_lo;                      // masked later
                    src = kc + (((size_t)it.h * cap + key) * D) * A::KVB + cc * 16;
                } else {
                    // V [nkv][cap / 32][d][32]: a part (16 d rows of the
                    // block's 32-key tile) is one contiguous 1 KB (bf16)
                    const int q = idx - A::KP, t = q / A::VH, hv = q - t * A::VH;
                    int key = k0 + 8 * g + 4 * hv;
                    key = key < it.k_hi ? key : it.k_lo;                      // masked later
                    src = vc + ((((size_t)it.h * (cap / 32) + key / 32) * D + 16 * t + n16) * 32 + key % 32) * A::KVB;
                }
                dma16(src, dst + v * 64);
            }
            loader_commit(S, ld);
        }
    }
    return true;
}

template <int WT, int D>
__device__ __forceinline__ void loader_main(SrLds &S) {
    Loader ld{0u, 0u};
    const int nl = SS.nl, np = npl();
    bool ok = true;
    for (int l = 0; l < nl && ok; ++l) {
        for (int i = 0; i < np && ok; ++i) {
            const int k = kind_at(i);
            const unsigned p = 1 + (unsigned)(l * np + i);
            trace_at(p, 3);
            if (k == K_A) ok = load_attn<WT, D>(S, ld, l);
            else if (k != K_M) ok = load_gemm<WT>(S, ld, k, l);
            trace_at(p, 4);
        }
    }
    vm_wait();
    if (ok) lds_st_nodep(&S.pub, ld.seq);
}

// ---------------------------------------------------------------------------
// compute waves: ring consumption
// ---------------------------------------------------------------------------
struct Cons {
    unsigned seq;       // next slot to use
    unsigned avail;     // slots known published
};

__device__ __forceinline__ bool ring_wait(SrLds &S, Cons &c, unsigned upto) {   // slots < upto available
    upto = __builtin_amdgcn_readfirstlane(upto);
    c.avail = __builtin_amdgcn_readfirstlane(c.avail);
    int spins = 0;
    while (c.avail < upto) {
        c.avail = lds_ld(&S.pub);
        if (c.avail >= upto) break;
        if (lds_ld(&S.abort_)) return false;
        if (++spins > SPIN_LIMIT) { set_error(S); return false; }
        __builtin_amdgcn_s_sleep(1);
    }
    return true;
}
__device__ __forceinline__ void ring_release(SrLds &S, unsigned upto) {
    cbar();
    // kept scalar up to the store, so no vector copy of it lives across the step loop
    unsigned u = __builtin_amdgcn_readfirstlane(upto);
    asm volatile("" : "+s"(u));
    lds_st(&S.cons[threadIdx.x >> 6], u);
}

// wait until `p` global phases are complete (wave 0 polls, the others read LDS)
__device__ __forceinline__ bool wait_phase(SrLds &S, unsigned p, unsigned E) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    int spins = 0;
    if (wave == 0) {
        static_assert(SR_NCTR <= 64 && 64 % SR_NCTR == 0, "one counter per lane group");
        const int x = lane % SR_NCTR;
        const unsigned nwg = gridDim.x;
        const unsigned per = nwg > (unsigned)x ? (nwg - x + SR_NCTR - 1) / SR_NCTR : 0u;
        const unsigned want = (E + p) * per;
        unsigned *ctr = SS.ctr + x * 32;
        bool seen = per == 0;       // counters are monotonic: a lane stops reading once its group is done
        while (true) {
            if (!seen) seen = (int)(ldc_u(ctr) - want) >= 0;
            if (__all(seen)) break;
            if (lds_ld(&S.abort_)) return false;
            if (++spins > SPIN_LIMIT / 8) { set_error(S); return false; }
            // about 0.43 us between polls: each poll reads 64 lines device-wide
            // from every workgroup, and tighter polling slows the whole grid
            // (measured at ctx 4096: pauses of 0.05 and 0.2 us cost 1.0% and
            // 0.6% of a round, 0.64 and 0.85 us 0.5% and 0.9%)
            __builtin_amdgcn_s_sleep(16);
        }
        if (blockIdx.x == 0 && lane == 0) {
            if (SS.trace && 8 * p < SR_TRACE) SS.trace[8 * p] = wall_clock64();
            // every workgroup has read the epoch before signalling phase 0
            if (p == 1) stc_u(SS.ctr + SR_CTR_EPOCH, E + 1 + (unsigned)SS.nl * npl());
        }
        lds_st(&S.phase, p);
        return true;
    }
    while (lds_ld(&S.phase) < p) {
        if (lds_ld(&S.abort_)) return false;
        if (++spins > SPIN_LIMIT) { set_error(S); return false; }
        __builtin_amdgcn_s_sleep(1);
    }
    return true;
}

// 1/rms of the 16 rows from partial sums of squares [nwg][16] (wave 0).
// Lane (r, q) sums workgroups q, q + 4, ...; every load is issued before the
// first add, and each load instruction reads 4 workgroups' 64 bytes at once.
__device__ __forceinline__ void compute_rinv(SrLds &S, const float *ssq, unsigned p, int width) {
    const int lane = lane_id(), r = lane & 15, q = lane >> 4;
    const int nwg = gridDim.x;
    constexpr int NPL = 256 / 4;                       // workgroups per lane at most
    float v[NPL];
#pragma unroll
    for (int i = 0; i < NPL; ++i) {
        const int w = q + 4 * i;
        v[i] = ssq[(size_t)(w < nwg ? w : 0) * 16 + r];
    }
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < NPL; ++i) s += q + 4 * i < nwg ? v[i] : 0.f;
    s = group4_sum(s);
    if (q == 0) S.rinv[r] = 1.f / sqrtf(s / (float)width + SS.eps);
    cbar();
    if (lane == 0) lds_st(&S.rphase, p + 1);
}
__device__ __forceinline__ bool wait_rinv(SrLds &S, unsigned p) {
    int spins = 0;
    while (lds_ld(&S.rphase) < p + 1) {
        if (lds_ld(&S.abort_)) return false;
        if (++spins > SPIN_LIMIT) { set_error(S); return false; }
        __builtin_amdgcn_s_sleep(1);
    }
    cbar();
    return true;
}

// arrival of a compute wave; true for the last of the eight
__device__ __forceinline__ bool arrive(SrLds &S) {
    cbar();
    unsigned old = 0;
    if ((threadIdx.x & 63) == 0) old = lds_add(&S.done, 1u);
    old = __builtin_amdgcn_readfirstlane(old);      // every lane is active again: lane 0's value
    cbar();
    return (old & 7u) == 7u;
}
__device__ __forceinline__ void signal_phase() {
    vm_wait();
    if ((threadIdx.x & 63) == 0) add_u(SS.ctr + (blockIdx.x % SR_NCTR) * 32, 1u);
}
// wave 1 of workgroup 0: stamp k of phase p at trace word 512 + 8p + k
__device__ __forceinline__ void dbg_at(unsigned p, int k) {
    if (blockIdx.x == 0 && (threadIdx.x >> 6) == 1 && (threadIdx.x & 63) == 0 && SS.trace && 8 * p + k < 512)
        SS.trace[512 + 8 * p + k] = wall_clock64();
}
// every workgroup's signal time of phases 7..18 (trace words 1024 + 256 (p - 7) + w)
__device__ __forceinline__ void trace_all(unsigned p) {
    if ((threadIdx.x & 63) == 0 && SS.trace && p >= 7 && p < 19) SS.trace[1024 + 256 * (p - 7) + blockIdx.x] = wall_clock64();
}

// ---------------------------------------------------------------------------
// residual slice -> next GEMM input (X * gain in fragment order) and partial
// sums of squares; with gain == nullptr only the sums (final norm).  gain
// points at the gain of this workgroup's first column.
// ---------------------------------------------------------------------------
template <int WT, bool HL>
__device__ __forceinline__ void emit_input(SrLds &S, const float *gain, char *frag, float *ssq) {
    const int lane = lane_id();
    const int ch = SS.ch, c0 = blockIdx.x * SS.ch, nq = ch / 4;
    if (frag && gain) {
        for (int i = lane; i < 16 * nq; i += 64) {
            const int r = i / nq, q = i - r * nq, c = 4 * q;
            const float4 gg = *reinterpret_cast<const float4 *>(gain + c);
            put4x<WT, HL>(frag, (size_t)16 * SS.H * 2, r, c0 + c, S.xown[r][c] * gg.x, S.xown[r][c + 1] * gg.y, S.xown[r][c + 2] * gg.z,
                     S.xown[r][c + 3] * gg.w);
        }
    }
    if (lane < 16) {
        // every LDS read of the row issued before the first add (ch is a multiple of 4)
        float s = 0.f;
#pragma unroll
        for (int c = 0; c < SR_MAXCH; c += 4) {
            if (c >= ch) break;
            const float4 x = *reinterpret_cast<const float4 *>(&S.xown[lane][c]);
            s += x.x * x.x + x.y * x.y + x.z * x.z + x.w * x.w;
        }
        // [workgroup][row]: the 16 sums of one workgroup are one 64-byte store
        st4(ssq, ((size_t)blockIdx.x * 16 + lane) * 4, __float_as_uint(s));
    }
}

// ---------------------------------------------------------------------------
// GEMM phase (compute waves)
// ---------------------------------------------------------------------------
template <int WT>
__device__ __forceinline__ void mac(f32x4 &acc, const u32x4 &w, const u32x4 *a) {
    if constexpr (WT == WT_BF16) {
        acc = mfma_bf16(__builtin_bit_cast(bf16x8, w), __builtin_bit_cast(bf16x8, a[0]), acc);
    } else if constexpr (WT == WT_FP8) {
        acc = mfma_bf16(fp8x8_to_bf16x8(w.x, w.y), __builtin_bit_cast(bf16x8, a[0]), acc);
        acc = mfma_bf16(fp8x8_to_bf16x8(w.z, w.w), __builtin_bit_cast(bf16x8, a[1]), acc);
    } else {
        acc = mfma_f32(f_of(w.x), f_of(a[0].x), acc);
        acc = mfma_f32(f_of(w.y), f_of(a[0].y), acc);
        acc = mfma_f32(f_of(w.z), f_of(a[0].z), acc);
        acc = mfma_f32(f_of(w.w), f_of(a[0].w), acc);
    }
}

// DFlash2 prepare conv on the staged activations of one k step ([DflashDraft]
// "d2_conv_prepare"): xc[r,c] = (b[c,0] + D[r,g(c),0]) xn[r-1,c] + (b[c,1] +
// D[r,g(c),1]) xn[r,c], xn = (X * gain) / rms, xn[-1] = 0.
template <int WT, bool HL>
__device__ __forceinline__ void d2_prepare(SrLds &S, u32x4 *a, u32x4 *alo, int kstep, const float *base, const float *Dc) {
    constexpr int KW = TR<WT>::KW, P = TR<WT>::P, AFR = TR<WT>::AFR;
    const int lane = lane_id(), r = lane & 15, g = lane >> 4;
    const int c0 = kstep * KW + g * P;
    const int G = SS.d2, grp = c0 * G / SS.H;
    const float ri = S.rinv[r], rp = r > 0 ? S.rinv[r - 1] : 0.f;
    const float d0 = Dc[r * 4 * G + 2 * grp], d1 = Dc[r * 4 * G + 2 * grp + 1];
    float x[P];
    if constexpr (TR<WT>::AB == 4) {
#pragma unroll
        for (int i = 0; i < 4; ++i) x[i] = f_of(a[0][i]);
    } else {
#pragma unroll
        for (int f = 0; f < AFR; ++f)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                x[8 * f + 2 * i] = bf16_bits_to_f32(a[f][i] & 0xFFFFu);
                x[8 * f + 2 * i + 1] = __uint_as_float(a[f][i] & 0xFFFF0000u);
                if constexpr (HL) {
                    x[8 * f + 2 * i] += bf16_bits_to_f32(alo[f][i] & 0xFFFFu);
                    x[8 * f + 2 * i + 1] += __uint_as_float(alo[f][i] & 0xFFFF0000u);
                }
            }
    }
    float y[P];
#pragma unroll
    for (int i = 0; i < P; ++i) {
        const float xp = row_shr1(x[i]);            // row r - 1 (unused for r = 0)
        const float2 bb = *reinterpret_cast<const float2 *>(base + (size_t)(c0 + i) * 2);
        y[i] = (bb.x + d0) * (r > 0 ? xp * rp : 0.f) + (bb.y + d1) * (x[i] * ri);
    }
    if constexpr (TR<WT>::AB == 4) {
        a[0] = u32x4{__float_as_uint(y[0]), __float_as_uint(y[1]), __float_as_uint(y[2]), __float_as_uint(y[3])};
    } else {
#pragma unroll
        for (int f = 0; f < AFR; ++f)
            a[f] = u32x4{bf2(y[8 * f], y[8 * f + 1]), bf2(y[8 * f + 2], y[8 * f + 3]), bf2(y[8 * f + 4], y[8 * f + 5]),
                         bf2(y[8 * f + 6], y[8 * f + 7])};
        if constexpr (HL) {
#pragma unroll
            for (int i = 0; i < P; ++i) y[i] -= bf_round(y[i]);
#pragma unroll
            for (int f = 0; f < AFR; ++f)
                alo[f] = u32x4{bf2(y[8 * f], y[8 * f + 1]), bf2(y[8 * f + 2], y[8 * f + 3]), bf2(y[8 * f + 4], y[8 * f + 5]),
                               bf2(y[8 * f + 6], y[8 * f + 7])};
        }
    }
}

// the epilogue's view of one tile: lane (r, g) holds columns 4g..4g+3 of row r
template <int WT>
__device__ __forceinline__ f32x4 tile_sum(SrLds &S, int t) {
    const int lane = lane_id();
    f32x4 s = S.red[0][t][lane];
#pragma unroll
    for (int v = 1; v < SR_CW; ++v) s += S.red[v][t][lane];
    return s;
}

// DFlash2 finish conv ([DflashDraft] "d2_conv_finish") of 4 columns of row r:
// y'[r,c] = (b[c,0] + D[r,G+g(c),0]) y[r-1,c] + (b[c,1] + D[r,G+g(c),1]) y[r,c]
__device__ __forceinline__ void d2_finish(float (&y)[4], int r, int c, const float *base, const float *Dc) {
    const int lane = lane_id();
    const int G = SS.d2, grp = c * G / SS.H;
    const float d0 = Dc[r * 4 * G + 2 * (G + grp)], d1 = Dc[r * 4 * G + 2 * (G + grp) + 1];
    const float *b1 = base + 2 * (size_t)SS.H;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float yp = row_shr1(y[i]);            // row r - 1 (unused for r = 0)
        const float2 bb = *reinterpret_cast<const float2 *>(b1 + (size_t)(c + i) * 2);
        y[i] = (bb.x + d0) * (r > 0 ? yp : 0.f) + (bb.y + d1) * y[i];
    }
}

template <int WT, int D, bool C>
__device__ __forceinline__ void gemm_epilogue(SrLds &S, int kind, int l, unsigned p, int nt) {
    constexpr bool HL = C && TR<WT>::AB == 2;      // two-plane activations with the DFlash2 wrap
    // fp8 weights always carry row scales (staged in S.aux); the others never
    constexpr bool FP8 = WT == WT_FP8;
    const int lane = lane_id(), r = lane & 15, g = lane >> 4;
    char *lb = layer_buf(l), *ln = layer_buf(l + 1);
    constexpr bool d2 = C;
    const int b = SS.b;
    if (kind == K_Q || kind == K_G || kind == K_DA || kind == K_DM)
        if (!wait_rinv(S, p)) return;
    const float rs = S.rinv[r];
    if (kind == K_Q) {
        constexpr int PQ = AT<WT, D>::PQ, KSA = 4 * PQ, AB = TR<WT>::AB;
        char *qkv = lb + SS.o_qkv;
        const size_t koff = (size_t)16 * SS.qd * AB, voff = (size_t)16 * (SS.qd + SS.kvd) * AB;
        char *vcache = SS.vc + (size_t)l * SS.kv_lstride;
#pragma unroll
        for (int t = 0; t < SR_MAXT; ++t) {
            if (t >= nt) break;
            const GT tl = gemm_tile<WT>(K_Q, l, t);
            const f32x4 sum = tile_sum<WT>(S, t);
            const int cl = 4 * g;
            if (cl >= tl.n) continue;
            float y[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) y[i] = sum[i] * (d2 ? 1.f : rs) * (FP8 ? S.aux[16 * t + cl + i] : 1.f);
            const int col = tl.col + cl;
            if (tl.seg < 2) {
                const int hh = col / D, dd = col - hh * D;
                const int s = dd / KSA, rem = dd - s * KSA, g2 = rem / PQ, j = rem - g2 * PQ;
                const size_t e = ((size_t)(hh * 16 + r) * 4 + g2) * (D / 4) + s * PQ + j;
                char *dst = qkv + (tl.seg == 1 ? koff : 0);
                if constexpr (AB == 4) st16(dst, e * 4, u32x4{__float_as_uint(y[0]), __float_as_uint(y[1]), __float_as_uint(y[2]), __float_as_uint(y[3])});
                else st8(dst, e * 2, u32x2{bf2(y[0], y[1]), bf2(y[2], y[3])});
            } else {
                const int hh = col / D, dd = col - hh * D;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const size_t e = ((size_t)hh * D + dd + i) * 16 + r;          // V^T of the block
                    const int key = SS.len + r;                                    // V [nkv][cap / 32][d][32]
                    const size_t ce = (((size_t)hh * (SS.cap / 32) + key / 32) * D + dd + i) * 32 + key % 32;
                    if constexpr (AB == 4) {
                        st4(qkv + voff, e * 4, __float_as_uint(y[i]));
                        if (r < b) st4(vcache, ce * 4, __float_as_uint(y[i]));
                    } else {
                        const uint16_t hb = (uint16_t)f32_to_bf16_bits(y[i]);
                        st2(qkv + voff, e * 2, hb);
                        if (r < b) st2(vcache, ce * 2, hb);
                    }
                }
            }
        }
    } else if (kind == K_O || kind == K_D) {
        const int c0 = blockIdx.x * SS.ch;
        const float *base = nullptr, *Dc = nullptr;
        if constexpr (C) {
            base = kind == K_O ? ka()->L[l].abase : ka()->L[l].mbase;
            Dc = (const float *)(lb + (kind == K_O ? SS.o_da : SS.o_dm));
        }
        for (int t = 0; t < nt; ++t) {
            const GT tl = gemm_tile<WT>(kind, l, t);
            const f32x4 sum = tile_sum<WT>(S, t);
            const int cl = 4 * g;
            float y[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) y[i] = sum[i] * (FP8 && cl < tl.n ? S.aux[16 * t + cl + i] : 1.f);
            if constexpr (C) d2_finish(y, r, tl.col + cl, base, Dc);
            if (cl < tl.n) {
                const int xc = tl.col - c0 + cl;
#pragma unroll
                for (int i = 0; i < 4; ++i) S.xown[r][xc + i] += r < b ? y[i] : 0.f;
            }
        }
        cbar();
        __builtin_amdgcn_wave_barrier();
        if (kind == K_O) {
            emit_input<WT, HL>(S, S.aux + 64, lb + SS.o_xm, (float *)(lb + SS.o_ssm));
        } else {
            const bool more = l + 1 < SS.nl;
            emit_input<WT, HL>(S, more ? S.aux + 64 : nullptr, more ? ln + SS.o_xa : nullptr, (float *)(ln + SS.o_ssa));
            if (!more && !SS.last) {
                for (int i = lane; i < 16 * SS.ch; i += 64) {
                    const int rr = i / SS.ch, c = i - rr * SS.ch;
                    st4(SS.xsave, ((size_t)rr * SS.H + c0 + c) * 4, __float_as_uint(S.xown[rr][c]));
                }
            }
        }
    } else if (kind == K_G) {
        const int ntg = nt / 2;
        char *zf = lb + SS.o_zf;
#pragma unroll
        for (int t = 0; t < SR_MAXT / 2; ++t) {
            if (t >= ntg) break;
            const GT tg = gemm_tile<WT>(K_G, l, t), tu = gemm_tile<WT>(K_G, l, t + ntg);
            const f32x4 sg = tile_sum<WT>(S, t), su = tile_sum<WT>(S, t + ntg);
            const int cl = 4 * g;
            if (cl >= tg.n) continue;
            float z[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float gv = sg[i] * (d2 ? 1.f : rs) * (FP8 ? S.aux[16 * t + cl + i] : 1.f);
                const float uv = su[i] * (d2 ? 1.f : rs) * (FP8 ? S.aux[16 * (t + ntg) + cl + i] : 1.f);
                z[i] = r < b ? gv / (1.f + __expf(-gv)) * uv : 0.f;
            }
            put4x<WT, HL>(zf, (size_t)16 * SS.I * 2, r, tg.col + cl, z[0], z[1], z[2], z[3]);
        }
    } else {   // K_DA, K_DM: dynamic conv coefficients D[r][j] = rinv[r] * s_j * (X * g)[r] . W_dyn[j]
        if (nt > 0) {
            const GT tl = gemm_tile<WT>(kind, l, 0);
            const f32x4 sum = tile_sum<WT>(S, 0);
            float *Dc = (float *)(lb + (kind == K_DA ? SS.o_da : SS.o_dm));
            const int cl = 4 * g;
            if (cl < tl.n) {
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    st4(Dc, ((size_t)r * 4 * SS.d2 + tl.col + cl + i) * 4,
                        __float_as_uint(sum[i] * rs * (FP8 ? S.aux[cl + i] : 1.f)));
            }
        }
    }
}

// One pass of NF k steps (groups of 4) with the pass's activations in
// registers.  The ring parts of a step are read together before its MFMAs,
// so the LDS latency is paid about once per step rather than once per part:
// every tile's part of a step (tiles past nt read a valid part that is not
// used).  The build for exactly NTF = 1 tile (its own function, so it holds
// a single accumulator) reads the parts of all four steps of a group at once.
template <int WT, bool C, int NTF>
__device__ __forceinline__ bool gemm_pass(SrLds &S, Cons &cs, const Grp &G, u32x4 *a, u32x4 *alo, int ks, int nst, int nt,
                                          bool conv, const float *cbase, const float *cD, f32x4 (&acc)[SR_MAXT]) {
    constexpr int AFR = TR<WT>::AFR, NF = PassCfg<WT>::NF;
    constexpr bool HL = C && TR<WT>::AB == 2;       // alo != a: the activations' low plane
    const int v = wave_id();
    const u32x4 *ringv = &S.ring[0][v][0];
    // ring part of tile t at step j4 of the group whose first slot is s0 in the
    // ring.  Lane L of a part of an n-wide tile holds row L % n of lane group
    // L / n (n is 16, 8 or 4, so shifts and masks instead of products).
    auto part = [&](unsigned s0, int j4, int t) -> u32x4 {
        const int n = G.n[t];
        const int lg = n == 16 ? 4 : n == 8 ? 3 : 2;
        // off < the group's slots <= SR_NSLOT - SR_DEPTH (sround_nwg), so one
        // subtraction wraps s0 + off into the ring
        unsigned slot = s0 + (unsigned)G.off[t][j4];
        slot = __builtin_amdgcn_readfirstlane(slot >= SR_NSLOT ? slot - SR_NSLOT : slot);
        const int ln = lane_id();
        const int m = (16 >> lg) - 1;                            // 16 / n - 1
        const int L = (((j4 & m) << 2) << lg) + (((ln >> 4) << lg) | (ln & (n - 1)));
        return ringv[(size_t)slot * (SR_SLOT / 16) + L];
    };
#pragma unroll
    for (int q = 0; q < NF / 4; ++q) {
        const unsigned g0 = cs.seq;
        const unsigned s0 = __builtin_amdgcn_readfirstlane(g0 % SR_NSLOT);
        if constexpr (NTF > 0) {
            if constexpr (C) {
                if (conv) {
#pragma unroll
                    for (int j4 = 0; j4 < 4; ++j4) {
                        const int j = 4 * q + j4;
                        if (ks + j < nst) d2_prepare<WT, HL>(S, &a[j * AFR], &alo[j * AFR], ks + j, cbase, cD);
                    }
                }
            }
            if (!ring_wait(S, cs, g0 + G.slots)) return false;
            constexpr int B = 4 / NTF;                   // steps per batch of 4 parts
#pragma unroll
            for (int j0 = 0; j0 < 4; j0 += B) {
                u32x4 wv[B][NTF];
#pragma unroll
                for (int jb = 0; jb < B; ++jb)
#pragma unroll
                    for (int t = 0; t < NTF; ++t) wv[jb][t] = part(s0, j0 + jb, t);
#pragma unroll
                for (int jb = 0; jb < B; ++jb) {
                    const int j = 4 * q + j0 + jb;
                    if (ks + j < nst) {
#pragma unroll
                        for (int t = 0; t < NTF; ++t) {
                            mac<WT>(acc[t], wv[jb][t], &a[j * AFR]);
                            if constexpr (HL) { if (alo != a) mac<WT>(acc[t], wv[jb][t], &alo[j * AFR]); }
                        }
                    }
                }
            }
        } else {
#pragma unroll
            for (int j4 = 0; j4 < 4; ++j4) {
                const int j = 4 * q + j4;
                u32x4 *aj = &a[j * AFR], *alj = &alo[j * AFR];
                const bool live = ks + j < nst;
                if constexpr (C) {
                    if (conv && live) d2_prepare<WT, HL>(S, aj, alj, ks + j, cbase, cD);
                }
                if (!ring_wait(S, cs, g0 + G.cnt[j4])) return false;
                u32x4 wv[SR_MAXT];
#pragma unroll
                for (int t = 0; t < SR_MAXT; ++t) wv[t] = part(s0, j4, t);
                if (live) {
#pragma unroll
                    for (int t = 0; t < SR_MAXT; ++t) {
                        if (t < nt) {
                            mac<WT>(acc[t], wv[t], aj);
                            if constexpr (HL) { if (alo != a) mac<WT>(acc[t], wv[t], alj); }
                        }
                    }
                }
            }
        }
        cs.seq = __builtin_amdgcn_readfirstlane(g0 + G.slots);
        ring_release(S, cs.seq);
    }
    return true;
}

// all k steps of one wave: up to SR_MAXPASS passes, activations double-buffered
template <int WT, bool C, int NTF>
__device__ __forceinline__ bool gemm_steps(SrLds &S, Cons &cs, const Grp &G, const char *act, int ks0, int nst, int nt, int npass,
                                           bool conv, bool hl, const float *cbase, const float *cD, f32x4 (&acc)[SR_MAXT],
                                           unsigned p) {
    constexpr int AFR = TR<WT>::AFR, NF = PassCfg<WT>::NF;
    u32x4 a0[NF * AFR], a1[NF * AFR];
    auto load_pass = [&](int ps, u32x4 *dst, size_t off) {
#pragma unroll
        for (int j = 0; j < NF; ++j) {
            int ks = ks0 + ps * NF + j;
            ks = ks < nst ? ks : 0;                   // dead steps reread step 0
#pragma unroll
            for (int f = 0; f < AFR; ++f)
                dst[j * AFR + f] = *reinterpret_cast<const u32x4 *>(act + off + (size_t)ks * 64 * 16 * AFR + 16 * f);
        }
    };
    if constexpr (C && TR<WT>::AB == 2) {
        if (hl) {
            // two-plane activations: a pass holds both planes of its steps
            // (a0 high, a1 low), so the next pass is not prefetched
            const size_t lo_off = (size_t)16 * nst * TR<WT>::KW * 2;
#pragma unroll
            for (int ps = 0; ps < SR_MAXPASS; ++ps) {
                if (ps < npass) {
                    load_pass(ps, a0, 0);
                    load_pass(ps, a1, lo_off);
                    if (!gemm_pass<WT, C, NTF>(S, cs, G, a0, a1, ks0 + ps * NF, nst, nt, conv, cbase, cD, acc)) return false;
                }
            }
            return true;
        }
    }
    load_pass(0, a0, 0);
    if (npass > 1) load_pass(1, a1, 0);
    if (blockIdx.x == 0 && (threadIdx.x >> 6) == 1 && SS.trace) {
        vm_wait();
        dbg_at(p, 1);
        if (!ring_wait(S, cs, cs.seq + G.cnt[0])) return false;
        dbg_at(p, 4);
    }
    if (!gemm_pass<WT, C, NTF>(S, cs, G, a0, a0, ks0, nst, nt, conv, cbase, cD, acc)) return false;
    if (npass > 1) {
        if (npass > 2) load_pass(2, a0, 0);
        if (!gemm_pass<WT, C, NTF>(S, cs, G, a1, a1, ks0 + NF, nst, nt, conv, cbase, cD, acc)) return false;
        if (npass > 2) {
            if (!gemm_pass<WT, C, NTF>(S, cs, G, a0, a0, ks0 + 2 * NF, nst, nt, conv, cbase, cD, acc)) return false;
        }
    }
    return true;
}

// Kept out of line: inlining every phase into one function makes the
// register allocator spill heavily.  Arguments arrive in VGPRs and are made
// scalar again.
// Returns the consumer's next ring slot, or ~0u if the kernel is aborting.
template <int WT, int D, bool C, int NTF>
__device__ __attribute__((noinline)) unsigned gemm_phase(int kind, int l, unsigned p, unsigned seq) {
    constexpr int KW = TR<WT>::KW, AFR = TR<WT>::AFR;
    kind = __builtin_amdgcn_readfirstlane(kind);
    l = __builtin_amdgcn_readfirstlane(l);
    p = __builtin_amdgcn_readfirstlane(p);
    Cons cs{(unsigned)__builtin_amdgcn_readfirstlane(seq), 0u};
    const int lane = lane_id(), v = wave_id();
    const int nt = NTF > 0 ? NTF : gemm_nt(kind);
    char *lb = layer_buf(l);
    if (nt > 0) {
        const int K = gemm_K(kind), nst = K / KW, npass = gemm_npass<WT>(nst);
        const char *act;
        switch (kind) {
            case K_O: act = lb + SS.o_of; break;
            case K_G: case K_DM: act = lb + SS.o_xm; break;
            case K_D: act = lb + SS.o_zf; break;
            default: act = lb + SS.o_xa; break;     // K_Q, K_DA
        }
        act += (size_t)lane * 16 * AFR;
        const int ks0 = v * npass * PassCfg<WT>::NF;
        const bool conv = C && (kind == K_Q || kind == K_G);
        const float *cbase = nullptr, *cD = nullptr;
        if (conv) {
            if (!wait_rinv(S, p)) return ~0u;
            cbase = kind == K_Q ? ka()->L[l].abase : ka()->L[l].mbase;
            cD = (const float *)(lb + (kind == K_Q ? SS.o_da : SS.o_dm));
        }
        f32x4 acc[SR_MAXT];
#pragma unroll
        for (int t = 0; t < SR_MAXT; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
        dbg_at(p, 0);
        if (v == SR_CW - 1) {
            // epilogue constants into LDS: fp8 scales of the tiles, the next norm's gains
            if (lane < 16 * nt) {
                const GT tl = gemm_tile<WT>(kind, l, lane >> 4);
                if (tl.sc && (lane & 15) < tl.n) S.aux[lane] = tl.sc[lane & 15];
            }
            const float *gn = kind == K_O ? ka()->L[l].g_post : (kind == K_D && l + 1 < SS.nl) ? ka()->L[l + 1].g_in : nullptr;
            if (gn && lane < SS.ch) S.aux[64 + lane] = gn[blockIdx.x * SS.ch + lane];
        }
        const Grp G = grp_layout<WT>(kind, l, nt);
        // with the DFlash2 wrap every GEMM input but o_proj's has two planes
        const bool hl = C && TR<WT>::AB == 2 && kind != K_O;
        const bool ok = gemm_steps<WT, C, NTF>(S, cs, G, act, ks0, nst, nt, npass, conv, hl, cbase, cD, acc, p);
        dbg_at(p, 2);
        if (!ok) return ~0u;
#pragma unroll
        for (int t = 0; t < SR_MAXT; ++t)
            if (t < nt) S.red[v][t][lane] = acc[t];
    }
    if (v == 0) trace_at(p, 1);
    dbg_at(p, 3);
    if (arrive(S)) {
        if (blockIdx.x == 0) trace_at(p, 5);
        if (nt > 0) gemm_epilogue<WT, D, C>(S, kind, l, p, nt);
        signal_phase();
        trace_at(p, 2);
        trace_all(p);
    }
    return cs.seq;
}

// ---------------------------------------------------------------------------
// attention phase (compute waves)
// ---------------------------------------------------------------------------
// q / k head vector of one lane: values (s, j) at d = KSA s + PQ g + j.
// RMSNorm over head_dim (gain gk), NeoX rope with the row's cos/sin pairs
// cs[d/2][2] (pairs s, s + NS/2), times scale.  gk and cs point into LDS.
template <int WT, int D>
__device__ __forceinline__ void norm_rope(float (&x)[D / 4], const float *gk, const float *cs, float scale) {
    constexpr int PQ = AT<WT, D>::PQ, KSA = 4 * PQ, NS = D / KSA, NQV = AT<WT, D>::NQV;
    const int g = lane_id() >> 4;
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < NQV; ++i) ss += x[i] * x[i];
    ss = group4_sum(ss);
    const float inv = 1.f / sqrtf(ss / (float)D + SS.eps);
#pragma unroll
    for (int s = 0; s < NS; ++s)
#pragma unroll
        for (int j = 0; j < PQ; ++j) x[s * PQ + j] *= inv * gk[KSA * s + PQ * g + j];
#pragma unroll
    for (int s = 0; s < NS / 2; ++s)
#pragma unroll
        for (int j = 0; j < PQ; ++j) {
            const int fi = KSA * s + PQ * g + j;
            const float2 csv = *reinterpret_cast<const float2 *>(cs + 2 * fi);
            const float y0 = x[s * PQ + j], y1 = x[(s + NS / 2) * PQ + j];
            x[s * PQ + j] = (y0 * csv.x - y1 * csv.y) * scale;
            x[(s + NS / 2) * PQ + j] = (y1 * csv.x + y0 * csv.y) * scale;
        }
}

template <int WT, int D>
__device__ __forceinline__ void load_head(float (&x)[D / 4], const char *src);

// a lane's q / k head values as raw 16-byte words, then decoded: split so a
// caller can issue several heads' loads before the first use
template <int WT, int D> struct HeadWords { static constexpr int N = (D / 4) / (WT == WT_F32 ? 4 : 8); };
template <int WT, int D>
__device__ __forceinline__ void load_head_raw(u32x4 *u, const char *src) {
#pragma unroll
    for (int i = 0; i < HeadWords<WT, D>::N; ++i) u[i] = *reinterpret_cast<const u32x4 *>(src + 16 * i);
}
template <int WT, int D>
__device__ __forceinline__ void decode_head(float (&x)[D / 4], const u32x4 *u) {
#pragma unroll
    for (int i = 0; i < HeadWords<WT, D>::N; ++i) {
        if constexpr (WT == WT_F32) {
            x[4 * i] = f_of(u[i].x); x[4 * i + 1] = f_of(u[i].y); x[4 * i + 2] = f_of(u[i].z); x[4 * i + 3] = f_of(u[i].w);
        } else {
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                x[8 * i + 2 * k] = bf16_bits_to_f32(u[i][k] & 0xFFFFu);
                x[8 * i + 2 * k + 1] = __uint_as_float(u[i][k] & 0xFFFF0000u);
            }
        }
    }
}

template <int WT, int D>
__device__ __forceinline__ void load_head(float (&x)[D / 4], const char *src) {
    constexpr int NQV = AT<WT, D>::NQV;
    if constexpr (WT == WT_F32) {
#pragma unroll
        for (int i = 0; i < NQV; i += 4) {
            const u32x4 u = *reinterpret_cast<const u32x4 *>(src + 4 * i);
            x[i] = f_of(u.x); x[i + 1] = f_of(u.y); x[i + 2] = f_of(u.z); x[i + 3] = f_of(u.w);
        }
    } else {
#pragma unroll
        for (int i = 0; i < NQV; i += 8) {
            const u32x4 u = *reinterpret_cast<const u32x4 *>(src + 2 * i);
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                x[i + 2 * k] = bf16_bits_to_f32(u[k] & 0xFFFFu);
                x[i + 2 * k + 1] = __uint_as_float(u[k] & 0xFFFF0000u);
            }
        }
    }
}

template <int WT, int D>
struct AttnState {
    static constexpr int NDT = D / 16;
    float m, l;
    f32x4 o[NDT];
};

// NB 32-key blocks at once: S^T = K Q^T (two key tiles per block; lane
// (q, g) ends up with keys 8g..8g+7 of each), one online-softmax update over
// all NB blocks' scores, O^T += V^T P^T.  kf(b, kt, c) / vf(b, t, hv) return
// block b's A fragments; valid(b, i) tells whether key 8g + i of block b
// exists.  Two blocks per update halve the serial max / exp / sum steps and
// the accumulator rescales per key, and let one block's MFMAs overlap the
// other's.
template <int WT, int D, int NB, class KF, class VF, class VALID>
__device__ __forceinline__ void attn_blocks(AttnState<WT, D> &st, const u32x4 *qf, KF kf, VF vf, VALID valid) {
    using A = AT<WT, D>;
    constexpr int NDT = D / 16;
    f32x4 sc4[NB][2];
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int c = 0; c < A::NC; ++c) {
                const u32x4 k = kf(b, kt, c);
                if constexpr (WT == WT_F32) {
                    acc = mfma_f32(f_of(k.x), f_of(qf[c].x), acc);
                    acc = mfma_f32(f_of(k.y), f_of(qf[c].y), acc);
                    acc = mfma_f32(f_of(k.z), f_of(qf[c].z), acc);
                    acc = mfma_f32(f_of(k.w), f_of(qf[c].w), acc);
                } else {
                    acc = mfma_bf16(__builtin_bit_cast(bf16x8, k), __builtin_bit_cast(bf16x8, qf[c]), acc);
                }
            }
            sc4[b][kt] = acc;
        }
    float sc[NB][8];
    float bmax = -INFINITY;
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float x = sc4[b][i >> 2][i & 3];
            sc[b][i] = valid(b, i) ? x : -INFINITY;
            bmax = fmaxf(bmax, sc[b][i]);
        }
    bmax = group4_max(bmax);
    const float m_new = fmaxf(st.m, bmax);
    const float corr = __builtin_amdgcn_exp2f(st.m - m_new);
    float psum = 0.f;
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            sc[b][i] = __builtin_amdgcn_exp2f(sc[b][i] - m_new);
            psum += sc[b][i];
        }
    psum = group4_sum(psum);
    st.l = st.l * corr + psum;
    st.m = m_new;
#pragma unroll
    for (int t = 0; t < NDT; ++t) st.o[t] *= corr;
#pragma unroll
    for (int b = 0; b < NB; ++b) {
        if constexpr (WT == WT_F32) {
#pragma unroll
            for (int t = 0; t < NDT; ++t) {
                const u32x4 v0 = vf(b, t, 0), v1 = vf(b, t, 1);
                const float vk[8] = {f_of(v0.x), f_of(v0.y), f_of(v0.z), f_of(v0.w), f_of(v1.x), f_of(v1.y), f_of(v1.z), f_of(v1.w)};
#pragma unroll
                for (int i = 0; i < 8; ++i) st.o[t] = mfma_f32(valid(b, i) ? vk[i] : 0.f, sc[b][i], st.o[t]);
            }
        } else {
            const bf16x8 pb = to_bf16x8(sc[b]);
#pragma unroll
            for (int t = 0; t < NDT; ++t) {
                u32x4 vv = vf(b, t, 0);
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    const uint32_t msk = (valid(b, 2 * w) ? 0x0000FFFFu : 0u) | (valid(b, 2 * w + 1) ? 0xFFFF0000u : 0u);
                    vv[w] &= msk;
                }
                st.o[t] = mfma_bf16(__builtin_bit_cast(bf16x8, vv), pb, st.o[t]);
            }
        }
    }
}

// one 32-key block (kf(kt, c), vf(t, hv), valid(i))
template <int WT, int D, class KF, class VF, class VALID>
__device__ __forceinline__ void attn_block(AttnState<WT, D> &st, const u32x4 *qf, KF kf, VF vf, VALID valid) {
    attn_blocks<WT, D, 1>(st, qf, [&](int, int kt, int c) { return kf(kt, c); },
                          [&](int, int t, int hv) { return vf(t, hv); }, [&](int, int i) { return valid(i); });
}

template <int WT, int D>
__device__ __forceinline__ bool attn_phase(SrLds &S, Cons &cs, int l, unsigned p) {
    using A = AT<WT, D>;
    constexpr int NQV = A::NQV, NC = A::NC, NDT = D / 16, AB = TR<WT>::AB;
    const int lane = lane_id(), v = wave_id(), r16 = lane & 15, g = lane >> 4;
    AItem it;
    if (attn_item(it)) {
        char *lb = layer_buf(l);
        const char *qkv = lb + SS.o_qkv;
        const size_t koff = (size_t)16 * SS.qd * AB, voff = (size_t)16 * (SS.qd + SS.kvd) * AB;
        const bool actw = v < SS.G;
        const int hq = it.h * SS.G + (actw ? v : 0);
        // The layer's q/k head-norm gains and the block rows' cos/sin go to
        // LDS (the GEMM reduction area is idle during attention), loaded in
        // the same round trip as this wave's q head: [0, D) g_q, [D, 2D) g_k,
        // then the cos/sin rows [16][D/2][2], CSR floats apart.  Lanes of one
        // head read the same pair of 16 different rows; the 4-float pad puts
        // those rows in different LDS banks.
        constexpr int CSR = D + 4, CS0 = 2 * D, STG = CS0 + 16 * CSR;
        float *stg = reinterpret_cast<float *>(&S.red[0][0][0]);
        constexpr int HW = HeadWords<WT, D>::N, NV = 18 * D / 4;
        // The last split also attends the block's own keys.  Their raw k rows
        // [16][D] (KRS bytes apart, padded like the cos/sin rows) and v^T
        // [D][16] of kv head h go to LDS after the staging area, 1 KB per wave
        // and load, in the same round trip as the q head.  Every wave then
        // reads them from LDS instead of loading them itself once q is done.
        constexpr int KRB = 16 * D * AB, RB = D * AB, KRS = RB + 16, NCH = 2 * KRB / 1024;
        static_assert(KRB % 1024 == 0 && NCH <= SR_CW, "block k / v rows fill at most one 1 KB load per wave");
        static_assert(sizeof(S.red) >= 4 * STG + 16 * KRS + KRB, "staging and block rows fit the reduction area");
        char *bk = reinterpret_cast<char *>(stg + STG), *bv = bk + 16 * KRS;
        // Loads below are unconditional (indices clamped into range; only the
        // LDS stores are guarded), so their values stay in registers and every
        // load of the round trip is in flight at once.
        u32x4 braw = u32x4{0, 0, 0, 0};
        if (it.last) {
            const char *ksrc = qkv + koff + (size_t)it.h * KRB, *vsrc = qkv + voff + (size_t)it.h * KRB;
            const int c = min(v, NCH - 1);
            braw = *reinterpret_cast<const u32x4 *>((c < NCH / 2 ? ksrc + 1024 * c : vsrc + 1024 * (c - NCH / 2)) + 16 * lane);
        }
        u32x4 qraw[HW];
        load_head_raw<WT, D>(qraw, qkv + (((size_t)(hq * 16 + r16) * 4 + g) * (D / 4)) * AB);
        {
            constexpr int NK = (NV + SR_CW * 64 - 1) / (SR_CW * 64);
            static_assert(NK <= 2, "staging takes at most two float4 per thread");
            auto src_of = [&](int i) -> const float4 * {
                const float *src = i < D / 4 ? ka()->L[l].g_q + 4 * i
                                 : i < D / 2 ? ka()->L[l].g_k + 4 * (i - D / 4) : SS.cs + 4 * (i - D / 2);
                return reinterpret_cast<const float4 *>(src);
            };
            auto put = [&](int i, float4 x) {
                const int f = 4 * (i - D / 2);      // cos/sin float index
                float *dst = i < D / 2 ? stg + 4 * i : stg + CS0 + (f / D) * CSR + f % D;
                if (i < NV) *reinterpret_cast<float4 *>(dst) = x;
            };
            const int i0 = (int)threadIdx.x, i1 = i0 + SR_CW * 64;
            const float4 sv0 = *src_of(min(i0, NV - 1));
            float4 sv1 = float4{0.f, 0.f, 0.f, 0.f};
            if constexpr (NK == 2) sv1 = *src_of(min(i1, NV - 1));
            put(i0, sv0);
            if constexpr (NK == 2) put(i1, sv1);
            if (it.last && v < NCH) {
                const int o = 1024 * v + 16 * lane;
                char *dst = v < NCH / 2 ? bk + (o / RB) * KRS + o % RB : bv + (o - KRB);
                *reinterpret_cast<u32x4 *>(dst) = braw;
            }
            cbar();
            if (lane == 0) lds_add(&S.stg, 1u);
            int spins = 0;
            while (lds_ld(&S.stg) < (unsigned)(SR_CW * (l + 1))) {
                if (lds_ld(&S.abort_)) return false;
                if (++spins > SPIN_LIMIT) { set_error(S); return false; }
                __builtin_amdgcn_s_sleep(1);
            }
        }
        // query fragments of q head hq, rows r16
        u32x4 qf[NC];
        {
            float x[NQV];
            decode_head<WT, D>(x, qraw);
            norm_rope<WT, D>(x, stg, stg + CS0 + r16 * CSR, SS.mscale * SS.qscale);
#pragma unroll
            for (int c = 0; c < NC; ++c) {
                if constexpr (WT == WT_F32) {
                    qf[c] = u32x4{__float_as_uint(x[4 * c]), __float_as_uint(x[4 * c + 1]), __float_as_uint(x[4 * c + 2]),
                                  __float_as_uint(x[4 * c + 3])};
                } else {
                    float t8[8];
#pragma unroll
                    for (int j = 0; j < 8; ++j) t8[j] = x[8 * c + j];
                    qf[c] = __builtin_bit_cast(u32x4, to_bf16x8(t8));
                }
            }
        }
        AttnState<WT, D> st;
        st.m = -1e30f;
        st.l = 0.f;
#pragma unroll
        for (int t = 0; t < NDT; ++t) st.o[t] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (it.last && actw) {
            // the block's own keys: normed + roped k and raw v of the b block
            // rows, read from the LDS copy.  Block key k takes position
            // 8 (k / 4) + k % 4 of a 32-key block, so every block key is a row
            // of key tile 0 (lane r16 holds key r16) and tile 1 is empty: one
            // head norm + rope per lane, and lane group g's positions
            // 8 g .. 8 g + 3 hold keys 4 g .. 4 g + 3 (the others are masked).
            u32x4 kraw[HW], vraw[NDT][A::VH];
            {
                const u32x4 *src = reinterpret_cast<const u32x4 *>(bk + r16 * KRS + g * (D / 4) * AB);
#pragma unroll
                for (int i = 0; i < HW; ++i) kraw[i] = src[i];
            }
#pragma unroll
            for (int t = 0; t < NDT; ++t) {
                const char *vsrc = bv + ((size_t)(16 * t + r16) * 16 + 4 * g) * AB;   // v^T row 16 t + r16, keys 4 g ..
                if constexpr (A::VH == 2) {
                    vraw[t][0] = *reinterpret_cast<const u32x4 *>(vsrc);
                    vraw[t][A::VH - 1] = u32x4{0, 0, 0, 0};
                } else {
                    const u32x2 x2 = *reinterpret_cast<const u32x2 *>(vsrc);
                    vraw[t][0] = u32x4{x2.x, x2.y, 0, 0};
                }
            }
            u32x4 kb[NC];
            {
                float x[NQV];
                decode_head<WT, D>(x, kraw);
                norm_rope<WT, D>(x, stg + D, stg + CS0 + r16 * CSR, SS.mscale);
                if (v == 0 && r16 < SS.b) {   // block K row to the cache (row len + r16)
                    constexpr int PQ = A::PQ;
                    char *kcache = SS.kc + (size_t)l * SS.kv_lstride;
                    const size_t rowb = (((size_t)it.h * SS.cap + SS.len + r16) * D) * A::KVB;
#pragma unroll
                    for (int c = 0; c < NC; ++c) {
                        const size_t off = rowb + (size_t)(4 * PQ * c + PQ * g) * A::KVB;
                        if constexpr (WT == WT_F32)
                            st16(kcache, off, u32x4{__float_as_uint(x[4 * c]), __float_as_uint(x[4 * c + 1]),
                                                    __float_as_uint(x[4 * c + 2]), __float_as_uint(x[4 * c + 3])});
                        else
                            st16(kcache, off, u32x4{bf2(x[8 * c], x[8 * c + 1]), bf2(x[8 * c + 2], x[8 * c + 3]),
                                                    bf2(x[8 * c + 4], x[8 * c + 5]), bf2(x[8 * c + 6], x[8 * c + 7])});
                    }
                }
#pragma unroll
                for (int c = 0; c < NC; ++c) {
                    if constexpr (WT == WT_F32) {
                        kb[c] = u32x4{__float_as_uint(x[4 * c]), __float_as_uint(x[4 * c + 1]), __float_as_uint(x[4 * c + 2]),
                                      __float_as_uint(x[4 * c + 3])};
                    } else {
                        kb[c] = u32x4{bf2(x[8 * c], x[8 * c + 1]), bf2(x[8 * c + 2], x[8 * c + 3]),
                                      bf2(x[8 * c + 4], x[8 * c + 5]), bf2(x[8 * c + 6], x[8 * c + 7])};
                    }
                }
            }
            auto kf = [&](int kt, int c) -> u32x4 { return kt == 0 ? kb[c] : u32x4{0, 0, 0, 0}; };
            auto vf = [&](int t, int hv) -> u32x4 { return vraw[t][hv]; };
            const int b4 = SS.b - 4 * g;
            auto valid = [&](int i) { return i < 4 && i < b4; };
            attn_block<WT, D>(st, qf, kf, vf, valid);
        }
        // cached keys, two blocks per softmax update (an odd last block alone)
        auto cache_blocks = [&](auto nbc, int blk) -> bool {
            constexpr int NB = decltype(nbc)::value;
            if (!ring_wait(S, cs, cs.seq + NB * A::SLOTS)) return false;
            const unsigned s0 = cs.seq;
            if (actw) {
                auto kf = [&](int b, int kt, int c) -> u32x4 {
                    const int kk = 8 * (r16 >> 2) + 4 * kt + (r16 & 3), cc = 4 * c + g;
                    const int idx = b * A::SLOTS * 8 + kk / A::KPP, pos = (kk % A::KPP) * A::CPR + (cc ^ A::kswz(kk));
                    return S.ring[(s0 + idx / 8) % SR_NSLOT][idx & 7][pos];
                };
                auto vf = [&](int b, int t, int hv) -> u32x4 {
                    const int idx = b * A::SLOTS * 8 + A::KP + t * A::VH + hv;
                    return S.ring[(s0 + idx / 8) % SR_NSLOT][idx & 7][lane];
                };
                const int kend = it.k_hi - (it.k_lo + 32 * blk) - 8 * g;
                auto valid = [&](int b, int i) { return i < kend - 32 * b; };
                attn_blocks<WT, D, NB>(st, qf, kf, vf, valid);
            }
            cs.seq = __builtin_amdgcn_readfirstlane(cs.seq + NB * A::SLOTS);
            ring_release(S, cs.seq);
            return true;
        };
        int blk = 0;
        for (; blk + 1 < it.nblk; blk += 2)
            if (!cache_blocks(std::integral_constant<int, 2>{}, blk)) return false;
        if (blk < it.nblk && !cache_blocks(std::integral_constant<int, 1>{}, blk)) return false;
        if (actw) {
            const int item = blockIdx.x;
            const int GQ = SS.G * 16, qi = v * 16 + r16;
            const size_t row = (size_t)item * GQ + qi;
            char *po = lb + SS.o_po;
            float *pml = (float *)(lb + SS.o_pml);
            // The wave's 16 rows of partial O are one contiguous block of
            // 16 D AB bytes.  Lane (r16, g) holds dims 16 t + 4 g .. + 3 of row
            // r16; stored as they are, an instruction writes 16 pieces of
            // 4 AB bytes, and such partial-line write-through stores cost
            // several microseconds per wave.  So the rows go through a 1 KB
            // LDS buffer of the wave, RPR rows at a time, and every store
            // instruction writes RPR whole rows.
            constexpr int RB2 = D * AB, RPR = 1024 / RB2, LPR = RB2 / 16;
            static_assert(1024 % RB2 == 0 && 16 % RPR == 0, "whole rows per 1 KB round");
            static_assert(sizeof(S.red) >= 4 * STG + 16 * KRS + KRB + SR_CW * 1024, "transpose buffers fit the reduction area");
            char *tb = bv + KRB + 1024 * v;
            char *wblk = po + ((size_t)item * GQ + v * 16) * RB2;
#pragma unroll
            for (int j = 0; j < 16 / RPR; ++j) {
                if (r16 / RPR == j) {
                    char *dst = tb + (r16 % RPR) * RB2 + 4 * g * AB;
#pragma unroll
                    for (int t = 0; t < NDT; ++t) {
                        if constexpr (AB == 4) *reinterpret_cast<f32x4 *>(dst + 16 * t * AB) = st.o[t];
                        else *reinterpret_cast<u32x2 *>(dst + 16 * t * AB) = u32x2{bf2(st.o[t][0], st.o[t][1]), bf2(st.o[t][2], st.o[t][3])};
                    }
                }
                cbar();
                const u32x4 x = *reinterpret_cast<const u32x4 *>(tb + 16 * lane);
                cbar();
                st16(wblk, (size_t)j * 1024 + 16 * lane, x);
            }
            if (g == 0) st8(pml, row * 8, u32x2{__float_as_uint(st.m), __float_as_uint(st.l)});
        }
        vm_wait();
    }
    if (v == 0) trace_at(p, 1);
    if (arrive(S)) {
        signal_phase();
        trace_at(p, 2);
        trace_all(p);
    }
    return true;
}

// ---------------------------------------------------------------------------
// merge phase: O[r, hq] = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s,
// written as o_proj input fragments
// ---------------------------------------------------------------------------
template <int WT, int D>
__device__ __forceinline__ bool merge_phase(SrLds &S, int l, unsigned p) {
    constexpr int AB = TR<WT>::AB;
    // one unit of work: a (row, q head) query and a 32-wide part of head_dim,
    // so every compute wave of the grid takes a share; lane (dg, sg) holds
    // 8 dims (group dg) of the splits sg, sg + NSG, ...
    constexpr int DP = 32, DQ = D / DP, NDG = DP / 8, NSG = 64 / NDG, NPS = SR_MAX_SPLITS / NSG;
    const int lane = lane_id(), v = wave_id();
    const int dg = lane % NDG, sg = lane / NDG;
    char *lb = layer_buf(l);
    const char *po = lb + SS.o_po;
    const float *pml = (const float *)(lb + SS.o_pml);
    char *of = lb + SS.o_of;
    const int GQ = SS.G * 16, ns = SS.nsplit;
    const int nu = SS.nkv * GQ * DQ;
    for (int u = blockIdx.x * SR_CW + v; u < nu; u += gridDim.x * SR_CW) {
        const int qq = u / DQ, dq = u - qq * DQ;
        const int h = qq / GQ, qi = qq - h * GQ;
        const int j = qi >> 4, r = qi & 15;
        const int hq = h * SS.G + j;
        float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        float L = 1.f;
        if (r < SS.b) {
            // every load (the splits' m, l and partial O) before the first use
            float2 ml = make_float2(-1e30f, 0.f);
            if (lane < ns) ml = *reinterpret_cast<const float2 *>(pml + ((size_t)(h * ns + lane) * GQ + qi) * 2);
            // the m of each split this lane sums, so its weight is computed
            // here rather than fetched from the lane that loaded it
            u32x4 raw[NPS][AB == 4 ? 2 : 1];
            float msp[NPS];
#pragma unroll
            for (int i = 0; i < NPS; ++i) {
                int sp = sg + NSG * i;
                sp = sp < ns ? sp : 0;
                msp[i] = pml[((size_t)(h * ns + sp) * GQ + qi) * 2];
                const size_t e = ((size_t)(h * ns + sp) * GQ + qi) * D + DP * dq + 8 * dg;
                raw[i][0] = *reinterpret_cast<const u32x4 *>(po + e * AB);
                if constexpr (AB == 4) raw[i][AB == 4 ? 1 : 0] = *reinterpret_cast<const u32x4 *>(po + e * AB + 16);
            }
            const float m = ml.x, lv = ml.y;
            const float M = wave_max(m);
            const float w = lane < ns ? __builtin_amdgcn_exp2f(m - M) : 0.f;
            L = wave_sum(w * lv);
#pragma unroll
            for (int i = 0; i < NPS; ++i) {
                const int sp = sg + NSG * i;
                const float ws = sp < ns ? __builtin_amdgcn_exp2f(msp[i] - M) : 0.f;
                if constexpr (AB == 4) {
                    const u32x4 a0 = raw[i][0], a1 = raw[i][AB == 4 ? 1 : 0];
                    acc[0] += ws * f_of(a0.x); acc[1] += ws * f_of(a0.y); acc[2] += ws * f_of(a0.z); acc[3] += ws * f_of(a0.w);
                    acc[4] += ws * f_of(a1.x); acc[5] += ws * f_of(a1.y); acc[6] += ws * f_of(a1.z); acc[7] += ws * f_of(a1.w);
                } else {
                    const u32x4 uu = raw[i][0];
#pragma unroll
                    for (int k = 0; k < 4; ++k) {
                        acc[2 * k] += ws * bf16_bits_to_f32(uu[k] & 0xFFFFu);
                        acc[2 * k + 1] += ws * __uint_as_float(uu[k] & 0xFFFF0000u);
                    }
                }
            }
        }
        static_assert(NDG == 4, "the split groups are the lanes that share lane % 4");
#pragma unroll
        for (int k = 0; k < 8; ++k) acc[k] = stride4_sum(acc[k]);
        if (sg == 0) {
            const float il = 1.f / L;
            const int c = hq * D + DP * dq + 8 * dg;
            put4<WT>(of, r, c, acc[0] * il, acc[1] * il, acc[2] * il, acc[3] * il);
            put4<WT>(of, r, c + 4, acc[4] * il, acc[5] * il, acc[6] * il, acc[7] * il);
        }
    }
    vm_wait();
    if (v == 0) trace_at(p, 1);
    if (arrive(S)) {
        signal_phase();
        trace_at(p, 2);
        trace_all(p);
    }
    return true;
}

// ---------------------------------------------------------------------------
// init and final phases
// ---------------------------------------------------------------------------
template <int WT, bool C>
__device__ __forceinline__ bool init_phase(SrLds &S) {
    constexpr bool HL = C && TR<WT>::AB == 2;
    const int lane = lane_id(), v = wave_id();
    const int ch = SS.ch, c0 = blockIdx.x * ch, H = SS.H, b = SS.b;
    for (int i = threadIdx.x; i < 16 * ch; i += SR_CW * 64) {
        const int r = i / ch, c = i - r * ch;
        float x = 0.f;
        if (r < b) x = SS.first ? SS.noise[(size_t)r * H + c0 + c] : SS.xsave[(size_t)r * H + c0 + c];
        S.xown[r][c] = x;
    }
    // cos / sin of the block positions (rows 0..b-1), angles in f64
    if (v == 0 && (int)blockIdx.x < b) {
        const int r = blockIdx.x, half = SS.d / 2;
        const double p = (double)SS.pos[r];
        for (int i = lane; i < half; i += 64) {
            double sv, cv;
            sincos(p * ka()->inv_freq[i], &sv, &cv);
            st8(SS.cs, ((size_t)r * half + i) * 8, u32x2{__float_as_uint((float)cv), __float_as_uint((float)sv)});
        }
    }
    vm_wait();
    if (arrive(S)) {
        if (SS.nl > 0) emit_input<WT, HL>(S, ka()->L[0].g_in + c0, layer_buf(0) + SS.o_xa, (float *)(layer_buf(0) + SS.o_ssa));
        else emit_input<WT, HL>(S, nullptr, nullptr, (float *)(layer_buf(0) + SS.o_ssa));
        signal_phase();
    }
    return true;
}

__device__ __forceinline__ void final_phase(SrLds &S, unsigned p) {
    const int ch = SS.ch, c0 = blockIdx.x * ch, H = SS.H, b = SS.b;
    if (!wait_rinv(S, p)) return;
    for (int i = threadIdx.x; i < 16 * ch; i += SR_CW * 64) {
        const int r = i / ch, c = i - r * ch;
        if (r < b) SS.out[(size_t)r * H + c0 + c] = SS.g_norm[c0 + c] * (S.xown[r][c] * S.rinv[r]);
    }
}

// ---------------------------------------------------------------------------
// the kernel
// ---------------------------------------------------------------------------
template <int WT, int D, bool C>
__device__ __forceinline__ bool compute_main(SrLds &S) {
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    unsigned E = 0;
    if (wave == 0) E = __builtin_amdgcn_readfirstlane(ldc_u(SS.ctr + SR_CTR_EPOCH));
    Cons cs{0u, 0u};
    const int nl = SS.nl, np = npl();
    if (!init_phase<WT, C>(S)) return false;
    unsigned p = 1;
    for (int l = 0; l < nl; ++l) {
        for (int i = 0; i < np; ++i, ++p) {
            if (!wait_phase(S, p, E)) return false;
            const int k = kind_at(i);
            bool ok;
            if (k == K_A) ok = attn_phase<WT, D>(S, cs, l, p);
            else if (k == K_M) ok = merge_phase<WT, D>(S, l, p);
            else {
                // a workgroup with a single tile runs the one-tile build (a
                // two-tile build measured slower: more code for the
                // instruction cache than it saves in the step loop)
                cs.seq = gemm_nt(k) == 1 ? gemm_phase<WT, D, C, 1>(k, l, p, cs.seq) : gemm_phase<WT, D, C, 0>(k, l, p, cs.seq);
                ok = cs.seq != ~0u;
            }
            if (!ok) return false;
        }
    }
    if (SS.last) {
        if (!wait_phase(S, p, E)) return false;
        final_phase(S, p);
    }
    return lds_ld(&S.abort_) == 0;
}

// The tail of this workgroup's gate|up weight run (the slots past what the
// ring can hold when the phase opens) into L2, so the loader's reads of those
// slots hit there: one 4-byte load per 128-byte line, all issued before the
// first wait.  The loaded values are folded into a word that is stored only
// under a condition no lane meets, which keeps the loads alive.
template <int WT>
__device__ __forceinline__ void prefetch_g_tail(SrLds &S, int l) {
    const long long run = pk_wg_bytes(WT, K_G, SS.H, SS.I, SS.qd, SS.cq, SS.ch, SS.ci);
    const long long lo = (long long)SR_NSLOT * SR_SLOT;
    if (run <= lo) return;
    const char *base = pk_run<WT>(K_G, l);
    const int lane = lane_id();
    constexpr int NPF = 16;                       // up to 16 slots past the ring
    unsigned v[NPF];
#pragma unroll
    for (int i = 0; i < NPF; ++i) {
        long long off = lo + (long long)i * SR_SLOT + 128 * lane;
        off = off < run ? off : lo;               // stays inside the run
        v[i] = *reinterpret_cast<const volatile unsigned *>(base + off);
    }
    unsigned x = 0;
#pragma unroll
    for (int i = 0; i < NPF; ++i) x ^= v[i];
    if (x == 0x9E3779B9u && lane == 64) S.sink_ = x;   // lane ids stop at 63
}

// Service wave: the rows' 1/rms of every norm-consuming phase (and of the
// final norm) as soon as the phase opens, from the producers' partial sums
// of squares, so no GEMM wave starts its share late.  When gate|up opens it
// first starts the L2 prefetch of the run's tail (the rows' scales are needed
// only by that phase's epilogue).
template <int WT>
__device__ __forceinline__ void service_main(SrLds &S) {
    const int nl = SS.nl, np = npl();
    unsigned p = 1;
    for (int l = 0; l < nl; ++l) {
        for (int i = 0; i < np; ++i, ++p) {
            const int k = kind_at(i);
            if (k == K_Q || k == K_G || k == K_DA || k == K_DM) {
                if (!wait_phase(S, p, 0u)) return;
                if (k == K_G) prefetch_g_tail<WT>(S, l);
                compute_rinv(S, (const float *)(layer_buf(l) + ((k == K_Q || k == K_DA) ? SS.o_ssa : SS.o_ssm)), p, SS.H);
            }
        }
    }
    if (SS.last && wait_phase(S, p, 0u)) compute_rinv(S, (const float *)(layer_buf(nl) + SS.o_ssa), p, SS.H);
}

// A launch that could not finish (a bounded wait expired, so some workgroup
// never arrived) leaves its result unmistakably invalid: every compute wave
// that gives up writes NaN over all b output rows (last launch of a round)
// or over the carried residual (earlier launches, whose successor then
// produces NaN as well), and the error word is set.  Valid values that other
// workgroups may still write cannot cover the columns of an aborted
// workgroup, whose final phase never runs.
__device__ __forceinline__ void poison_outputs() {
    const int n = SS.b * SS.H;
    float *dst = SS.last ? SS.out : SS.xsave;
    for (int i = lane_id(); i < n; i += 64) st4(dst, (size_t)i * 4, 0x7FC00000u);
    vm_wait();
}

template <int WT, int D, bool C>
__global__ __launch_bounds__(SR_THREADS, 1) void sround_kernel(SrArgs a) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    // Every device function reads the arguments through ka(), which assumes
    // the implicit arguments follow SrArgs directly in the kernel-argument
    // segment.  Check that against the segment pointer this launch received;
    // on a mismatch nothing below could be trusted, so the launch only marks
    // its output invalid (through the by-value argument) and sets the error
    // word.
    if ((const void *)ka() != (const void *)__builtin_amdgcn_kernarg_segment_ptr()) {
        if (threadIdx.x == 0) __hip_atomic_store(a.s.ctr + SR_CTR_ERR, 2u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        float *dst = a.s.last ? a.s.out : a.s.xsave;
        for (int i = threadIdx.x; i < a.s.b * a.s.H; i += SR_THREADS) dst[i] = __uint_as_float(0x7FC00000u);
        return;
    }
    if (threadIdx.x < 64) {
        if (lane < SR_CW) S.cons[lane] = 0;
        if (lane == 0) { S.pub = 0; S.phase = 0; S.rphase = 0; S.done = 0; S.stg = 0; S.abort_ = 0; }
    }
    __syncthreads();
    if (wave == SR_CW) {
        loader_main<WT, D>(S);
        if (lds_ld_nodep(&S.abort_)) stc_u(SS.ctr + SR_CTR_ERR, 1u);
        return;
    }
    if (wave == SR_CW + 1) {
        service_main<WT>(S);
        return;
    }
    // compute waves
    if (!compute_main<WT, D, C>(S)) {
        stc_u(SS.ctr + SR_CTR_ERR, 1u);
        poison_outputs();
    }
}

// one wave per workgroup writes that workgroup's slot runs of every layer
template <int WT>
__global__ __launch_bounds__(64) void sround_pack_kernel(SrArgs) {
    const int nl = SS.nl, np = npl();
    for (int l = 0; l < nl; ++l)
        for (int i = 0; i < np; ++i) {
            const int k = kind_at(i);
            if (k != K_A && k != K_M) pack_gemm<WT>(k, l);
        }
}

template <int WT, bool C>
hipError_t launch_d(const SrArgs &a, int nwg, hipStream_t s) {
    if (a.s.d == 64) hipLaunchKernelGGL((sround_kernel<WT, 64, C>), dim3(nwg), dim3(SR_THREADS), 0, s, a);
    else if constexpr (WT != WT_F32) hipLaunchKernelGGL((sround_kernel<WT, 128, C>), dim3(nwg), dim3(SR_THREADS), 0, s, a);
    else return hipErrorInvalidValue;
    return hipGetLastError();
}

template <int WT>
hipError_t launch_c(const SrArgs &a, int nwg, hipStream_t s) {
    return a.s.d2 ? launch_d<WT, true>(a, nwg, s) : launch_d<WT, false>(a, nwg, s);
}

}  // namespace

SrLayout sround_layout(int H, int I, int qd, int kvd, int nkv, int G, int d, int wt, int nwg, int d2) {
    const long long AB = wt == WT_F32 ? 4 : 2;
    long long off = 0;
    auto take = [&](long long bytes) { const long long o = off; off += (bytes + 255) / 256 * 256; return o; };
    SrLayout L;
    const int planes = d2 > 0 && AB == 2 ? 2 : 1;      // DFlash2: two-plane GEMM inputs
    L.xa = take(16LL * H * AB * planes);
    L.ssa = take(16LL * nwg * 4);
    L.qkv = take(16LL * (qd + 2 * kvd) * AB);
    L.po = take((long long)nkv * SR_MAX_SPLITS * G * 16 * d * AB);
    L.pml = take((long long)nkv * SR_MAX_SPLITS * G * 16 * 2 * 4);
    L.of = take(16LL * qd * AB);
    L.xm = take(16LL * H * AB * planes);
    L.ssm = take(16LL * nwg * 4);
    L.zf = take(16LL * I * AB * planes);
    L.da = take(16LL * 4 * (d2 > 0 ? d2 : 1) * 4);
    L.dm = take(16LL * 4 * (d2 > 0 ? d2 : 1) * 4);
    L.stride = off;
    return L;
}

// tiles of a run of m columns: 16-wide tiles plus an 8- and/or 4-wide rest
static int host_run_tiles(int m) {
    const int r = m & 15;
    return (m >> 4) + (r == 12 ? 2 : r ? 1 : 0);
}

// tiles that workgroup w gets of the concatenated q|k|v outputs
static int q_tiles(int w, int cq, int qd, int kvd) {
    const int c0 = w * cq, c1 = c0 + cq;
    const int a[3] = {0, qd, qd + kvd}, e[3] = {qd, qd + kvd, qd + 2 * kvd};
    int nt = 0;
    for (int s = 0; s < 3; ++s) {
        const int lo = c0 > a[s] ? c0 : a[s], hi = c1 < e[s] ? c1 : e[s];
        if (hi > lo) nt += host_run_tiles(hi - lo);
    }
    return nt;
}

int sround_nwg(int H, int I, int qd, int kvd, int wt, int d2, int cus) {
    const int nqkv = qd + 2 * kvd;
    const int kw = wt == WT_BF16 ? 32 : wt == WT_FP8 ? 64 : 16;
    const int nf = wt == WT_FP8 ? 4 : 8;
    for (const int K : {H, I, qd}) {
        if (K % kw) return 0;
        const int nkw = (K / kw + SR_CW - 1) / SR_CW;
        if ((nkw + nf - 1) / nf > 3) return 0;      // passes built per GEMM
    }
    // a group of 4 k steps of all of a workgroup's columns (one ring slot per
    // 4 columns) must fit in the ring beside the loader's in-flight slots
    const int max_cols = 4 * (SR_NSLOT - SR_DEPTH);
    for (int n = cus < 256 ? cus : 256; n >= 1; --n) {
        if (H % n || I % n || nqkv % n) continue;
        const int ch = H / n, ci = I / n, cq = nqkv / n;
        if (ch % 4 || ci % 4 || cq % 4 || ch > SR_MAXCH) continue;
        if (ch > max_cols || 2 * ci > max_cols || cq > max_cols) continue;
        if (host_run_tiles(ch) > SR_MAXT || 2 * host_run_tiles(ci) > SR_MAXT) continue;
        bool ok = true;
        for (int w = 0; w < n && ok; ++w) ok = q_tiles(w, cq, qd, kvd) <= SR_MAXT;
        if (!ok) continue;
        if (d2 > 0 && 4 * d2 > 16 * n) continue;
        return n;
    }
    return 0;
}

long long sround_pack_layer_bytes(int H, int I, int qd, int kvd, int wt, int d2, int nwg) {
    if (nwg <= 0) return 0;
    return pk_layer_off(wt, -1, H, I, qd, (qd + 2 * kvd) / nwg, H / nwg, I / nwg, nwg, d2);
}

hipError_t sround_pack_launch(const SrArgs &a, int wt, int nwg, hipStream_t s) {
    switch (wt) {
        case WT_F32: hipLaunchKernelGGL(sround_pack_kernel<WT_F32>, dim3(nwg), dim3(64), 0, s, a); break;
        case WT_BF16: hipLaunchKernelGGL(sround_pack_kernel<WT_BF16>, dim3(nwg), dim3(64), 0, s, a); break;
        default: hipLaunchKernelGGL(sround_pack_kernel<WT_FP8>, dim3(nwg), dim3(64), 0, s, a); break;
    }
    return hipGetLastError();
}

hipError_t sround_launch(const SrArgs &a, int wt, int nwg, hipStream_t s) {
    switch (wt) {
        case WT_F32: return launch_c<WT_F32>(a, nwg, s);
        case WT_BF16: return launch_c<WT_BF16>(a, nwg, s);
        default: return launch_c<WT_FP8>(a, nwg, s);
    }
}

}  // namespace dfl
