// Device-side view of one sequence's draft KV cache, contiguous or paged
// ([memra dflash module] "DflashKv": per-layer ctx K (normed + roped) and
// V (raw); [atlas dflash_head] "DflashProposerState": one paged cache per
// drafter layer, one block table shared by every layer).
//
// Storage of one layer, with P rows per page:
//   K [pages][nkv][P][d]      V [pages][nkv][P / 32][d][32]
// (V transposed per tile of 32 rows, so that a 32-key block's V is one
// contiguous run and P.V streams contiguous keys).  A contiguous cache is
// the one-page case: P = capacity, no block table.  Logical row r of a
// sequence lives in physical page table[r / P] (page 0 without a table), at
// row r % P.  P is a multiple of 64, so an aligned block of 32 keys never
// straddles a page.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dfl {

struct KvView {
    char *k, *v;              // layer 0 bases
    long long lstride;        // bytes per layer, K and V alike
    const int32_t *table;     // device block table (logical page -> physical page), or nullptr
    int page_rows;            // P
    int pool_pages;           // physical pages per layer (1 when contiguous)
    int esize;                // bytes per stored value (4 f32, 2 bf16)
};

// physical page of logical row r; out-of-range table entries are clamped
// into the pool, so a bad table gives wrong values but never a wild access
__device__ __forceinline__ int kv_page(const KvView &v, int r) {
    if (!v.table) return 0;
    const int p = v.table[r / v.page_rows];
    return p < 0 ? 0 : p >= v.pool_pages ? v.pool_pages - 1 : p;
}

// byte offsets within a layer
__device__ __forceinline__ size_t kv_k_off(const KvView &v, int page, int nkv, int h, int r, int d, int dd) {
    return ((((size_t)page * nkv + h) * v.page_rows + (r % v.page_rows)) * d + dd) * v.esize;
}
__device__ __forceinline__ size_t kv_v_off(const KvView &v, int page, int nkv, int h, int r, int d, int dd) {
    const int rp = r % v.page_rows;
    return (((((size_t)page * nkv + h) * (v.page_rows / 32) + rp / 32) * d + dd) * 32 + (rp % 32)) * v.esize;
}

}  // namespace dfl
