// Internal declarations shared by the host API and the kernel translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace kvp {

// Arguments of the row-write kernel.
struct RowsArgs {
    uint16_t *k_pages;
    uint16_t *v_pages;
    const uint16_t *k_new;
    const uint16_t *v_new;
    const int32_t *table;
    const int32_t *seq_len;
    int num_pages, P, Hkv, D;
    int S, R, stride, ring_pages;
};

// Arguments of the split-context part kernels (VALU and MFMA).  Each workgroup handles one
// (stream, KV head, key chunk[, query tile]) and writes an unnormalised partial result:
// acc[D] plus (m, l) per query vector, m in log2 units.
struct PartArgs {
    const uint16_t *k_pages;
    const uint16_t *v_pages;
    const int32_t *table;
    const int32_t *seq_len;
    const uint16_t *q;
    float *ws_acc;   // [S][R][Hq][n_splits][D]
    float *ws_ml;    // [S][R][Hq][n_splits][2]
    int num_pages, P, Hkv, stride, ring_pages;
    int R, Hq, window, n_splits;
    int chunk;         // keys per split (a multiple of the kernel's key tile)
    int S, tiles;      // streams and query tiles per (stream, KV head) of an MFMA call
    int per_xcd;       // MFMA work items per XCD (the grid is 8 * per_xcd workgroups)
    const uint32_t *tree;  // NULL, or [S][R] ancestor bits of a tree-shaped verify window:
                           // row r sees window slot i (i <= r) only if bit i is set
    uint16_t *out;     // MFMA with n_splits == 1: bf16 output [S][R][Hq][D] written directly
    int direct;        //   (1), with no partials and no merge; 0: partials into the workspace
    float scale_log2;  // scale * log2(e)
    // decode with the row write fused: k_new/v_new [S][1][Hkv][D] (NULL: no row to write)
    const uint16_t *k_new;
    const uint16_t *v_new;
};

// Arguments of the page copy (kept states): page dst[i] gets page src[i], K and V.
struct CopyArgs {
    uint16_t *k_pages;
    uint16_t *v_pages;
    const int32_t *src;
    const int32_t *dst;
    int n, num_pages;
    size_t page_elems;   // Hkv * P * D
};

struct MergeArgs {
    const float *ws_acc;
    const float *ws_ml;
    const int32_t *seq_len;
    uint16_t *out;   // [S][R][Hq][D]
    int S, R, Hq, D, window, n_splits, chunk;
    int even;        // 1: splits are the even pieces of split_piece(); 0: chunks of `chunk` keys
    int align;       // piece granularity of the even split
};

// The even split of one stream's keys: the positions a call can see, [lo, L) with lo the
// lowest first visible key over the call's rows, start at base = lo rounded down to `align`;
// piece i covers [base + i piece, base + (i + 1) piece) with piece = ceil((L - base) / n)
// rounded up to `align`.  Every stream gets n pieces of about equal length, so workgroup i of
// every (stream, head), which the dispatcher places on XCD i mod 8, reads the same number of
// bytes.  Depends on (L, R, window, n, align) only.
__host__ __device__ inline int split_base(int L, int R, int window, int align) {
    const int lo = window > 0 ? (L - R - window + 1 > 0 ? L - R - window + 1 : 0) : 0;
    return (lo / align) * align;
}
__host__ __device__ inline int split_piece(int L, int base, int n, int align) {
    const int per = (L - base + n - 1) / n;
    return (per + align - 1) / align * align;
}

// Splits of a VALU call (about one round of resident workgroups) and the longest piece.
struct ValuPlan {
    int n_splits, max_piece, align;
};
ValuPlan valu_plan(int D, int NQ, int S, int Hkv, int span);
bool valu_supported(int D, int G, int NQ);
bool mfma_supported(int D, int G, int R);

// Launch shape of the MFMA part kernel for one call: query-column blocks per wave (tile of
// 64 * qw query vectors), query tiles per (stream, KV head), keys per split.  A function of
// the call's shape only.
struct MfmaPlan {
    int qw, tiles, chunk;
    int ks;       // key sub-tiles per step (2: 8-wave workgroups, D = 128 only)
    bool direct;  // one split per query tile, covering exactly the keys its rows see; the bf16
                  // output is written by the part kernel (chunk then bounds that key span)
};
MfmaPlan mfma_plan(int D, int G, int R, int S, int Hkv, int P, int max_seq_len, int window);

hipError_t launch_rows_put(const RowsArgs &a, hipStream_t st);
hipError_t launch_part_valu(int D, int G, int NQ, const PartArgs &a, int S, hipStream_t st);
hipError_t launch_part_mfma(int D, int G, const MfmaPlan &p, const PartArgs &a, int S, hipStream_t st);
hipError_t launch_merge(const MergeArgs &a, hipStream_t st);
hipError_t launch_pages_copy(const CopyArgs &a, hipStream_t st);

// Device address and size of the current GPU's static scratch array (looked up on the first
// call per GPU, with that GPU current).
hipError_t static_scratch(void **ptr, size_t *bytes);

}  // namespace kvp
