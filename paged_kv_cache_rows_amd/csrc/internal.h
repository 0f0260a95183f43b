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
    int max_len;       // the call's max_seq_len (device lengths are read through kernel_len)
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
    int max_len;       // the call's max_seq_len (device lengths are read through kernel_len)
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
    int max_len;     // the call's max_seq_len (device lengths are read through kernel_len)
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

// A stream's length as every kernel reads it.  A device length above the call's max_seq_len
// is a caller error (the optional host check refuses it); the kernels then take it as
// max_seq_len, so that every index they derive from it stays inside the table entries, key
// ranges and workspace the host planned for the call.
__host__ __device__ inline int kernel_len(int L, int max_len) { return L < max_len ? L : max_len; }

// Page-table entries a part workgroup caches in LDS.
constexpr int kTableCache = 160;

// How a part kernel finds the pages of its keys, fixed per launch from the page size P and the
// longest run of keys a workgroup reads (`chunk`, read in steps of `unit` keys):
//  0: the run's table entries are cached in LDS and a step never straddles a page (one lookup
//     per step);
//  1: entries cached, one lookup per row (the rows one load instruction covers straddle at
//     most one page boundary: P >= min_page);
//  2: one lookup per row in the table in memory (tiny pages, or runs too long to cache).
__host__ __device__ inline int table_mode(int P, int chunk, int unit, int min_page) {
    const bool cached = ((int64_t)chunk + unit) / P + 2 <= kTableCache;
    if (cached && P % unit == 0) return 0;
    if (cached && P >= min_page) return 1;
    return 2;
}

// With a full layer whose whole table fits the cache, the cached entries are the stream's
// logical pages from 0 on; otherwise they start at the logical page of the workgroup's first
// step.
__host__ __device__ inline bool whole_table(int mode, int ring_pages, int stride) {
    return mode != 2 && ring_pages == 0 && stride <= kTableCache;
}

// Keys of one workgroup: its run starts at c0; it reads [kbeg, kend), the keys of the run that
// the call's rows see.  kbeg >= kend: nothing to read.
struct KeyRange {
    int c0, kbeg, kend;
};

// Piece `split` of a VALU call for a stream of length L >= 1: the even piece of split_piece(),
// cut to the positions [lo, L) the call's rows see and to the host's longest piece `chunk`
// (which it never exceeds for L <= max_seq_len).  c0 >= L: the piece is past the stream.
__host__ __device__ inline KeyRange valu_keys(int L, int R, int window, int n_splits, int align, int chunk,
                                             int split) {
    const int lo = window > 0 ? (L - R - window + 1 > 0 ? L - R - window + 1 : 0) : 0;
    const int base = split_base(L, R, window, align);
    const int piece = split_piece(L, base, n_splits, align);
    KeyRange k;
    k.c0 = base + split * piece;
    k.kbeg = k.c0 > lo ? k.c0 : lo;
    const int run = piece < chunk ? piece : chunk;
    k.kend = k.c0 + run < L ? k.c0 + run : L;
    return k;
}

// Split `split` of an MFMA query tile whose vectors hold rows r_first .. r_last of the window
// (positions L - R + r): `chunk` absolute positions counted from the first chunk any row of the
// stream sees, or, for a direct call (one split), the keys from the tile's first visible one,
// whose chunk covers every key the tile's rows see; cut to the keys those rows see.
__host__ __device__ inline KeyRange mfma_keys(int L, int R, int window, int chunk, int split, bool direct,
                                             int r_first, int r_last) {
    const int p_first = L - R + r_first, p_last = L - R + r_last;
    const int lo_stream = window > 0 ? (L - R - window + 1 > 0 ? L - R - window + 1 : 0) : 0;
    const int lo_tile = window > 0 ? (p_first - window + 1 > 0 ? p_first - window + 1 : 0) : 0;
    KeyRange k;
    k.c0 = direct ? lo_tile : (lo_stream / chunk + split) * chunk;
    k.kbeg = k.c0 > lo_tile ? k.c0 : lo_tile;
    k.kend = k.c0 + chunk < p_last + 1 ? k.c0 + chunk : p_last + 1;
    return k;
}

// The splits the merge combines for the row at position pos >= 0 of a stream of length L: the
// ones holding its keys [max(0, pos - window + 1), pos], as [first, end) (end <= n_splits).
struct SplitSpan {
    int first, end;
};
__host__ __device__ inline SplitSpan row_splits(int L, int R, int window, int pos, int n_splits, int chunk,
                                               bool even, int align) {
    const int lo_r = window > 0 ? (pos - window + 1 > 0 ? pos - window + 1 : 0) : 0;
    SplitSpan sp;
    if (even) {
        const int base = split_base(L, R, window, align);
        const int piece = split_piece(L, base, n_splits, align);
        sp.first = (lo_r - base) / piece;
        sp.end = (pos - base) / piece + 1;
    } else {
        const int lo_stream = window > 0 ? (L - R - window + 1 > 0 ? L - R - window + 1 : 0) : 0;
        const int first = lo_stream / chunk;
        sp.first = lo_r / chunk - first;
        sp.end = pos / chunk - first + 1;
    }
    if (sp.end > n_splits) sp.end = n_splits;
    return sp;
}

// Splits of a VALU call (about one round of resident workgroups) and the longest piece.
struct ValuPlan {
    int n_splits, max_piece, align;
};
ValuPlan valu_plan(int D, int NQ, int S, int Hkv, int span);
bool valu_supported(int D, int G, int NQ);
bool mfma_supported(int D, int G, int R);

// Key steps of the part kernels (VALU: keys per batch and rows per load instruction; MFMA: keys
// per tile) and the page lookup mode (table_mode) a launch of each uses.
int valu_batch_keys(int D);
int valu_rows_per_load(int D);
int valu_table_mode(int D, int P, int chunk);
// VALU waves per workgroup and load slots per wave (RPI rows each) for NQ query vectors at head
// dim D.
void valu_load_shape(int D, int NQ, int *waves, int *slots_per_wave);
int mfma_tile_keys(int D);
int mfma_table_mode(int D, int P, int chunk);

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

// Launch plan of one attention call, a function of its shape only (no device data): which part
// kernel, keys per split (VALU: the longest even piece), splits per (stream, KV head).
struct CallPlan {
    bool mfma;
    int chunk, n_splits;
    bool even;   // VALU: even pieces per stream; MFMA: absolute chunks of `chunk` keys
    int align;   // piece granularity of the even split (1 for MFMA)
    MfmaPlan mp;
};
// false when no kernel serves (D, G, R); the shape is otherwise assumed valid (R >= 1,
// max_seq_len >= R, window >= 0).
bool call_plan(int D, int G, int R, int S, int Hkv, int P, int max_seq_len, int window, CallPlan *p);

hipError_t launch_rows_put(const RowsArgs &a, hipStream_t st);
hipError_t launch_part_valu(int D, int G, int NQ, const PartArgs &a, int S, hipStream_t st);
hipError_t launch_part_mfma(int D, int G, const MfmaPlan &p, const PartArgs &a, int S, hipStream_t st);
hipError_t launch_merge(const MergeArgs &a, hipStream_t st);
hipError_t launch_pages_copy(const CopyArgs &a, hipStream_t st);

// Device address and size of the current GPU's static scratch array (looked up on the first
// call per GPU, with that GPU current).
hipError_t static_scratch(void **ptr, size_t *bytes);

}  // namespace kvp
