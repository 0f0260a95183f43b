// Paged GQA attention part kernel for few query vectors per KV head (rows * group < 16):
// decode and short verify windows, with VALU bf16 dot products.
//
// TensorFold PR #1620 (Reads bullet; the author's kernel-timing reply): decode reads keys
// through a page table, split over parts of the context that a merge kernel combines, and the
// page of a tile is looked up once per tile rather than once per key.
//
// Design for gfx950 (one wave64 per workgroup; one workgroup per (stream, KV head, chunk)):
//  * A batch is 16 load instructions per lane of 16 bytes each: 64 keys at D=128 (16 lanes
//    per row, 4 rows per instruction) or 16 keys at D=512.  The chunk's page-table entries are
//    read once into LDS; when P is a multiple of the batch, the whole batch lies in one page
//    and needs one lookup, otherwise each lane steps through its rows' pages without dividing.
//  * Loads are unconditional and always land inside the pool (absent pages read page 0), so
//    no load waits on a branch; V rows outside the chunk are zeroed when staged.
//  * K and V of a batch go through registers into LDS (rows padded by 16 bytes so that
//    lane-per-key reads are bank-conflict free); the next batch's loads stay in flight while
//    the current batch is computed (the barriers fence LDS only).
//  * QK: one lane per key (D=128) or four lanes per key (D=512, 128 channels each), all G*R
//    query vectors of the KV head against that key with v_dot2c_f32_bf16, so each K byte is
//    read from HBM once for the whole GQA group.
//  * Online softmax in the log2 domain with wave-uniform running max; masked keys are
//    selected out (never multiplied by zero), so NaN in unused slots cannot leak.
//  * PV: a lane owns 8 channels and every 4th key (D=128) or all 16 keys (D=512); the
//    weights of key pairs are packed to bf16 and V pairs interleaved so PV is also dot2.
//  * The workgroup writes an unnormalised partial (acc, m, l) per query vector.
#include <algorithm>

#include "internal.h"
#include "device_common.h"

namespace kvp {

template <int D>
struct ValuGeom {
    static constexpr int LPR = D / 8;         // lanes per row in a 16-byte-per-lane load
    static constexpr int RPI = 64 / LPR;      // rows per load instruction
    static constexpr int NB = 16 * RPI;       // keys per batch
    static constexpr int QL = 64 / NB;        // lanes per key in the QK stage
    static constexpr int SEG = D / QL;        // channels per QK lane
    static constexpr int RS = D + 8;          // LDS row stride (bf16 elements)
    static constexpr int TC = kTableCache;    // page-table entries cached per chunk
};

// Splits of one call, a function of the call's shape only.  Each stream is cut into n_splits
// even pieces (split_piece), one workgroup per (stream, KV head, piece).
//  * n_splits is a multiple of 8 when it is 8 or more: the dispatcher hands workgroups to the
//    8 XCDs round-robin in grid order, so piece i of every (stream, head) then lands on XCD
//    i mod 8 and every XCD reads the same number of bytes (measured: 8, 16, 24 or 32 pieces
//    beat 10 or 12 by 5 to 10 percent on the 12-stream decode).
//  * About 768 workgroups (three per CU), and pieces of at most about 2,560 keys (at d 128; the
//    same bytes at d 512): every split writes a partial (D + 2 floats per query vector) that
//    the merge reads back, which costs far more than its bytes, so fewer, longer pieces are
//    better while every CU stays busy; past about 2,560 keys, more workgroups in flight win
//    (part + merge: the 12-stream decode at 32k-40k keys takes 312.7 us with 16 pieces per
//    stream, 320.0 with 8; one stream at 40k keys 39.1 us with 96 pieces, 44.2 with 192).
//  * Pieces of at least 2 batches (short streams: a 2048-key decode at d 512 takes 12.4 us
//    with 2-batch pieces, 15.6 us with 4 and 13.9 us with 1).
// `span` bounds L - base over the call's streams.
ValuPlan valu_plan(int D, int NQ, int S, int Hkv, int span) {
    (void)NQ;
    ValuPlan p;
    p.align = valu_batch_keys(D);
    const int64_t groups = (int64_t)S * Hkv;
    int64_t n = (768 + groups - 1) / groups;
    const int64_t piece_keys = 2560 * 128 / D;
    n = std::max<int64_t>(n, ((int64_t)span + piece_keys - 1) / piece_keys);
    if (n >= 8) n = (n + 7) / 8 * 8;
    const int64_t most = ((int64_t)span + 2 * p.align - 1) / (2 * p.align);
    if (n > most) n = most;
    if (n < 1) n = 1;
    p.n_splits = (int)n;
    p.max_piece = split_piece(span, 0, p.n_splits, p.align);
    return p;
}

// Loads of one batch.  A batch is 16 load slots t per operand; slot t is rows t*RPI .. +RPI-1
// (16 bytes per lane).  Wave w owns the contiguous slots [w*NS, w*NS + NS) (NS even, so both
// keys of a PV pair (2 tp, 2 tp + 1) are loaded by one wave).  Every load reads inside the
// pool: an absent page reads page 0 and an out-of-range row keeps its slot; rows outside the
// chunk are zeroed when V is staged.  MODE is fixed per launch from P so that each loop is
// straight-line code.
template <int D, int NW>
struct BatchLoader {
    static constexpr int NS = ((16 + NW - 1) / NW + 1) / 2 * 2;   // slots per wave (even)
    const uint16_t *k_pages, *v_pages;
    const int32_t *trow;
    const int32_t *t_lds;      // page-table entries of the chunk from logical page idx0 on
    size_t page_elems, head_off;
    int P, idx0, lrow, wave, ring_pages, stride, num_pages;

    template <int MODE>
    __device__ __forceinline__ void load(int b, u32x4 (&kr)[NS], u32x4 (&vr)[NS]) const {
        constexpr int RPI = ValuGeom<D>::RPI;
        const int t0 = wave * NS;
        if constexpr (MODE == 0) {
            // the whole batch lies in one page: one lookup
            const int idx = b / P;
            const int pg = cached_page<ValuGeom<D>::TC>(t_lds, idx - idx0);
            const size_t base = (size_t)pg * page_elems + head_off + (size_t)(b - idx * P + lrow) * D;
#pragma unroll
            for (int i = 0; i < NS; ++i) {
                const int t = min(t0 + i, 15);
                kr[i] = stream_load(k_pages + base + (size_t)(t * RPI) * D);
                vr[i] = stream_load(v_pages + base + (size_t)(t * RPI) * D);
            }
        } else if constexpr (MODE == 1) {
            // rows straddle pages: step RPI rows at a time, crossing at most one boundary
            const int j0 = b + t0 * RPI + lrow;
            int idx = j0 / P;
            int off = j0 - idx * P;
#pragma unroll
            for (int i = 0; i < NS; ++i) {
                const int pg = cached_page<ValuGeom<D>::TC>(t_lds, idx - idx0);
                const size_t e = (size_t)pg * page_elems + head_off + (size_t)off * D;
                kr[i] = stream_load(k_pages + e);
                vr[i] = stream_load(v_pages + e);
                off += RPI;
                const bool wrap = off >= P;
                off = wrap ? off - P : off;
                idx += wrap ? 1 : 0;
            }
        } else {
            // tiny pages: divide per row and read the table from global memory
#pragma unroll
            for (int i = 0; i < NS; ++i) {
                const int t = min(t0 + i, 15);
                const int j = b + t * RPI + lrow;
                int idx = j / P;
                const int off = j - idx * P;
                if (ring_pages) idx %= ring_pages;
                const int tp = trow[min(idx, stride - 1)];
                const int pg = (idx < stride && (unsigned)tp < (unsigned)num_pages) ? tp : 0;
                const size_t e = (size_t)pg * page_elems + head_off + (size_t)off * D;
                kr[i] = stream_load(k_pages + e);
                vr[i] = stream_load(v_pages + e);
            }
        }
    }
};

// Query vectors per wave (VW) and waves per workgroup (NW = NQ / VW).  At d 512 with 8 vectors,
// one per wave (8 waves, two per SIMD): a d 512 decode is a short chain of dependent LDS reads
// and dot2s per batch, which a second wave on the SIMD hides (2,048-key decode over pages of
// 37, cold part kernel 11.9 -> 11.3 us; bytes unchanged).
template <int D, int NQ>
constexpr int valu_vw() { return D == 512 && NQ == 8 ? 1 : NQ % 2 == 0 && NQ <= 8 ? 2 : 4; }
template <int D, int NQ>
constexpr int valu_waves() { return NQ / valu_vw<D, NQ>(); }

// Load modes, fixed per launch from P (table_mode over batches of NB keys): 0 when P is a
// multiple of the batch, 1 when rows straddle pages but the chunk's table entries fit the LDS
// cache, 2 for tiny pages.
template <int D>
int valu_mode(int P, int chunk) {
    return table_mode(P, chunk, ValuGeom<D>::NB, ValuGeom<D>::RPI);
}

// At d 128 with 8 query vectors and one lookup per batch (MODE 0, pages a multiple of the
// batch: the headline) the kernel keeps four waves per SIMD (128 registers); the per-row
// lookups of MODEs 1 and 2 need a few more registers than that and would spill, so those modes
// have no occupancy floor.
template <int D, int G, int NQ, int MODE>
__global__ __launch_bounds__(64 * (valu_waves<D, NQ>())) __attribute__((amdgpu_waves_per_eu(D == 128 && NQ == 8 && MODE == 0 ? 4 : 1, 8))) void part_valu_kernel(const PartArgs a) {
    using Geo = ValuGeom<D>;
    constexpr int LPR = Geo::LPR, RPI = Geo::RPI, NB = Geo::NB, QL = Geo::QL, SEG = Geo::SEG;
    constexpr int RS = Geo::RS, TC = Geo::TC;
    constexpr int R = NQ / G;
    constexpr int VW = valu_vw<D, NQ>();                // query vectors per wave
    constexpr int NW = valu_waves<D, NQ>();
    using Loader = BatchLoader<D, NW>;
    constexpr int NS = Loader::NS;
    constexpr int PRS = 2 * D + 8;                      // V pair-row stride (bf16 elements): 528 bytes at
                                                        // D = 128 keeps the PV reads free of bank conflicts
    static_assert(NQ % G == 0 && NQ % VW == 0, "query vectors split evenly over the waves");

    // K tile (row-major, rows padded by 16 bytes for conflict-free lane-per-key reads), V tile
    // as key pairs (pair row pr = tp*RPI + lrow holds, per channel, the two keys 2tp*RPI + lrow
    // and (2tp+1)*RPI + lrow packed as one bf16x2 word), queries, weights, page table.
    __shared__ __attribute__((aligned(16))) uint16_t k_lds[NB * RS];
    __shared__ __attribute__((aligned(16))) uint16_t v_lds[(NB / 2) * PRS];
    __shared__ __attribute__((aligned(16))) uint16_t q_lds[NQ * RS];
    __shared__ __attribute__((aligned(16))) uint32_t p_lds[NW][(NB / 2) * VW];
    __shared__ int32_t t_lds[TC];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int split = blockIdx.x, kvh = blockIdx.y, s = blockIdx.z;
    const int32_t *trow = a.table + (size_t)s * a.stride;

    // All query vectors of this KV head go to LDS (vector v is row v / G, query head
    // kvh*G + v%G; wave w computes vectors [VW*w, VW*w + VW)), and so do the page-table entries
    // the workgroup reads (logical page idx0 + i at entry i; entries past the table or outside
    // the pool become -1).  When the stream's whole table fits the cache (a full layer of at
    // most TC pages), idx0 is 0 and the entries, like the queries, do not depend on the
    // stream's length: both are loaded before the length, so that the first K/V loads wait for
    // one round trip to memory, not two.
    constexpr int QN = NQ * (D / 8);                          // 16-byte query pieces
    constexpr int QPT = (QN + 64 * NW - 1) / (64 * NW);       // per thread
    constexpr int TPT = (TC + 64 * NW - 1) / (64 * NW);       // table entries per thread
    const bool whole = whole_table(MODE, a.ring_pages, a.stride);
    const int Lv = load_uniform_i32(a.seq_len + s);
    u32x4 qv[QPT];
    int tv[TPT];
#pragma unroll
    for (int k = 0; k < QPT; ++k) {
        const int i = tid + k * 64 * NW;
        if (i < QN) {
            const int v = i / (D / 8), c = i - (i / (D / 8)) * (D / 8);
            qv[k] = *reinterpret_cast<const u32x4 *>(a.q + ((size_t)(s * R + v / G) * a.Hq + kvh * G + (v % G)) * D + c * 8);
        }
    }
    if (whole) {
#pragma unroll
        for (int k = 0; k < TPT; ++k) {
            const int i = tid + k * 64 * NW;
            tv[k] = i < a.stride ? trow[i] : -1;
        }
    }
    const int L = kernel_len(__builtin_amdgcn_readfirstlane(Lv), a.max_len);
#pragma unroll
    for (int k = 0; k < QPT; ++k) {
        const int i = tid + k * 64 * NW;
        if (i < QN) {
            const int v = i / (D / 8), c = i - (i / (D / 8)) * (D / 8);
            *reinterpret_cast<u32x4 *>(q_lds + v * RS + c * 8) = qv[k];
        }
    }
    if (whole) {
#pragma unroll
        for (int k = 0; k < TPT; ++k) {
            const int i = tid + k * 64 * NW;
            if (i < TC) t_lds[i] = ((unsigned)tv[k] < (unsigned)a.num_pages) ? tv[k] : -1;
        }
    }

    const int W = a.window;
    if (L <= 0 || split >= a.n_splits) return;
    const KeyRange keys = valu_keys(L, R, W, a.n_splits, NB, a.chunk, split);
    if (keys.c0 >= L) return;
    const int kbeg = keys.kbeg, kend = keys.kend;

    const int lrow = lane / LPR;            // row inside a group of RPI rows (load and PV)
    const int lch = lane - lrow * LPR;      // 16-byte piece of the row
    const size_t page_elems = (size_t)a.Hkv * a.P * D;
    const size_t head_off = (size_t)kvh * a.P * D + (size_t)lch * 8;
    const int P = a.P;
    const int b_first = (kbeg / NB) * NB;

    // otherwise the chunk's entries, from the logical page of its first batch on
    const int idx0 = whole ? 0 : b_first / P;
    if (MODE != 2 && !whole) {
        for (int i = tid; i < TC; i += 64 * NW) {
            int idx = idx0 + i;
            if (a.ring_pages) idx %= a.ring_pages;
            int pg = -1;
            if (idx < a.stride) pg = trow[idx];
            t_lds[i] = ((unsigned)pg < (unsigned)a.num_pages) ? pg : -1;
        }
    }
    lds_fence();
    const Loader ld{a.k_pages, a.v_pages, trow, t_lds, page_elems, head_off, P, idx0, lrow, wave,
                    a.ring_pages, a.stride, a.num_pages};
    // decode with the row write fused (R = 1): the workgroup whose piece ends at the stream's
    // length writes the new K/V row of its KV head into the page slot of position L - 1, as
    // kv_rows_put does, before any of its loads; the barrier's workgroup-scope release and
    // acquire order that write before the loads of its last batch, which read the slot
    const bool put = a.k_new != nullptr && kend == L;
    if (put) {
        if (wave == 0 && lrow == 0) {
            const size_t src = ((size_t)s * a.Hkv + kvh) * D + (size_t)lch * 8;
            int idx = (L - 1) / P;
            const int off = (L - 1) - idx * P;
            if (a.ring_pages) idx %= a.ring_pages;
            // with the whole table cached, its entry is already in LDS (validated, -1 if bad)
            const int pg = idx < a.stride ? (whole ? t_lds[idx] : trow[idx]) : -1;
            if ((unsigned)pg < (unsigned)a.num_pages) {
                const size_t dst = (size_t)pg * page_elems + head_off + (size_t)off * D;   // head_off has the lane's 8 channels
                *reinterpret_cast<u32x4 *>(const_cast<uint16_t *>(a.k_pages) + dst) =
                    *reinterpret_cast<const u32x4 *>(a.k_new + src);
                *reinterpret_cast<u32x4 *>(const_cast<uint16_t *>(a.v_pages) + dst) =
                    *reinterpret_cast<const u32x4 *>(a.v_new + src);
            }
        }
        __syncthreads();
    }
    u32x4 kr[NS], vr[NS];

    float m_run[VW], l_run[VW], acc[VW][8];
#pragma unroll
    for (int v = 0; v < VW; ++v) {
        m_run[v] = -INFINITY;
        l_run[v] = 0.f;
#pragma unroll
        for (int c = 0; c < 8; ++c) acc[v][c] = 0.f;
    }

    const int nb = (kend - b_first + NB - 1) / NB;
    const int kk = (QL == 1) ? lane : (lane % NB);     // key of this lane in the QK stage
    const int seg = (QL == 1) ? 0 : (lane / NB);       // its channel segment
    const float scale_log2 = a.scale_log2;
    // keys every row of the call sees: up to row 0's own position, and inside every window
    // (with a tree-shaped window, only the keys before the window: a row may skip slot 0)
    const int all_hi = a.tree ? L - R : L - R + 1;
    const int win0 = L - R;                              // first slot of the window
    uint32_t anc[VW];                                    // ancestor bits of each vector's row
#pragma unroll
    for (int v = 0; v < VW; ++v) anc[v] = a.tree ? a.tree[s * R + (VW * wave + v) / G] : 0xFFFFFFFFu;
    const int all_lo = W > 0 ? L - W : 0;
    uint32_t *p_mine = p_lds[wave];
    const uint16_t *qb = q_lds + (VW * wave) * RS + seg * SEG;

    ld.template load<MODE>(b_first, kr, vr);
    for (int ib = 0; ib < nb; ++ib) {
        const int b = b_first + ib * NB;
        lds_fence();                        // every wave is done with the previous tiles
        const bool inside = b >= kbeg && b + NB <= kend;
#pragma unroll
        for (int i = 0; i < NS; i += 2) {
            const int t = wave * NS + i;
            if (NS * NW == 16 || t < 16) {
                const int row0 = t * RPI + lrow, row1 = row0 + RPI;
                *reinterpret_cast<u32x4 *>(k_lds + row0 * RS + lch * 8) = kr[i];
                *reinterpret_cast<u32x4 *>(k_lds + row1 * RS + lch * 8) = kr[i + 1];
                // at the chunk's edges, V rows outside it become zeros, so that a zero weight
                // never meets a NaN in an unused slot
                const uint32_t k0 = (inside || (b + row0 >= kbeg && b + row0 < kend)) ? 0xFFFFFFFFu : 0u;
                const uint32_t k1 = (inside || (b + row1 >= kbeg && b + row1 < kend)) ? 0xFFFFFFFFu : 0u;
                const u32x4 va = vr[i] & k0, vb = vr[i + 1] & k1;
                // interleave the pair: word c holds channel c of both keys
                const u32x4 p0 = u32x4{(va.x & 0xFFFFu) | (vb.x << 16), (va.x >> 16) | (vb.x & 0xFFFF0000u),
                                       (va.y & 0xFFFFu) | (vb.y << 16), (va.y >> 16) | (vb.y & 0xFFFF0000u)};
                const u32x4 p1 = u32x4{(va.z & 0xFFFFu) | (vb.z << 16), (va.z >> 16) | (vb.z & 0xFFFF0000u),
                                       (va.w & 0xFFFFu) | (vb.w << 16), (va.w >> 16) | (vb.w & 0xFFFF0000u)};
                uint16_t *dst = v_lds + ((t / 2) * RPI + lrow) * PRS + lch * 16;
                *reinterpret_cast<u32x4 *>(dst) = p0;
                *reinterpret_cast<u32x4 *>(dst + 8) = p1;
            }
        }
        if (ib + 1 < nb) ld.template load<MODE>(b + NB, kr, vr);     // a full batch ahead
        lds_fence();

        // ---- scores: this lane's key against this wave's query vectors
        float sc[VW];
#pragma unroll
        for (int v = 0; v < VW; ++v) sc[v] = 0.f;
        const uint16_t *krow = k_lds + kk * RS + seg * SEG;
#pragma unroll
        for (int cb = 0; cb < SEG / 8; ++cb) {
            const u32x4 kv = *reinterpret_cast<const u32x4 *>(krow + cb * 8);
#pragma unroll
            for (int v = 0; v < VW; ++v) {
                const u32x4 qv = *reinterpret_cast<const u32x4 *>(qb + v * RS + cb * 8);
                float x = sc[v];
                x = dot2_bf16(qv.x, kv.x, x);
                x = dot2_bf16(qv.y, kv.y, x);
                x = dot2_bf16(qv.z, kv.z, x);
                x = dot2_bf16(qv.w, kv.w, x);
                sc[v] = x;
            }
        }
        // the QL lanes of a key are lanes kk + NB j: sum their channel segments
        if constexpr (QL == 4) {
#pragma unroll
            for (int v = 0; v < VW; ++v) sc[v] = sc[v] + __shfl_xor(sc[v], 16);
        }
        if constexpr (QL >= 2) {
#pragma unroll
            for (int v = 0; v < VW; ++v) sc[v] = sc[v] + __shfl_xor(sc[v], 32);
        }

        // ---- online softmax (log2 domain).  A batch that every row sees whole needs no mask;
        // otherwise masked keys are selected out (never multiplied by zero).
        float x[VW];
        if (inside && b + NB <= all_hi && b >= all_lo) {
#pragma unroll
            for (int v = 0; v < VW; ++v) x[v] = sc[v] * scale_log2;
        } else {
            const int j = b + kk;
#pragma unroll
            for (int v = 0; v < VW; ++v) {
                const int pr = L - R + (VW * wave + v) / G;   // position of this vector's row
                const int lor = W > 0 ? pr - W + 1 : 0;
                const int t = j - win0;                     // window slot of the key, if >= 0
                const bool vis = j >= kbeg && j < kend && j <= pr && j >= lor &&
                                 (t < 0 || ((anc[v] >> (t & 31)) & 1u));
                x[v] = vis ? sc[v] * scale_log2 : -INFINITY;
            }
        }
        // The running max moves only when a score of the batch exceeds it (rare after the first
        // batches); only then are the wave maxima reduced and the sums rescaled.
        uint64_t over = 0;
#pragma unroll
        for (int v = 0; v < VW; ++v) over |= __builtin_amdgcn_ballot_w64(x[v] > m_run[v]);
        if (over) {
#pragma unroll
            for (int v = 0; v < VW; ++v) {
                const float mn = fmaxf(m_run[v], wave_max(x[v]));
                const float al = (mn == -INFINITY) ? 1.f : fast_exp2(m_run[v] - mn);
                m_run[v] = mn;
                l_run[v] *= al;
#pragma unroll
                for (int c = 0; c < 8; ++c) acc[v][c] *= al;
            }
        }
        float pv[VW];
#pragma unroll
        for (int v = 0; v < VW; ++v) {
            pv[v] = (x[v] == -INFINITY) ? 0.f : fast_exp2(x[v] - m_run[v]);
            l_run[v] += (seg == 0) ? pv[v] : 0.f;
        }
        // pack (p[key], p[key + RPI]) as bf16 pairs for the PV dot2
        {
            uint32_t w[VW];
#pragma unroll
            for (int v = 0; v < VW; ++v) w[v] = pack_bf16x2(pv[v], __shfl_down(pv[v], RPI));
            const bool writer = seg == 0 && ((kk / RPI) & 1) == 0;
            const int pid = (kk / (2 * RPI)) * RPI + (kk % RPI);
            if (writer) {
                if constexpr (VW == 4)
                    *reinterpret_cast<u32x4 *>(p_mine + pid * VW) = u32x4{w[0], w[1], w[2], w[3]};
                else if constexpr (VW == 2)
                    *reinterpret_cast<uint2 *>(p_mine + pid * VW) = make_uint2(w[0], w[1]);
                else
                    p_mine[pid] = w[0];
            }
        }
        wave_lds_fence();

        // ---- PV: lane owns channels lch*8..+8 of the key pairs (2tp*RPI + lrow, +RPI)
#pragma unroll
        for (int tp = 0; tp < 8; ++tp) {
            const int pr = tp * RPI + lrow;
            const uint16_t *src = v_lds + pr * PRS + lch * 16;
            const u32x4 p0 = *reinterpret_cast<const u32x4 *>(src);
            const u32x4 p1 = *reinterpret_cast<const u32x4 *>(src + 8);
            const uint32_t vp[8] = {p0.x, p0.y, p0.z, p0.w, p1.x, p1.y, p1.z, p1.w};
            uint32_t pw[VW];
            if constexpr (VW == 4) {
                const u32x4 pp = *reinterpret_cast<const u32x4 *>(p_mine + pr * VW);
                pw[0] = pp.x; pw[1] = pp.y; pw[2] = pp.z; pw[3] = pp.w;
            } else if constexpr (VW == 2) {
                const uint2 pp = *reinterpret_cast<const uint2 *>(p_mine + pr * VW);
                pw[0] = pp.x; pw[1] = pp.y;
            } else {
                pw[0] = p_mine[pr];
            }
#pragma unroll
            for (int v = 0; v < VW; ++v)
#pragma unroll
                for (int c = 0; c < 8; ++c) acc[v][c] = dot2_bf16(pw[v], vp[c], acc[v][c]);
        }
    }

    // ---- epilogue: combine lanes, write this wave's partials of the chunk
    float l_tot[VW];
#pragma unroll
    for (int v = 0; v < VW; ++v) l_tot[v] = wave_sum(l_run[v]);
    // the RPI lanes of a channel block are lanes lch + LPR j: sum their key rows
    if constexpr (RPI == 4) {
#pragma unroll
        for (int v = 0; v < VW; ++v)
#pragma unroll
            for (int c = 0; c < 8; ++c) acc[v][c] = acc[v][c] + __shfl_xor(acc[v][c], 16);
    }
    if constexpr (RPI >= 2) {
#pragma unroll
        for (int v = 0; v < VW; ++v)
#pragma unroll
            for (int c = 0; c < 8; ++c) acc[v][c] = acc[v][c] + __shfl_xor(acc[v][c], 32);
    }
#pragma unroll
    for (int i = 0; i < VW; ++i) {
        if ((i % RPI) != lrow) continue;
        const int v = VW * wave + i;
        const int r = v / G, h = kvh * G + (v % G);
        const size_t slot = (((size_t)(s * R + r) * a.Hq + h) * a.n_splits + split);
        float4 *dst = reinterpret_cast<float4 *>(a.ws_acc + slot * D + lch * 8);
        dst[0] = make_float4(acc[i][0], acc[i][1], acc[i][2], acc[i][3]);
        dst[1] = make_float4(acc[i][4], acc[i][5], acc[i][6], acc[i][7]);
        if (lch == 0) *reinterpret_cast<float2 *>(a.ws_ml + slot * 2) = make_float2(m_run[i], l_tot[i]);
    }
}

int valu_batch_keys(int D) {
    return D == 512 ? ValuGeom<512>::NB : D == 256 ? ValuGeom<256>::NB : ValuGeom<128>::NB;
}
int valu_rows_per_load(int D) {
    return D == 512 ? ValuGeom<512>::RPI : D == 256 ? ValuGeom<256>::RPI : ValuGeom<128>::RPI;
}
int valu_table_mode(int D, int P, int chunk) {
    return D == 512 ? valu_mode<512>(P, chunk) : D == 256 ? valu_mode<256>(P, chunk) : valu_mode<128>(P, chunk);
}
template <int D, int NQ>
static void load_shape(int *waves, int *slots) {
    *waves = valu_waves<D, NQ>();
    *slots = BatchLoader<D, valu_waves<D, NQ>()>::NS;
}
void valu_load_shape(int D, int NQ, int *waves, int *slots_per_wave) {
    *waves = *slots_per_wave = 0;
#define KVP_SHAPE(d)                                           \
    if (D == d && NQ == 4) load_shape<d, 4>(waves, slots_per_wave);   \
    if (D == d && NQ == 8) load_shape<d, 8>(waves, slots_per_wave);   \
    if (D == d && NQ == 12) load_shape<d, 12>(waves, slots_per_wave);
    KVP_SHAPE(128) KVP_SHAPE(256) KVP_SHAPE(512)
#undef KVP_SHAPE
}

bool valu_supported(int D, int G, int NQ) {
    if (D != 128 && D != 256 && D != 512) return false;
    if (G == 4) return NQ == 4 || NQ == 8 || NQ == 12;
    if (G == 8) return NQ == 8;
    if (G == 12) return NQ == 12;
    return false;
}

template <int D, int G, int NQ>
static hipError_t launch_one(const PartArgs &a, int S, hipStream_t st) {
    constexpr int NW = valu_waves<D, NQ>();
    const dim3 grid(a.n_splits, a.Hkv, S);
    if (a.chunk % ValuGeom<D>::NB != 0) return hipErrorInvalidValue;
    switch (valu_mode<D>(a.P, a.chunk)) {
        case 0: hipLaunchKernelGGL((part_valu_kernel<D, G, NQ, 0>), grid, dim3(64 * NW), 0, st, a); break;
        case 1: hipLaunchKernelGGL((part_valu_kernel<D, G, NQ, 1>), grid, dim3(64 * NW), 0, st, a); break;
        default: hipLaunchKernelGGL((part_valu_kernel<D, G, NQ, 2>), grid, dim3(64 * NW), 0, st, a); break;
    }
    return hipGetLastError();
}

hipError_t launch_part_valu(int D, int G, int NQ, const PartArgs &a, int S, hipStream_t st) {
#define KVP_VALU_CASE(d, g, nq) \
    if (D == d && G == g && NQ == nq) return launch_one<d, g, nq>(a, S, st);
    KVP_VALU_CASE(128, 4, 4) KVP_VALU_CASE(128, 4, 8) KVP_VALU_CASE(128, 4, 12) KVP_VALU_CASE(128, 8, 8)
    KVP_VALU_CASE(128, 12, 12)
    KVP_VALU_CASE(256, 4, 4) KVP_VALU_CASE(256, 4, 8) KVP_VALU_CASE(256, 4, 12) KVP_VALU_CASE(256, 8, 8)
    KVP_VALU_CASE(256, 12, 12)
    KVP_VALU_CASE(512, 4, 4) KVP_VALU_CASE(512, 4, 8) KVP_VALU_CASE(512, 4, 12) KVP_VALU_CASE(512, 8, 8)
    KVP_VALU_CASE(512, 12, 12)
#undef KVP_VALU_CASE
    return hipErrorInvalidValue;
}

}  // namespace kvp
