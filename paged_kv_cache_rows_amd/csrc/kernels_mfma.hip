// Paged GQA attention part kernel for many query vectors per KV head (rows * group >= 16):
// speculative verify windows and prompt chunks, on MFMA.
//
// TensorFold PR #1620, opening description (Reads bullet: prompts and drafted verify read keys
// through the page table) and TensorFold PR #2730 (verify windows of up to eight rows).
//
// Design for gfx950.  A workgroup of 4 waves takes a tile of 64 * QW query vectors of one KV
// head (rows x GQA heads, row-major) and one chunk of keys; each wave owns QW blocks of 16
// query vectors.
//  * K and V tiles of KT keys are loaded through the page table (one lookup per tile when the
//    page size is a multiple of KT, else per 16-byte piece from a copy of the chunk's table
//    entries in LDS) into registers, one tile ahead, then staged in LDS: K row-major, V
//    transposed into 8-byte units of 4 keys of one channel.  Each thread loads 4 (or 8)
//    consecutive keys of one 8-channel block, so the transpose is a register permute and the
//    unit stores are 8 bytes wide; the units are XOR-swizzled so that both the stores and the
//    MFMA operand reads touch every LDS bank equally.
//  * Scores are computed transposed, S^T = K Q^T, with v_mfma_f32_16x16x32_bf16: the wave's
//    queries are the B operand, held in registers for the whole chunk, and each K fragment read
//    from LDS feeds QW MFMAs.  In the C layout a lane owns one query column and 4 keys per
//    16-key block, which is exactly the B-operand layout that O^T = V^T P^T needs, so the
//    softmax weights feed the second MFMA from registers.
//  * Online softmax per query column in the log2 domain; masked keys are selected out and V
//    units outside the chunk are zeroed, so NaN in unused slots never reaches the sums.  Tiles
//    that every column sees in full skip the mask.
//  * The workgroup writes an unnormalised partial (acc, m, l) per query vector, merged later
//    in fixed chunk order.
#include <algorithm>

#include "internal.h"
#include "device_common.h"

namespace kvp {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

template <int D>
struct MfmaGeom {
    static constexpr int KT = D == 128 ? 64 : 32;       // keys per tile
    static constexpr int KRS = D + 16;                  // K tile row stride (bf16): 288 or 1056 bytes, so
                                                        // that an MFMA operand read is free of bank conflicts
    static constexpr int CB = D / 8;                    // 16-byte channel blocks per row
    static constexpr int NT = 256;                      // threads
    static constexpr int KPT = KT * CB / NT;            // keys per thread per tile (4 or 8)
    static constexpr int UPR = KT / 4;                  // V^T units (4 keys) per channel
    static constexpr int RPS = 32 / UPR;                // channels per 32-unit (256-byte) row
    static constexpr int TC = 160;                      // cached page-table entries
};

static_assert(MfmaGeom<128>::KPT == 4 && MfmaGeom<512>::KPT == 8, "thread tiling");

// Position of the V^T unit (channel ch, keys 4 kg .. 4 kg + 3) in units of 8 bytes.  The
// 32 units of a 256-byte row are permuted by an XOR of the row number's bits, chosen so that
// a unit store (lanes: 16 or 64 channel blocks x key groups) and an MFMA A-operand read
// (lanes: 16 channels x 4 key groups) each hit every bank pair exactly twice.
__host__ __device__ constexpr int vt_swz(int sr) { return (((sr ^ (sr >> 3)) & 7) << 2) ^ ((sr >> 1) & 3); }

// At D = 128, V^T is kept as 16-byte pair units instead: unit (ch, pp), pp = 4 pm + g, holds
// the keys 4 kg .. 4 kg + 3 and 4 kg + 16 .. 4 kg + 19 of channel ch with kg = 8 pm + g, which
// are exactly the 8 values of one lane's A operand in O^T = V^T P^T (key order of the C layout
// of S^T), so one 16-byte read feeds one MFMA.  The XOR of the unit index with bits of the
// channel spreads both the operand reads (16 channels x 4 pairs per instruction) and the
// 8-byte half-unit stores of the staging over the banks (measured with an LDS probe: 4.3
// cycles per 16-byte read, 8.1 per 8-byte store, against 16 and 64 without the XOR).
__device__ __forceinline__ int vt_pair(int ch, int pp) { return ch * 8 + (pp ^ ((ch >> 1) & 7) ^ ((ch >> 4) & 7)); }

template <int D>
__device__ __forceinline__ int vt_unit(int ch, int kg) {
    using Geo = MfmaGeom<D>;
    const int sr = ch / Geo::RPS, rr = ch % Geo::RPS;
    return sr * 32 + ((rr * Geo::UPR + kg) ^ vt_swz(sr));
}

int mfma_tile_keys(int D) { return D == 512 ? MfmaGeom<512>::KT : MfmaGeom<128>::KT; }

bool mfma_supported(int D, int G, int R) {
    return (D == 128 || D == 512) && (G == 4 || G == 8) && R >= 1 && R * G >= 16;
}

// Query-column blocks per wave, query tiles and chunk length of one call.  Everything here is
// a function of the call's shape (never of page ids or device lengths), so the chunk
// boundaries, and with them the result, do not depend on where pages live.
MfmaPlan mfma_plan(int D, int G, int R, int S, int Hkv, int P, int max_seq_len, int window) {
    MfmaPlan p;
    const int nq = R * G;
    // one 16-column block per wave: two (QW = 2) halve the LDS reads per MFMA but need
    // about 280 registers, one wave per SIMD, and measured slower on every workload here
    p.qw = 1;
    // at d 128 a workgroup is 8 waves over two key sub-tiles (half the tile chain of a 4-wave
    // one, and half the partials for the merge to read); a d 512 tile fills the LDS of one
    p.ks = D == 128 ? 2 : 1;
    p.direct = false;
    p.tiles = (nq + 64 * p.qw - 1) / (64 * p.qw);
    const int kt = mfma_tile_keys(D);
    int span = max_seq_len;
    if (window > 0 && (int64_t)window + R - 1 < span) span = window + R - 1;
    if (span < 1) span = 1;
    const int64_t groups = (int64_t)S * Hkv * p.tiles;
    // enough query tiles to fill the CUs: one split per tile, whose output is then written
    // directly (partials and their merge cost far more than their bytes: a 512-row prompt
    // chunk over 2048 keys takes 53 us with 4 splits and a merge, 38 us with one)
    if (groups >= 256) {
        p.direct = true;
        p.chunk = (span + kt - 1) / kt * kt;     // bounds the keys of one tile
        if (p.chunk < kt) p.chunk = kt;
        return p;
    }
    // at d 512 a chunk of at least 3 tiles (one round of about 190 workgroups on the 4-row
    // verify at 9000 keys: 29.3 -> 27.4 us; 2 tiles need a second round and take 38 us)
    const int64_t lo = (D == 512 ? 3 : 4) * kt;
    // the longest chunk whose page-table entries the kernel caches in LDS (longer ones read the
    // table from memory per key piece); none if even the shortest does not fit
    int64_t hi = ((int64_t)(MfmaGeom<128>::TC - 2) * P - kt) / kt * kt;
    if (hi < lo) hi = (int64_t)1 << 40;
    if ((int64_t)R * 8 <= span) {
        // The rows span at most an eighth of the keys (every verify window; a prompt chunk far
        // into its stream): every row sees about the same keys, so all workgroups of the call do
        // the same work, and one of them fills a CU (137 KB of LDS at d 128; 4 waves of more
        // than 256 registers at d 512): the call runs in rounds of 256 workgroups.  Take the
        // chunk that minimises rounds x (time of one workgroup), a workgroup costing its K/V
        // bytes at an even share of about 85 % of HBM plus about 5 us of start-up and drain
        // (both measured on the 4-stream verify).  A round left nearly empty by the chunk
        // count doubles the time: 4 streams x 36k keys in 9 chunks of 4096 (288 workgroups)
        // took 161 us, in 8 of 4608 (256) 112 us; a 128-row chunk at 40,960 keys takes 144 us in
        // one round against 152 us in two.
        const double us_per_key = 4.0 * D / (0.85 * 8000.0e3 / 256.0), t0 = 5.0;
        double best = 0;
        int64_t best_chunk = lo;
        for (int64_t n = 1;; ++n) {
            int64_t c = ((span + n - 1) / n + kt - 1) / kt * kt;
            if (c < lo) c = lo;
            if (c <= hi) {
                int64_t ns = (max_seq_len + c - 1) / c;      // as the call's split count
                if (window > 0) ns = std::min(ns, (span + c - 1) / c + 1);
                const int64_t rounds = (groups * ns + 255) / 256;
                const double t = (double)rounds * ((double)c * us_per_key + t0);
                if (best == 0 || t < best) {
                    best = t;
                    best_chunk = c;
                }
            }
            if (c == lo) break;
        }
        p.chunk = (int)best_chunk;
        return p;
    }
    // Rows spread over much of the keys (an early prompt chunk on few streams): aim at 16
    // waves per CU over the whole call (the causal triangle gives the query tiles unequal work,
    // so several rounds keep the grid busy): long enough chunks to amortise the per-workgroup
    // set-up, short enough to keep every CU busy.  The 8-wave workgroups of d 128 come half as
    // many for the same waves.
    const int64_t target = p.ks == 2 ? 512 : 1024;
    int64_t chunk = ((int64_t)span * groups + target - 1) / target;
    chunk = (chunk + kt - 1) / kt * kt;
    if (chunk < lo) chunk = lo;
    if (chunk > hi) chunk = hi;
    p.chunk = (int)chunk;
    return p;
}

__device__ __forceinline__ f32x4_t mfma16(const bf16x8_t &a, const bf16x8_t &b, const f32x4_t &c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// MODE 0: P % KT == 0 and the chunk's table entries cached in LDS (one lookup per tile);
// MODE 1: entries cached, lookup per piece; MODE 2: lookup per piece in the global table.
// NTL: K/V loads are nontemporal.  Used at d 128 where each key tile has one reader, so that
// nothing is gained by keeping it in the caches (4 streams x 36k keys: 112 -> 96 us).  With
// several query tiles per chunk the tiles reread it from L2, and at d 512 plain loads measured
// faster (4-row verify at 9000 keys in pages of 37: 23.2 against 26.1 us), so those stay plain.
// KS: key sub-tiles per iteration.  With KS = 2 the workgroup has 8 waves: waves 4 g .. 4 g + 3
// compute sub-tile g of each 2 KT-key step with an online softmax of their own, and the two
// states are combined through LDS at the end, which halves the tile chain of a workgroup
// without splitting the keys over workgroups (no partials in memory).
template <int D, int G, int QW, int MODE, int KS, bool NTL>
__global__ __launch_bounds__(256 * KS) void part_mfma_kernel(const PartArgs a) {
    using Geo = MfmaGeom<D>;
    constexpr int KT = Geo::KT, KRS = Geo::KRS, CB = Geo::CB, KPT = Geo::KPT, TC = Geo::TC;
    constexpr int M = 64 * QW;       // query vectors per workgroup
    constexpr int NB = KT / 16;      // 16-key blocks per tile
    constexpr int NKB = D / 32;      // 32-channel blocks (QK k-steps)
    constexpr int NCB = D / 16;      // 16-channel blocks (PV output blocks)
    constexpr int NPM = KT / 32;     // 32-key PV k-steps

    constexpr int NTH = 256 * KS;    // threads
    static_assert((KS == 2) == (D == 128) && (KS == 1 || KS == 2), "key sub-tiles: 2 at D = 128, 1 at D = 512");

    // NBUF tile buffers: with two, a step stages the next step's tiles into one buffer while it
    // computes on the other (one barrier per step); one buffer stages and computes in turn
    constexpr int NBUF = KS == 2 ? 2 : 1;
    __shared__ __attribute__((aligned(16))) uint16_t k_lds_all[NBUF][KS][KT * KRS];
    __shared__ __attribute__((aligned(16))) uint2 vt_lds_all[NBUF][KS][D * KT / 4];
    __shared__ int32_t t_lds[TC];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    // wave-uniform by construction; readfirstlane tells the compiler, so that tests on them
    // (a sub-tile inside the split, a full tile) become scalar branches, not exec-mask ones
    const int wave = __builtin_amdgcn_readfirstlane((tid >> 6) & 3);   // column wave: query vectors 16 (wave QW + b) + col
    const int ksub = __builtin_amdgcn_readfirstlane(tid >> 8);         // key sub-tile this wave computes (and thread stages)
    const int col = lane & 15, grp = lane >> 4;
    // work item: the dispatcher hands workgroups to the 8 XCDs round-robin (dispatch id
    // d goes to XCD d mod 8), so XCD x gets the contiguous items [x per, (x + 1) per), ordered
    // (stream, KV head, split, tile) with the tile fastest: the query tiles that share a key
    // chunk run together on one XCD and reread it from that XCD's L2, not from HBM
    const int item = (blockIdx.x & 7) * a.per_xcd + (blockIdx.x >> 3);
    if (item >= a.S * a.Hkv * a.n_splits * a.tiles) return;
    const int tile = item % a.tiles;
    const int split = (item / a.tiles) % a.n_splits;
    const int kvh = (item / (a.tiles * a.n_splits)) % a.Hkv;
    const int s = item / (a.tiles * a.n_splits * a.Hkv);
    const int R = a.R, W = a.window, CH = a.chunk;
    const int L = a.seq_len[s];
    const int NQ = R * G;
    const int v0 = tile * M;
    if (v0 >= NQ || split >= a.n_splits) return;
    const int r_first = v0 / G;
    const int r_last = (min(NQ, v0 + M) - 1) / G;
    const int p_first = L - R + r_first, p_last = L - R + r_last;
    const int lo_stream = W > 0 ? max(0, L - R - W + 1) : 0;
    const int lo_tile = W > 0 ? max(0, p_first - W + 1) : 0;
    // a split is a chunk of absolute positions; a direct call's one split starts at the tile's
    // first visible key, and its chunk (>= window + R - 1, or >= max_seq_len) then covers every
    // key the tile's rows see (the bound only matters for lengths beyond max_seq_len: it keeps
    // the table entries the tile reads within the cached ones)
    const int c0 = a.direct ? lo_tile : (lo_stream / CH + split) * CH;
    const int kbeg = max(c0, lo_tile);
    const int kend = min(c0 + CH, p_last + 1);
    if (kbeg >= kend) {
        // no row of the tile sees this chunk: nothing to merge; a direct call owns the output
        // of its rows, which are then rows before the start of the stream: zeros
        if (a.direct && ksub == 0) {
#pragma unroll
            for (int b = 0; b < QW; ++b) {
                const int vq = v0 + (wave * QW + b) * 16 + col;
                if (vq < NQ) {
                    uint16_t *dst = a.out + ((size_t)(s * R + vq / G) * a.Hq + kvh * G + vq % G) * D + 4 * grp;
                    for (int cb = 0; cb < NCB; ++cb) *reinterpret_cast<uint2 *>(dst + 16 * cb) = make_uint2(0u, 0u);
                }
            }
        }
        return;
    }
    const int lo_full = W > 0 ? p_last - W + 1 : 0;   // every column sees keys >= this ...
    // ... and <= this (with a tree-shaped window, only the keys before the window)
    const int hi_full = a.tree ? min(p_first, L - R - 1) : p_first;
    const int win0 = L - R;                           // first slot of the window

    // this lane's query columns, and the queries as the B operand of S^T = K Q^T: the lane
    // holds channels 32 kb + 8 grp .. + 8 of its column
    bool col_ok[QW];
    int rq[QW], hq[QW], p_col[QW], lo_col[QW];
    uint32_t anc[QW];                                 // ancestor bits of the column's row
    bf16x8_t qf[QW][NKB];
#pragma unroll
    for (int b = 0; b < QW; ++b) {
        const int vq = v0 + (wave * QW + b) * 16 + col;
        col_ok[b] = vq < NQ;
        rq[b] = col_ok[b] ? vq / G : 0;
        hq[b] = kvh * G + (col_ok[b] ? vq % G : 0);
        p_col[b] = L - R + rq[b];
        lo_col[b] = W > 0 ? p_col[b] - W + 1 : 0;
        anc[b] = a.tree ? a.tree[s * R + rq[b]] : 0xFFFFFFFFu;
        const uint16_t *qrow = a.q + ((size_t)(s * R + rq[b]) * a.Hq + hq[b]) * D + 8 * grp;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
            u32x4 x = *reinterpret_cast<const u32x4 *>(qrow + 32 * kb);
            if (!col_ok[b]) x = u32x4{0, 0, 0, 0};
            qf[b][kb] = __builtin_bit_cast(bf16x8_t, x);
        }
    }

    // a wave whose query columns all lie past the tile's vectors (a partly filled tile: 4 rows
    // x GQA 8 leaves waves 2 and 3 without columns) stages its share and passes every barrier,
    // but computes nothing
    const bool wave_live = v0 + wave * QW * 16 < NQ;

    const int P = a.P;
    const int kt_first = (kbeg / KT) * KT;
    const int nt = (kend - kt_first + KT - 1) / KT;     // KT-key sub-tiles
    const int idx0 = kt_first / P;
    const int32_t *trow = a.table + (size_t)s * a.stride;
    if (MODE != 2) {
        for (int i = tid; i < TC; i += NTH) {
            int idx = idx0 + i;
            if (a.ring_pages) idx %= a.ring_pages;
            int pg = -1;
            if (idx < a.stride) pg = trow[idx];
            t_lds[i] = ((unsigned)pg < (unsigned)a.num_pages) ? pg : -1;
        }
    }
    lds_fence();

    const size_t page_elems = (size_t)a.Hkv * P * D;
    const size_t head_off = (size_t)kvh * P * D;
    // this thread's pieces: keys KPT kq .. KPT kq + KPT - 1 of sub-tile ksub, channels 8 kc .. + 8
    const int kc = (tid & 255) % CB, kq = (tid & 255) / CB;
    // buffer `buf` of the sub-tile this thread stages (ksub: thread tid stages sub-tile tid / 256,
    // which is also the sub-tile its wave computes)
    constexpr int KBUF = KS * KT * KRS, VBUF = KS * D * KT / 4;
    uint16_t *const k_st0 = k_lds_all[0][ksub];
    uint2 *const vt_st0 = vt_lds_all[0][ksub];
    u32x4 kreg0[KPT], vreg0[KPT], kreg1[KPT], vreg1[KPT];
    auto ld16 = [](const uint16_t *p) {
        if constexpr (NTL) return stream_load(p);
        else return *reinterpret_cast<const u32x4 *>(p);
    };
    // this thread's pieces of sub-tile tb of one operand (K or V pages)
    auto load_one = [&](int tb, const uint16_t *pages, u32x4 (&r)[KPT]) {
        if (MODE == 0) {
            // the whole tile lies in one page
            const int idx = tb / P;
            const int pg = max(t_lds[idx - idx0], 0);
            const size_t base = (size_t)pg * page_elems + head_off + (size_t)(tb - idx * P + KPT * kq) * D + 8 * kc;
#pragma unroll
            for (int u = 0; u < KPT; ++u) r[u] = ld16(pages + base + (size_t)u * D);
        } else {
#pragma unroll
            for (int u = 0; u < KPT; ++u) {
                const int j = tb + KPT * kq + u;
                int idx = j / P;
                const int off = j - idx * P;
                int pg;
                if (MODE == 1) {
                    pg = t_lds[idx - idx0];
                } else {
                    if (a.ring_pages) idx %= a.ring_pages;
                    const int tp = trow[min(idx, a.stride - 1)];
                    pg = (idx < a.stride && (unsigned)tp < (unsigned)a.num_pages) ? tp : -1;
                }
                const size_t e = (size_t)max(pg, 0) * page_elems + head_off + (size_t)off * D + 8 * kc;
                r[u] = ld16(pages + e);
            }
        }
    };
    auto load_tile = [&](int tb, u32x4 (&kreg)[KPT], u32x4 (&vreg)[KPT]) {
        load_one(tb, a.k_pages, kreg);
        load_one(tb, a.v_pages, vreg);
    };

    f32x4_t o[QW][NCB];
    float m_run[QW], l_run[QW];
#pragma unroll
    for (int b = 0; b < QW; ++b) {
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) o[b][cb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        m_run[b] = -INFINITY;
        l_run[b] = 0.f;
    }
    const float c2 = a.scale_log2;
    // a running max is raised only when a score passes it by more than this (8 in the log2
    // domain): the weights then stay below 2^8, which bf16 and the fp32 sums hold exactly
    // as well as weights below 1, and most tiles skip the cross-lane max and the rescale
    const float slack = fminf(8.0f / c2, 3.0e38f);      // finite, so that -inf + slack stays -inf

    // V^T operand reads (channel 16 cb + col, unit 8 pm + 4 hh + grp): vt_swz is linear over
    // GF(2) and the row number 16 cb / RPS + col / RPS has disjoint bit fields, so the unit
    // index is (lane part ^ instruction constant) + lane row + instruction row
    constexpr int RPS = Geo::RPS, CPS = 16 / RPS;
    const int vt_row_l = (col / RPS) * 32;
    const int vt_x_l = ((col % RPS) * Geo::UPR + grp) ^ vt_swz(col / RPS);
    // D = 128: byte offset of this lane's pair unit (channel 16 cb + col, pair 4 pm + grp) within
    // a 16-channel block, for each of the 8 values of the instruction constant (4 pm) ^ cb
    int pv_off[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) pv_off[c] = 16 * (8 * col + ((grp ^ (col >> 1)) ^ c));
    const bf16x8_t ones8 = __builtin_bit_cast(bf16x8_t, u32x4{0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u});

    // Step it covers sub-tiles KS it .. KS it + KS - 1; loads past the last sub-tile reread it
    // (in bounds, never computed on), and sub-tiles past it are all masked out.
    const int kt_last = kt_first + (nt - 1) * KT;
    const int nsteps = (nt + KS - 1) / KS;
    // stage step it's sub-tile of this thread from (kreg, vreg) into buffer buf
    // stage K rows as loaded into buffer buf
    auto stage_k = [&](const u32x4 (&kreg)[KPT], int buf) {
        uint16_t *const k_st = k_st0 + buf * KBUF;
#pragma unroll
        for (int u = 0; u < KPT; ++u)
            *reinterpret_cast<u32x4 *>(k_st + (KPT * kq + u) * KRS + 8 * kc) = kreg[u];
    };
    // stage V of step it transposed into 4-key units of buffer buf, keys outside [kbeg, kend)
    // zeroed (they may be unused slots holding NaN)
    auto stage_v = [&](int it, const u32x4 (&vreg)[KPT], int buf) {
        const int ts = kt_first + (it * KS + ksub) * KT;          // sub-tile this thread stages
        uint2 *const vt_st = vt_st0 + buf * VBUF;
        const bool inside = ts >= kbeg && ts + KT <= kend;
#pragma unroll
        for (int h = 0; h < KPT / 4; ++h) {
            u32x4 x[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                x[u] = vreg[4 * h + u];
                if (!inside) {
                    const int j = ts + KPT * kq + 4 * h + u;
                    const uint32_t keep = (j >= kbeg && j < kend) ? 0xFFFFFFFFu : 0u;
                    x[u] = x[u] & keep;
                }
            }
            const int kg = (KPT * kq) / 4 + h;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint2 ev = make_uint2(__builtin_amdgcn_perm(x[1][i], x[0][i], 0x05040100u),
                                            __builtin_amdgcn_perm(x[3][i], x[2][i], 0x05040100u));
                const uint2 od = make_uint2(__builtin_amdgcn_perm(x[1][i], x[0][i], 0x07060302u),
                                            __builtin_amdgcn_perm(x[3][i], x[2][i], 0x07060302u));
                if constexpr (D == 128) {
                    // half hh = bit 2 of kg of pair 4 (kg >> 3) + (kg & 3)
                    const int pp = 4 * (kg >> 3) + (kg & 3), hh = (kg >> 2) & 1;
                    vt_st[2 * vt_pair(8 * kc + 2 * i, pp) + hh] = ev;
                    vt_st[2 * vt_pair(8 * kc + 2 * i + 1, pp) + hh] = od;
                } else {
                    vt_st[vt_unit<D>(8 * kc + 2 * i, kg)] = ev;
                    vt_st[vt_unit<D>(8 * kc + 2 * i + 1, kg)] = od;
                }
            }
        }
    };
    auto stage = [&](int it, const u32x4 (&kreg)[KPT], const u32x4 (&vreg)[KPT], int buf) {
        stage_k(kreg, buf);
        stage_v(it, vreg, buf);
    };
    auto ts_of = [&](int it) { return kt_first + (it * KS + ksub) * KT; };
    // compute step it's sub-tile of this wave from buffer buf
    // S^T of step it's sub-tile for this wave's query columns, from K buffer buf; each K
    // fragment feeds QW MFMAs (a padded step past the split computes nothing)
    auto qk = [&](int it, int buf, f32x4_t (&sacc)[QW][NB]) {
        const int tb = kt_first + (it * KS + ksub) * KT;          // sub-tile this wave computes
        if (tb >= kend || !wave_live) return;
        const uint16_t *const k_lds = k_st0 + buf * KBUF;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
            for (int b = 0; b < QW; ++b) sacc[b][nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) {
                const bf16x8_t kf = *reinterpret_cast<const bf16x8_t *>(k_lds + (16 * nb + col) * KRS + 32 * kb + 8 * grp);
#pragma unroll
                for (int b = 0; b < QW; ++b) sacc[b][nb] = mfma16(kf, qf[b][kb], sacc[b][nb]);
            }
        }
    };
    // mask, online softmax and O^T += V^T P^T of step it's sub-tile, from its scores and V
    // buffer buf
    auto smpv = [&](int it, int buf, f32x4_t (&sacc)[QW][NB]) {
        const int tb = kt_first + (it * KS + ksub) * KT;
        if (tb >= kend || !wave_live) return;
        const uint2 *const vt_lds = vt_st0 + buf * VBUF;
        const bool full = tb >= kbeg && tb + KT <= kend && tb + KT - 1 <= hi_full && tb >= lo_full;
        bf16x8_t pf[QW][NPM];
#pragma unroll
        for (int b = 0; b < QW; ++b) {
            // mask (raw scores; the scale is applied inside the exponent), tile max
            float tmax = -INFINITY;
            if (full) {
#pragma unroll
                for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                    for (int r = 0; r < 4; ++r) tmax = fmaxf(tmax, sacc[b][nb][r]);
            } else {
#pragma unroll
                for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int j = tb + 16 * nb + 4 * grp + r;
                        const int t = j - win0;             // window slot of the key, if >= 0
                        // bitwise, not short-circuit, so that the test is straight-line selects
                        // rather than a branch per score
                        const bool vis = col_ok[b] & (j >= kbeg) & (j < kend) & (j <= p_col[b]) & (j >= lo_col[b]) &
                                         ((t < 0) | (((anc[b] >> (t & 31)) & 1u) != 0));
                        const float x = vis ? sacc[b][nb][r] : -INFINITY;
                        sacc[b][nb][r] = x;
                        tmax = fmaxf(tmax, x);
                    }
            }
            // the running max of a column moves only when one of its scores passes it by more
            // than the slack (rare after the first tile): only then is the tile max reduced over
            // the column's four lane groups and the sums rescaled
            if (__builtin_amdgcn_ballot_w64(tmax > m_run[b] + slack)) {
                tmax = fmaxf(tmax, __shfl_xor(tmax, 16));
                tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
                const float m_new = fmaxf(m_run[b], tmax);
                const float mc_new = (m_new == -INFINITY) ? 0.f : m_new * c2;
                const float alpha = fast_exp2(m_run[b] * c2 - mc_new);   // 0 while nothing was seen
                m_run[b] = m_new;
                l_run[b] *= alpha;
                if (alpha != 1.f) {
#pragma unroll
                    for (int cb = 0; cb < NCB; ++cb) o[b][cb] *= alpha;
                }
            }
            const float mc = (m_run[b] == -INFINITY) ? 0.f : m_run[b] * c2;
#pragma unroll
            for (int pm = 0; pm < NPM; ++pm) {
#pragma unroll
                for (int hh = 0; hh < 2; ++hh)
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        pf[b][pm][4 * hh + r] = (__bf16)fast_exp2(__builtin_fmaf(sacc[b][2 * pm + hh][r], c2, -mc));
            }
            // the tile's weight sum of each column, from the same bf16 weights that PV uses:
            // a ones matrix times P^T puts the column's sum over all the tile's keys in every
            // lane of the column, so no lane adds or reduces them
            f32x4_t ls = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int pm = 0; pm < NPM; ++pm) ls = mfma16(ones8, pf[b][pm], ls);
            l_run[b] += ls[0];
        }
        // O^T += V^T P^T: A = V^T rows (channels 16 cb + col), keys 32 pm + 4 grp + {0..3}
        // and 32 pm + 16 + 4 grp + {0..3}; each V fragment feeds QW MFMAs
        // (kept opaque so that the 2 NCB NPM addresses are formed in the loop, one ALU op
        // each, not held in registers across it)
        if constexpr (D == 128) {
            // unit vt_pair(16 cb + col, 4 pm + grp) = 8 (16 cb + col) + ((grp ^ (col >> 1)) ^ (4 pm ^ cb)):
            // the lane's offset for the constant (4 pm) ^ cb, plus 2048 bytes per channel block
            const char *vtb = reinterpret_cast<const char *>(vt_lds);
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb) {
#pragma unroll
                for (int pm = 0; pm < NPM; ++pm) {
                    const bf16x8_t vv = __builtin_bit_cast(
                        bf16x8_t, *reinterpret_cast<const u32x4 *>(vtb + pv_off[(4 * pm) ^ cb] + 2048 * cb));
#pragma unroll
                    for (int b = 0; b < QW; ++b) o[b][cb] = mfma16(vv, pf[b][pm], o[b][cb]);
                }
            }
        } else {
            int vx = vt_x_l;
            asm volatile("" : "+v"(vx));
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb) {
#pragma unroll
                for (int pm = 0; pm < NPM; ++pm) {
                    const int rowc = CPS * cb * 32;
                    const uint2 lo = vt_lds[((vx ^ ((8 * pm) ^ vt_swz(CPS * cb))) + vt_row_l) + rowc];
                    const uint2 hi = vt_lds[((vx ^ ((8 * pm + 4) ^ vt_swz(CPS * cb))) + vt_row_l) + rowc];
                    const bf16x8_t vv = __builtin_bit_cast(bf16x8_t, u32x4{lo.x, lo.y, hi.x, hi.y});
#pragma unroll
                    for (int b = 0; b < QW; ++b) o[b][cb] = mfma16(vv, pf[b][pm], o[b][cb]);
                }
            }
        }
    };
    auto compute = [&](int it, int buf) {
        f32x4_t sacc[QW][NB];
        qk(it, buf, sacc);
        smpv(it, buf, sacc);
    };
    // d 512, one buffer and one step in flight (a tile is 8 registers x 4 per thread and
    // operand): the loads for step it + 1 go into the registers step it was staged from
    auto step = [&](int it, u32x4 (&kreg)[KPT], u32x4 (&vreg)[KPT]) {
        lds_fence();
        stage(it, kreg, vreg, 0);
        load_tile(min(ts_of(it + 1), kt_last), kreg, vreg);
        lds_fence();
        compute(it, 0);
    };
    if constexpr (NBUF == 2) {
        // Software pipeline over two K and two V buffers.  Step it computes the scores of step
        // it + 1 (MFMA) before the softmax and PV of step it, whose scores came from the step
        // before: the MFMAs and the softmax of one wave are independent and overlap.  K is
        // staged two steps ahead and V one step ahead, each into the buffer its previous
        // reader released before the last barrier; register set r of an operand holds the
        // steps of parity r, and the loads are issued in one fixed order (K it + 4, then V
        // it + 3), so every wait is for the oldest set only.
        u32x4 (&k0)[KPT] = kreg0, (&k1)[KPT] = kreg1, (&v0)[KPT] = vreg0, (&v1)[KPT] = vreg1;
        load_one(min(ts_of(0), kt_last), a.k_pages, k0);
        asm volatile("" ::: "memory");
        load_one(min(ts_of(1), kt_last), a.k_pages, k1);
        asm volatile("" ::: "memory");
        load_one(min(ts_of(0), kt_last), a.v_pages, v0);
        asm volatile("" ::: "memory");
        stage_k(k0, 0);
        load_one(min(ts_of(2), kt_last), a.k_pages, k0);
        asm volatile("" ::: "memory");
        stage_k(k1, 1);
        load_one(min(ts_of(1), kt_last), a.v_pages, v1);
        asm volatile("" ::: "memory");
        load_one(min(ts_of(3), kt_last), a.k_pages, k1);
        asm volatile("" ::: "memory");
        stage_v(0, v0, 0);
        load_one(min(ts_of(2), kt_last), a.v_pages, v0);
        asm volatile("" ::: "memory");
        lds_fence();
        f32x4_t s0[QW][NB], s1[QW][NB];
        qk(0, 0, s0);
        // Steps it and it + 1 per iteration.  The last iterations (the second loop, the same
        // body) neither load nor stage steps past the split, so that the split ends when its
        // own data has arrived, not after loads that would only reread its last tile (4-stream
        // verify at 9k keys: 32.4 -> 29.9 us).  The body is written out twice rather than
        // guarded in one loop: conditional loads in the main loop would make every wait in it
        // conservative, and a shared lambda put the step registers in scratch memory.
        int it = 0;
        for (; it + 6 <= nsteps; it += 2) {
            qk(it + 1, 1, s1);
            smpv(it, 0, s0);
            stage_k(k0, 0);                                   // K(it + 2)
            load_one(min(ts_of(it + 4), kt_last), a.k_pages, k0);
            asm volatile("" ::: "memory");
            stage_v(it + 1, v1, 1);                           // V(it + 1)
            load_one(min(ts_of(it + 3), kt_last), a.v_pages, v1);
            asm volatile("" ::: "memory");
            lds_fence();
            qk(it + 2, 0, s0);
            smpv(it + 1, 1, s1);
            stage_k(k1, 1);                                   // K(it + 3)
            load_one(min(ts_of(it + 5), kt_last), a.k_pages, k1);
            asm volatile("" ::: "memory");
            stage_v(it + 2, v0, 0);                           // V(it + 2)
            load_one(min(ts_of(it + 4), kt_last), a.v_pages, v0);
            asm volatile("" ::: "memory");
            lds_fence();
        }
        for (; it < nsteps; it += 2) {
            qk(it + 1, 1, s1);
            smpv(it, 0, s0);
            if (it + 2 < nsteps) stage_k(k0, 0);
            if (it + 4 < nsteps) load_one(min(ts_of(it + 4), kt_last), a.k_pages, k0);
            asm volatile("" ::: "memory");
            if (it + 1 < nsteps) stage_v(it + 1, v1, 1);
            if (it + 3 < nsteps) load_one(min(ts_of(it + 3), kt_last), a.v_pages, v1);
            asm volatile("" ::: "memory");
            lds_fence();
            qk(it + 2, 0, s0);
            smpv(it + 1, 1, s1);
            if (it + 3 < nsteps) stage_k(k1, 1);
            if (it + 5 < nsteps) load_one(min(ts_of(it + 5), kt_last), a.k_pages, k1);
            asm volatile("" ::: "memory");
            if (it + 2 < nsteps) stage_v(it + 2, v0, 0);
            if (it + 4 < nsteps) load_one(min(ts_of(it + 4), kt_last), a.v_pages, v0);
            asm volatile("" ::: "memory");
            lds_fence();
        }
    } else {
        load_tile(min(ts_of(0), kt_last), kreg0, vreg0);
        for (int it = 0; it < nsteps; ++it) step(it, kreg0, vreg0);
    }

    if constexpr (KS == 2) {
        // combine the two key sub-tile groups: waves 4..7 hand their state to waves 0..3
        // through LDS (field f of lane (wave, lane) at f * 256 + 64 wave + lane), then only
        // waves 0..3 go on
        constexpr int NF = 4 * NCB + 2;
        static_assert(NF * 256 * 4 <= KS * KT * KRS * 2, "exchange fits the K tiles");
        float *xch = reinterpret_cast<float *>(&k_lds_all[0][0][0]);
        const int xi = 64 * wave + lane;
        lds_fence();
        if (ksub == 1) {
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
                for (int r = 0; r < 4; ++r) xch[(4 * cb + r) * 256 + xi] = o[0][cb][r];
            xch[(4 * NCB) * 256 + xi] = m_run[0];
            xch[(4 * NCB + 1) * 256 + xi] = l_run[0];
        }
        lds_fence();
        if (ksub == 1) return;
        const float m1 = xch[(4 * NCB) * 256 + xi];
        const float l1 = xch[(4 * NCB + 1) * 256 + xi];
        const float m = fmaxf(m_run[0], m1);
        const float mc = (m == -INFINITY) ? 0.f : m * c2;
        const float a0 = m_run[0] == -INFINITY ? 0.f : fast_exp2(m_run[0] * c2 - mc);
        const float a1 = m1 == -INFINITY ? 0.f : fast_exp2(m1 * c2 - mc);
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
            for (int r = 0; r < 4; ++r) o[0][cb][r] = o[0][cb][r] * a0 + xch[(4 * cb + r) * 256 + xi] * a1;
        l_run[0] = l_run[0] * a0 + l1 * a1;
        m_run[0] = m;
    }

    // write the normalised bf16 output (a direct call: the one split is the whole result, with
    // the merge's arithmetic) or the partials
#pragma unroll
    for (int b = 0; b < QW; ++b) {
        const float l_tot = l_run[b];      // already the column's sum in every lane of it
        if (a.direct) {
            if (col_ok[b]) {
                const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
                uint16_t *dst = a.out + ((size_t)(s * R + rq[b]) * a.Hq + hq[b]) * D + 4 * grp;
#pragma unroll
                for (int cb = 0; cb < NCB; ++cb)
                    *reinterpret_cast<uint2 *>(dst + 16 * cb) =
                        make_uint2(pack_bf16x2(o[b][cb][0] * inv, o[b][cb][1] * inv),
                                   pack_bf16x2(o[b][cb][2] * inv, o[b][cb][3] * inv));
            }
        } else if (col_ok[b]) {
            const size_t slot = ((size_t)(s * R + rq[b]) * a.Hq + hq[b]) * a.n_splits + split;
            float *dst = a.ws_acc + slot * D + 4 * grp;
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb)
                *reinterpret_cast<float4 *>(dst + 16 * cb) =
                    make_float4(o[b][cb][0], o[b][cb][1], o[b][cb][2], o[b][cb][3]);
            if (grp == 0) {
                const float m2 = m_run[b] == -INFINITY ? -INFINITY : m_run[b] * c2;
                *reinterpret_cast<float2 *>(a.ws_ml + slot * 2) = make_float2(m2, l_tot);
            }
        }
    }
}

template <int D, int G, int QW, int KS, bool NTL>
static hipError_t launch_dgq(const PartArgs &a, hipStream_t st) {
    using Geo = MfmaGeom<D>;
    const dim3 grid(8 * a.per_xcd);
    const bool cached = (a.chunk + Geo::KT) / a.P + 2 <= Geo::TC;
    if (cached && a.P % Geo::KT == 0)
        hipLaunchKernelGGL((part_mfma_kernel<D, G, QW, 0, KS, NTL>), grid, dim3(256 * KS), 0, st, a);
    else if (cached)
        hipLaunchKernelGGL((part_mfma_kernel<D, G, QW, 1, KS, NTL>), grid, dim3(256 * KS), 0, st, a);
    else
        hipLaunchKernelGGL((part_mfma_kernel<D, G, QW, 2, KS, NTL>), grid, dim3(256 * KS), 0, st, a);
    return hipGetLastError();
}

template <int D, int G, int KS>
static hipError_t launch_dg(const PartArgs &a, hipStream_t st) {
    if constexpr (D == 128)
        if (a.tiles == 1) return launch_dgq<D, G, 1, KS, true>(a, st);
    return launch_dgq<D, G, 1, KS, false>(a, st);
}

hipError_t launch_part_mfma(int D, int G, const MfmaPlan &p, const PartArgs &args, int S, hipStream_t st) {
    if (args.chunk != p.chunk || args.chunk % mfma_tile_keys(D) != 0) return hipErrorInvalidValue;
    PartArgs a = args;
    a.S = S;
    a.tiles = p.tiles;
    const int64_t items = (int64_t)S * a.Hkv * a.n_splits * p.tiles;
    if (items == 0) return hipSuccess;
    if (items > (int64_t)1 << 30) return hipErrorInvalidValue;
    a.per_xcd = (int)((items + 7) / 8);
    if (p.qw != 1 || p.ks != (D == 128 ? 2 : 1)) return hipErrorInvalidValue;
    if (D == 128 && G == 4) return launch_dg<128, 4, 2>(a, st);
    if (D == 128 && G == 8) return launch_dg<128, 8, 2>(a, st);
    if (D == 512 && G == 4) return launch_dg<512, 4, 1>(a, st);
    if (D == 512 && G == 8) return launch_dg<512, 8, 1>(a, st);
    return hipErrorInvalidValue;
}

}  // namespace kvp
