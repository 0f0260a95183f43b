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
//    MFMA operand reads touch every LDS bank equally.  At d 128 with pages holding whole tiles
//    the tiles go from memory straight into LDS instead (DMA below), and V^T is read from plain
//    rows with transposing LDS reads.
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
typedef short v4i16_t __attribute__((ext_vector_type(4)));
#define LDS __attribute__((address_space(3)))

template <int D>
struct MfmaGeom {
    static constexpr int KT = D == 128 ? 64 : 32;       // keys per tile
    static constexpr int KRS = D + 16;                  // K tile row stride (bf16): 288, 544 or 1056 bytes, so
                                                        // that an MFMA operand read is free of bank conflicts
    static constexpr int CB = D / 8;                    // 16-byte channel blocks per row
    static constexpr int NT = 256;                      // threads
    static constexpr int KPT = KT * CB / NT;            // keys per thread per tile (4 or 8)
    static constexpr int UPR = KT / 4;                  // V^T units (4 keys) per channel
    static constexpr int RPS = 32 / UPR;                // channels per 32-unit (256-byte) row
    static constexpr int TC = kTableCache;              // cached page-table entries
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

// Whether a call of this shape runs the direct-to-LDS kernel, which fuses the row write of
// its own rows (PartArgs::k_new / v_new); the other MFMA kernels ignore k_new.
bool mfma_fuses_rows(int D, int P, int chunk) { return D == 128 && table_mode(P, chunk, MfmaGeom<128>::KT, 1) == 0; }

int mfma_tile_keys(int D) { return D == 512 ? MfmaGeom<512>::KT : D == 256 ? MfmaGeom<256>::KT : MfmaGeom<128>::KT; }
int mfma_table_mode(int D, int P, int chunk) { return table_mode(P, chunk, mfma_tile_keys(D), 1); }

bool mfma_supported(int D, int G, int R) {
    return (D == 128 || D == 256 || D == 512) && (G == 4 || G == 8 || G == 12 || G == 16) && R >= 1 && R * G >= 16;
}

// d 512 calls of 16 to 32 query vectors per KV head over pages of at least 32 keys (a verify
// window of a few rows) run the channel-split kernel (part_narrow_kernel below); its plan counts
// chunks in units of this many 32-key tiles.
constexpr int kNarrowTiles = 3;
constexpr bool narrow_shape(int D, int NQ, int P) { return D == 512 && NQ >= 16 && NQ <= 32 && P >= 32; }

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
    // The channel-split kernel at d 512 (not for direct calls, which fill the GPU with tiles):
    // chunks of whole batches, as few batches per workgroup as keep the call in one round of one
    // workgroup per CU, within the table entries a workgroup caches.
    if (groups < 256 && narrow_shape(D, nq, P)) {
        const int64_t unit = (int64_t)kNarrowTiles * kt;
        const int64_t cap = ((int64_t)(MfmaGeom<128>::TC - 2) * P - kt) / kt * kt;
        int64_t c = unit;
        for (;;) {
            int64_t ns = (max_seq_len + c - 1) / c;
            if (window > 0) ns = std::min(ns, (span + c - 1) / c + 1);
            if (groups * ns <= 256 || c + unit > cap) break;
            c += unit;
        }
        p.chunk = (int)c;
        return p;
    }
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
        // a d 256 workgroup (34 KB of LDS, two waves per SIMD) shares its CU with another
        const int64_t per_round = D == 256 ? 512 : 256;
        double best = 0;
        int64_t best_chunk = lo;
        for (int64_t n = 1;; ++n) {
            int64_t c = ((span + n - 1) / n + kt - 1) / kt * kt;
            if (c < lo) c = lo;
            if (c <= hi) {
                int64_t ns = (max_seq_len + c - 1) / c;      // as the call's split count
                if (window > 0) ns = std::min(ns, (span + c - 1) / c + 1);
                const int64_t rounds = (groups * ns + per_round - 1) / per_round;
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

// Waits for all of this wave's vector memory operations (vmcnt 0; expcnt and lgkmcnt left
// alone): loads that write LDS directly have landed once it returns.
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// The loading waves' workgroup barrier: their LDS stores (zeroed rows) complete (lgkmcnt 0),
// loads into LDS still in flight stay in flight (the loads a barrier publishes are waited for
// explicitly before it).  A barrier with a workgroup release fence would wait for every load
// that writes LDS.
__device__ __forceinline__ void loader_barrier() {
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt 0
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Waits until at most N of this wave's vector memory operations are outstanding (they complete
// in issue order; expcnt and lgkmcnt left alone).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

// 16 bytes per lane from global memory straight into LDS: lane l's bytes land at dst + 16 l
// (dst wave-uniform).  NT: nontemporal.
template <bool NT>
__device__ __forceinline__ void load_to_lds(const char *src, char *dst) {
    __builtin_amdgcn_global_load_lds((const void *)src, (LDS void *)dst, 16, 0, NT ? 2 : 0);
}

// Transposed 8-byte LDS read of 16-bit elements (ds_read_b64_tr_b16; see the DMA layout).
__device__ __forceinline__ v4i16_t lds_read_tr16(const char *p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS v4i16_t *)(p));
}

// Loading waves of the d 128 direct-to-LDS kernel (a multiple of its 2 key sub-tiles): one
// wave issues a 1 KB load about every 70 cycles, so a step's 64 loads need several of them.
constexpr int kLoadWaves = 4;

__device__ __forceinline__ f32x4_t mfma16(const bf16x8_t &a, const bf16x8_t &b, const f32x4_t &c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// MODE 0: P % KT == 0 and the chunk's table entries cached in LDS (one lookup per tile);
// MODE 1: entries cached, lookup per piece; MODE 2: lookup per piece in the global table.
// NTL: K/V loads are nontemporal.  Used wherever each key tile has one reader (one query tile
// per chunk), so that nothing is gained by keeping it in the caches (4 streams x 36k keys at
// d 128: 112 -> 96 us; 16/1 heads at d 512, 4 rows over pages of 512, cold part kernel at
// 32,768 keys 41.0 -> 31.1 us, at 9,000 keys 28.1 -> 27.0 us).  With several query tiles per
// chunk the tiles reread it from L2 and the loads stay plain.
// KS: key sub-tiles per iteration.  With KS = 2 the workgroup has 8 waves: waves 4 g .. 4 g + 3
// compute sub-tile g of each 2 KT-key step with an online softmax of their own, and the two
// states are combined through LDS at the end, which halves the tile chain of a workgroup
// without splitting the keys over workgroups (no partials in memory).
// DMA (d 128, pages holding whole tiles): K and V go from memory straight into LDS
// (global_load_lds_dwordx4: lane l of a load writes the 16 bytes at the load's LDS base + 16 l,
// from an address of its own), with no pass through registers and no staging instructions.  A
// tile is kept as plain rows of 256 bytes whose 16-byte pieces are permuted per row (an XOR
// with the row number, chosen through each lane's source address), and the V^T operand of PV
// comes from transposed 8-byte LDS reads (ds_read_b64_tr_b16): within each 16-lane group,
// lane 4 a + e receives element e of the 8-byte pieces that lanes a, a + 4, a + 8 and a + 12
// address, i.e. four consecutive keys of one channel when those lanes address four
// consecutive rows.  Four more waves (a workgroup of 768 threads) issue all the loads: a wave
// issues a 1 KB load about every 70 cycles, so a burst of a step's 64 loads would otherwise
// hold the computing waves at issue (two loading waves: the 2,048-token prompt 99.6 µs, four:
// 97.8 µs; the verify window's cold part kernel 35.8 and 34.4 µs).
template <int D, int G, int QW, int MODE, int KS, bool NTL, bool DMA, bool DEEP = false>
__global__ __launch_bounds__(DMA ? 256 * KS + 64 * kLoadWaves : 256 * KS) void part_mfma_kernel(const PartArgs a) {
    using Geo = MfmaGeom<D>;
    constexpr int KRS = Geo::KRS, CB = Geo::CB, KPT = Geo::KPT, TC = Geo::TC;
    // DEEP (with DMA, split calls): 32-key sub-tiles in four buffers per operand, loaded two
    // steps further ahead
    static_assert(!DEEP || DMA, "deep prefetch loads straight into LDS");
    constexpr int KT = DEEP ? 32 : Geo::KT;   // keys per sub-tile
    static_assert(!DMA || (D == 128 && MODE == 0 && KS == 2), "direct-to-LDS tiles: d 128, whole tiles per page");
    constexpr int KROW = DMA ? D : KRS;   // K tile row stride (bf16)
    constexpr int M = 64 * QW;       // query vectors per workgroup
    constexpr int NB = KT / 16;      // 16-key blocks per tile
    constexpr int NKB = D / 32;      // 32-channel blocks (QK k-steps)
    constexpr int NCB = D / 16;      // 16-channel blocks (PV output blocks)
    constexpr int NPM = KT / 32;     // 32-key PV k-steps

    constexpr int NTH = DMA ? 256 * KS + 64 * kLoadWaves : 256 * KS;   // threads (with DMA: 8 computing waves and the loading ones)
    static_assert((KS == 2) == (D == 128) && (KS == 1 || KS == 2), "key sub-tiles: 2 at D = 128, 1 at D = 256 and 512");

    // NBUF tile buffers: with two, a step stages the next step's tiles into one buffer while it
    // computes on the other (one barrier per step); one buffer stages and computes in turn
    constexpr int NBUF = DEEP ? 4 : (KS == 2 || (D == 256 && MODE == 0)) ? 2 : 1;
    __shared__ __attribute__((aligned(16))) uint16_t k_lds_all[NBUF][KS][KT * KROW];
    // V^T units, or with DMA the V rows of a tile (KT x D bf16, the same bytes)
    __shared__ __attribute__((aligned(16))) uint2 vt_lds_all[NBUF][KS][D * KT / 4];
    __shared__ int32_t t_lds[TC];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    // wave-uniform by construction; readfirstlane tells the compiler, so that tests on them
    // (a sub-tile inside the split, a full tile) become scalar branches, not exec-mask ones
    const int wave = __builtin_amdgcn_readfirstlane((tid >> 6) & 3);   // column wave: query vectors 16 (wave QW + b) + col
    const int ksub = __builtin_amdgcn_readfirstlane(min(tid >> 8, KS - 1));   // key sub-tile this wave computes (and thread stages)
    // DMA: waves 8 .. 8 + kLoadWaves - 1 only load (wave 8 + p rows of sub-tile p / LPS of every
    // step, LPS waves per sub-tile), so that the computing waves never wait at the issue of a
    // burst of loads
    const bool producer = DMA && tid >= 512;
    const int pw = __builtin_amdgcn_readfirstlane(producer ? (tid >> 6) - 8 : 0);
    constexpr int LPS = kLoadWaves / KS;                 // loading waves per sub-tile
    const int psub = pw / LPS, prow0 = (pw % LPS) * (KT / LPS);
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
    const int NQ = R * G;
    const int v0 = tile * M;
    if (v0 >= NQ || split >= a.n_splits) return;
    const int32_t *trow = a.table + (size_t)s * a.stride;

    // This lane's query columns and the queries as the B operand of S^T = K Q^T (the lane holds
    // channels 32 kb + 8 grp .. + 8 of its column), a tree window's ancestor bits, and, when the
    // stream's whole page table fits the cache (a full layer of at most TC pages), its table
    // entries: none of them depends on the stream's length, so they are loaded together with
    // it, and the first K/V loads wait for one round trip to memory rather than two.
    const bool whole = whole_table(MODE, a.ring_pages, a.stride);
    const int Lv = load_uniform_i32(a.seq_len + s);
    bool col_ok[QW];
    int rq[QW], hq[QW];
    uint32_t anc[QW];                                 // ancestor bits of the column's row
    bf16x8_t qf[QW][NKB];
#pragma unroll
    for (int b = 0; b < QW; ++b) {
        const int vq = v0 + (wave * QW + b) * 16 + col;
        col_ok[b] = vq < NQ;
        rq[b] = col_ok[b] ? vq / G : 0;
        hq[b] = kvh * G + (col_ok[b] ? vq % G : 0);
        anc[b] = a.tree ? a.tree[s * R + rq[b]] : 0xFFFFFFFFu;
        const uint16_t *qrow = a.q + ((size_t)(s * R + rq[b]) * a.Hq + hq[b]) * D + 8 * grp;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
            u32x4 x = *reinterpret_cast<const u32x4 *>(qrow + 32 * kb);
            if (!col_ok[b]) x = u32x4{0, 0, 0, 0};
            qf[b][kb] = __builtin_bit_cast(bf16x8_t, x);
        }
    }
    constexpr int TPT = (TC + NTH - 1) / NTH;         // table entries per thread
    int tv[TPT];
    if (whole) {
#pragma unroll
        for (int k = 0; k < TPT; ++k) {
            const int i = tid + k * NTH;
            tv[k] = i < a.stride ? trow[i] : -1;
        }
    }
    const int L = kernel_len(__builtin_amdgcn_readfirstlane(Lv), a.max_len);
    if (whole) {
#pragma unroll
        for (int k = 0; k < TPT; ++k) {
            const int i = tid + k * NTH;
            if (i < TC) t_lds[i] = ((unsigned)tv[k] < (unsigned)a.num_pages) ? tv[k] : -1;
        }
    }

    // The call's own rows go in with the attention (kv_rows_put fused, direct-to-LDS kernel):
    // split 0 of the tile in which a row's first query vector lies writes that row's K and V of
    // head kvh into its page slot, exactly as kv_rows_put does, and every workgroup reads the
    // call's rows from k_new and v_new, never from those slots.  The slots written hold
    // positions that no row of the call sees (the ring holds at least window + R - 1
    // positions, as for kv_rows_put followed by the attention), so no workgroup reads what
    // another writes.  The loading waves do it once their last loads are issued, while the
    // computing waves finish the last steps.
    auto put_rows = [&](int t, int nt_) {
        if (a.k_new == nullptr || split != 0) return;
        constexpr int PPR = D / 8;                     // 16-byte pieces of a row
        const int rb = (v0 + G - 1) / G, re = min((v0 + M + G - 1) / G, R);
        for (int w = t; w < (re - rb) * 2 * PPR; w += nt_) {
            const int rr = rb + w / (2 * PPR), op = (w / PPR) & 1, pc = w % PPR;
            const int pos = L - R + rr;
            if (pos < 0) continue;
            int idx = pos / a.P;
            const int off = pos - idx * a.P;
            if (a.ring_pages) idx %= a.ring_pages;
            if (idx >= a.stride) continue;
            const int pg = trow[idx];
            if ((unsigned)pg >= (unsigned)a.num_pages) continue;
            const uint16_t *src = (op ? a.v_new : a.k_new) + ((size_t)(s * R + rr) * a.Hkv + kvh) * D + 8 * pc;
            uint16_t *dst = const_cast<uint16_t *>(op ? a.v_pages : a.k_pages) +
                            (((size_t)pg * a.Hkv + kvh) * a.P + off) * D + 8 * pc;
            *reinterpret_cast<u32x4 *>(dst) = *reinterpret_cast<const u32x4 *>(src);
        }
    };
    const int r_first = v0 / G;
    const int r_last = (min(NQ, v0 + M) - 1) / G;
    const int p_first = L - R + r_first, p_last = L - R + r_last;
    // a split is a chunk of absolute positions; a direct call's one split starts at the tile's
    // first visible key, and its chunk (>= window + R - 1, or >= max_seq_len) then covers every
    // key the tile's rows see
    const KeyRange keys = mfma_keys(L, R, W, CH, split, a.direct != 0, r_first, r_last);
    const int kbeg = keys.kbeg, kend = keys.kend;
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
        if constexpr (DMA) put_rows(tid, NTH);
        return;
    }
    const int lo_full = W > 0 ? p_last - W + 1 : 0;   // every column sees keys >= this ...
    // ... and <= this (with a tree-shaped window, only the keys before the window)
    const int hi_full = a.tree ? min(p_first, L - R - 1) : p_first;
    const int win0 = L - R;                           // first slot of the window
    int p_col[QW], lo_col[QW];
#pragma unroll
    for (int b = 0; b < QW; ++b) {
        p_col[b] = L - R + rq[b];
        lo_col[b] = W > 0 ? p_col[b] - W + 1 : 0;
    }

    // a wave whose query columns all lie past the tile's vectors (a partly filled tile: 4 rows
    // x GQA 8 leaves waves 2 and 3 without columns) stages its share and passes every barrier,
    // but computes nothing
    const bool wave_live = v0 + wave * QW * 16 < NQ;

    const int P = a.P;
    const int kt_first = (kbeg / KT) * KT;
    const int nt = (kend - kt_first + KT - 1) / KT;     // KT-key sub-tiles
    // otherwise the entries from the logical page of the split's first tile on
    const int idx0 = whole ? 0 : kt_first / P;
    if (MODE != 2 && !whole) {
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
    constexpr int KBUF = KS * KT * KROW, VBUF = KS * D * KT / 4;
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
            const int pg = cached_page<TC>(t_lds, idx - idx0);
            const size_t base = (size_t)pg * page_elems + head_off + (size_t)(tb - idx * P + KPT * kq) * D + 8 * kc;
#pragma unroll
            for (int u = 0; u < KPT; ++u) r[u] = ld16(pages + base + (size_t)u * D);
        } else if (MODE == 1 && D == 512 && P >= KPT) {
            // the thread's KPT consecutive keys lie in at most two pages: one division and two
            // table lookups serve all of them.  A d 512 workgroup runs one wave per SIMD, with
            // nothing to hide a per-key division and 64-bit address behind (the 4-row verify at
            // 9,000 keys over pages of 37: warm 27.1 -> 25.4 us, cold part kernel 28.9 -> 28.0);
            // at d 128, two waves per SIMD, the per-key form measured faster (51.1 against
            // 53.7 us over pages of 37).
            const int j0 = tb + KPT * kq;
            const int i0 = j0 / P;
            const int off0 = j0 - i0 * P;
            const uint16_t *const pa =
                pages + (size_t)cached_page<TC>(t_lds, i0 - idx0) * page_elems + head_off + 8 * kc;
            const uint16_t *const pb =
                pages + (size_t)cached_page<TC>(t_lds, i0 + 1 - idx0) * page_elems + head_off + 8 * kc;
#pragma unroll
            for (int u = 0; u < KPT; ++u) {
                const int off = off0 + u;
                const bool next = off >= P;
                r[u] = ld16((next ? pb : pa) + (next ? off - P : off) * D);
            }
        } else {
#pragma unroll
            for (int u = 0; u < KPT; ++u) {
                const int j = tb + KPT * kq + u;
                int idx = j / P;
                const int off = j - idx * P;
                int pg;
                if (MODE == 1) {
                    pg = cached_page<TC>(t_lds, idx - idx0);
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
    // DMA: a tile is kept as 256-byte rows; LDS piece p of row r holds the row's 16-byte piece
    // p ^ f(r), f = r & 15 for K and 2 (r & 7) for V (V's 32-byte halves of 16 channels stay
    // whole).  This lane's byte offsets of its operand reads:
    //  - K: row 16 nb + col, piece 4 kb + grp, which sits at piece (4 kb + grp) ^ col;
    //  - V^T: row 4 grp + (col >> 2) (+ 32 pm + 16 hh), channels 16 cb + 4 (col & 3).
    int k_rd[NKB], v_rd[NCB];
    if constexpr (DMA) {
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) k_rd[kb] = col * 2 * D + 16 * ((4 * kb + grp) ^ col);
        const int vr = 4 * grp + (col >> 2);
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) v_rd[cb] = vr * 2 * D + 32 * (cb ^ (vr & 7)) + 8 * (col & 3);
    }

    // Step it covers sub-tiles KS it .. KS it + KS - 1; loads past the last sub-tile reread it
    // (in bounds, never computed on), and sub-tiles past it are all masked out.
    const int kt_last = kt_first + (nt - 1) * KT;
    const int nsteps = (nt + KS - 1) / KS;
    auto ts_of = [&](int it) { return kt_first + (it * KS + ksub) * KT; };
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
        const int ts = ts_of(it);                                 // sub-tile this thread stages
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
    // compute step it's sub-tile of this wave from buffer buf
    // S^T of step it's sub-tile for this wave's query columns, from K buffer buf; each K
    // fragment feeds QW MFMAs (a padded step past the split computes nothing)
    auto qk = [&](int it, int buf, f32x4_t (&sacc)[QW][NB]) {
        const int tb = ts_of(it);                                 // sub-tile this wave computes
        if (tb >= kend || !wave_live) return;
        const uint16_t *const k_lds = k_st0 + buf * KBUF;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
            for (int b = 0; b < QW; ++b) sacc[b][nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) {
                bf16x8_t kf;
                if constexpr (DMA)
                    kf = *reinterpret_cast<const bf16x8_t *>(reinterpret_cast<const char *>(k_lds) + k_rd[kb] + 4096 * nb);
                else
                    kf = *reinterpret_cast<const bf16x8_t *>(k_lds + (16 * nb + col) * KRS + 32 * kb + 8 * grp);
#pragma unroll
                for (int b = 0; b < QW; ++b) sacc[b][nb] = mfma16(kf, qf[b][kb], sacc[b][nb]);
            }
        }
    };
    // mask, online softmax and O^T += V^T P^T of step it's sub-tile, from its scores and V
    // buffer buf
    auto smpv = [&](int it, int buf, f32x4_t (&sacc)[QW][NB]) {
        const int tb = ts_of(it);
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
        if constexpr (DMA) {
            // rows 32 pm + 4 grp + {0..3} and 32 pm + 16 + 4 grp + {0..3} of channel 16 cb + col,
            // two transposed reads per operand
            const char *vb = reinterpret_cast<const char *>(vt_lds);
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb) {
#pragma unroll
                for (int pm = 0; pm < NPM; ++pm) {
                    const v4i16_t lo = lds_read_tr16(vb + v_rd[cb] + 256 * (32 * pm));
                    const v4i16_t hi = lds_read_tr16(vb + v_rd[cb] + 256 * (32 * pm + 16));
                    const uint2 l2 = __builtin_bit_cast(uint2, lo), h2 = __builtin_bit_cast(uint2, hi);
                    const bf16x8_t vv = __builtin_bit_cast(bf16x8_t, u32x4{l2.x, l2.y, h2.x, h2.y});
#pragma unroll
                    for (int b = 0; b < QW; ++b) o[b][cb] = mfma16(vv, pf[b][pm], o[b][cb]);
                }
            }
        } else if constexpr (D == 128) {
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
    if constexpr (DMA) {
        // The same pipeline with the loads going straight to LDS: step it computes the scores
        // of step it + 1 and the softmax and PV of step it, while the loading waves bring K of
        // step it + 2 and V of step it + 1 into the buffers whose last readers finished before
        // the previous barrier; they wait for their loads before each barrier.  (With every
        // wave issuing its share of a step's loads at the step's start, the 2,048-token prompt
        // took 111.5 µs against 99.5 µs now; spreading those loads over the step's MFMAs took
        // 117.5 µs.)
        if (producer) {
            // loads of sub-tile psub of step it of one operand into LDS rows at sub (16 loads of
            // 4 rows, the pieces permuted through each lane's source address); V rows of keys
            // outside [kbeg, kend) are zeroed once they have landed (unused slots may hold NaN,
            // which a zero weight would not cancel)
            char *const pk0 = reinterpret_cast<char *>(k_lds_all[0][psub]), *const pk1 = reinterpret_cast<char *>(k_lds_all[1][psub]);
            char *const pv0 = reinterpret_cast<char *>(vt_lds_all[0][psub]), *const pv1 = reinterpret_cast<char *>(vt_lds_all[1][psub]);
            // with the row write fused, keys from L - R on (the call's own rows) come from
            // k_new / v_new [S][R][Hkv][D]; a key past the stream (tail of the last sub-tile,
            // masked) rereads row R - 1
            const int new0 = L - R;
            // Per-lane part of a load's source offset: the lane's row within its group of 4
            // (lane >> 4) and its permuted piece.  prow0 is a multiple of 16, so the
            // permutation of load j repeats every 4 loads for K (row & 15) and every 2 for V
            // (2 (row & 7)); a load's address is then a wave-uniform base plus one of these,
            // about 2 VALU instructions per load instead of 7.  Split calls (which the loads
            // bound) use them: the verify window, warm 37.6-37.8 -> 35.5-35.8 us, cold part
            // kernel 33.9-34.4 -> 32.9-33.5 us; prompt chunks, which the math bounds, measured
            // 1 us slower per prompt with them and keep the per-load form.
            static_assert((KT / LPS) % 16 == 0, "rows of a loading wave start at a multiple of 16");
            int pk_off[4], pv_off[2];
#pragma unroll
            for (int q = 0; q < 4; ++q) pk_off[q] = 16 * ((lane & 15) ^ ((4 * q + (lane >> 4)) & 15));
#pragma unroll
            for (int q = 0; q < 2; ++q) pv_off[q] = 16 * ((lane & 15) ^ (2 * ((4 * q + (lane >> 4)) & 7)));
            const int lrow = (lane >> 4) * 2 * D;
            auto poff = [&](int j, bool is_v) { return is_v ? pv_off[j & 1] : pk_off[j & 3]; };
            auto pload = [&](int it, const uint16_t *pages, char *sub, bool is_v) {
                const int ts = kt_first + (it * KS + psub) * KT;
                if (ts >= kend) return;
                const int idx = (int)((unsigned)ts / (unsigned)P);
                const int pg = __builtin_amdgcn_readfirstlane(cached_page<TC>(t_lds, idx - idx0));
                const char *base = reinterpret_cast<const char *>(pages + (size_t)pg * page_elems + head_off +
                                                                  (size_t)(ts - idx * P) * D);
                if (a.k_new != nullptr && ts + KT > new0) {
                    const char *nb = reinterpret_cast<const char *>((is_v ? a.v_new : a.k_new) +
                                                                    ((size_t)s * R * a.Hkv + kvh) * D);
                    const size_t rs = (size_t)a.Hkv * 2 * D;          // bytes from one new row to the next
                    if (ts >= new0 && ts + KT <= L) {
                        // the whole sub-tile is new rows: one base, as for a page
                        if constexpr (DEEP) {
                            const char *nt = nb + (size_t)(ts - new0 + prow0) * rs;
                            const int lnew = (lane >> 4) * (int)rs;
#pragma unroll
                            for (int j = 0; j < KT / 4 / LPS; ++j)
                                load_to_lds<NTL>(nt + (size_t)(4 * j) * rs + (lnew + poff(j, is_v)),
                                                 sub + (prow0 + 4 * j) * 2 * D);
                        } else {
                            const char *nt = nb + (size_t)(ts - new0) * rs;
#pragma unroll
                            for (int j = 0; j < KT / 4 / LPS; ++j) {
                                const int r = prow0 + 4 * j + (lane >> 4);
                                const int piece = (lane & 15) ^ (is_v ? 2 * (r & 7) : (r & 15));
                                load_to_lds<NTL>(nt + r * rs + 16 * piece, sub + (prow0 + 4 * j) * 2 * D);
                            }
                        }
                        return;
                    }
#pragma unroll
                    for (int j = 0; j < KT / 4 / LPS; ++j) {
                        const int r = prow0 + 4 * j + (lane >> 4);
                        const int piece = (lane & 15) ^ (is_v ? 2 * (r & 7) : (r & 15));
                        const int key = ts + r;
                        const char *src = key >= new0
                                              ? nb + (size_t)min(key - new0, R - 1) * rs + 16 * piece
                                              : base + r * 2 * D + 16 * piece;
                        load_to_lds<NTL>(src, sub + (prow0 + 4 * j) * 2 * D);
                    }
                    return;
                }
                if constexpr (DEEP) {
                    const char *bp = base + prow0 * 2 * D;
#pragma unroll
                    for (int j = 0; j < KT / 4 / LPS; ++j)
                        load_to_lds<NTL>(bp + 4 * j * 2 * D + (lrow + poff(j, is_v)), sub + (prow0 + 4 * j) * 2 * D);
                } else {
#pragma unroll
                    for (int j = 0; j < KT / 4 / LPS; ++j) {
                        const int r = prow0 + 4 * j + (lane >> 4);
                        const int piece = (lane & 15) ^ (is_v ? 2 * (r & 7) : (r & 15));
                        load_to_lds<NTL>(base + r * 2 * D + 16 * piece, sub + (prow0 + 4 * j) * 2 * D);
                    }
                }
            };
            auto pfix = [&](int it, char *sub) {
                const int ts = kt_first + (it * KS + psub) * KT;
                if (ts >= kend || (ts >= kbeg && ts + KT <= kend)) return;
#pragma unroll
                for (int j = 0; j < KT / 4 / LPS; ++j) {
                    const int key = ts + prow0 + 4 * j + (lane >> 4);
                    if (key < kbeg || key >= kend)
                        *reinterpret_cast<u32x4 *>(sub + (prow0 + 4 * j) * 2 * D + 16 * lane) = u32x4{0u, 0u, 0u, 0u};
                }
            };
            if constexpr (DEEP) {
                // Four buffers per operand: in step j the computing waves read K(j + 1) and
                // V(j), while K(j + 4) and V(j + 3) are issued into the buffers of K(j) and
                // V(j - 1), and the wait is for K(j + 2) and V(j + 1), issued two steps before:
                // the 4 newest groups of NL loads of this wave may stay in flight when all of them
                // were issued in full, else every load is waited for (with four loading waves
                // NL is 4; two, which issue the same loads at the same cold time, would make it 8).
                auto kb = [&](int i) { return reinterpret_cast<char *>(k_lds_all[i & (NBUF - 1)][psub]); };
                auto vb = [&](int i) { return reinterpret_cast<char *>(vt_lds_all[i & (NBUF - 1)][psub]); };
                constexpr int NL = KT / 4 / LPS;   // loads per wave, operand and step
                static_assert(6 * NL < 64, "vmcnt range");
                const bool ahead = nsteps >= 5;
                pload(0, a.k_pages, kb(0), false);
                pload(1, a.k_pages, kb(1), false);
                pload(0, a.v_pages, vb(0), true);
                pload(2, a.k_pages, kb(2), false);
                pload(1, a.v_pages, vb(1), true);
                pload(3, a.k_pages, kb(3), false);
                pload(2, a.v_pages, vb(2), true);
                if (ahead) wait_vmcnt<6 * NL>(); else wait_vmem();    // K(0)
                loader_barrier();
                if (ahead) wait_vmcnt<4 * NL>(); else wait_vmem();    // K(1), V(0)
                pfix(0, vb(0));
                loader_barrier();   // the computing waves' scores of step 0
                for (int it = 0; it < nsteps; it += 2) {
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        const int j = it + h;
                        pload(j + 4, a.k_pages, kb(j + 4), false);
                        pload(j + 3, a.v_pages, vb(j + 3), true);
                        if (j + 4 <= nsteps - 2) wait_vmcnt<4 * NL>(); else wait_vmem();   // K(j + 2), V(j + 1)
                        pfix(j + 1, vb(j + 1));
                        loader_barrier();
                    }
                }
                put_rows(tid - 512, 64 * kLoadWaves);
                lds_fence();   // the two barriers of the key groups' combine
                lds_fence();
                return;
            }
            pload(0, a.k_pages, pk0, false);
            pload(1, a.k_pages, pk1, false);
            pload(0, a.v_pages, pv0, true);
            wait_vmem();
            pfix(0, pv0);
            lds_fence();
            lds_fence();   // the computing waves' scores of step 0
            for (int it = 0; it < nsteps; it += 2) {
                pload(it + 2, a.k_pages, pk0, false);
                pload(it + 1, a.v_pages, pv1, true);
                wait_vmem();
                pfix(it + 1, pv1);
                lds_fence();
                pload(it + 3, a.k_pages, pk1, false);
                pload(it + 2, a.v_pages, pv0, true);
                wait_vmem();
                pfix(it + 2, pv0);
                lds_fence();
            }
            put_rows(tid - 512, 64 * kLoadWaves);
            lds_fence();   // the two barriers of the key groups' combine
            lds_fence();
            return;
        }
        lds_fence();   // step 0's tiles have landed
        f32x4_t s0[QW][NB], s1[QW][NB];
        qk(0, 0, s0);
        lds_fence();   // K buffer 0 is loaded again next
        for (int it = 0; it < nsteps; it += 2) {
            qk(it + 1, (it + 1) & (NBUF - 1), s1);
            smpv(it, it & (NBUF - 1), s0);
            lds_fence();
            qk(it + 2, (it + 2) & (NBUF - 1), s0);
            smpv(it + 1, (it + 1) & (NBUF - 1), s1);
            lds_fence();
        }
    } else if constexpr (NBUF == 2) {
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
        // the first iteration stages K(2) into K buffer 0, which qk(0) has just read: every
        // wave must be done with it first (later iterations write a buffer only after a barrier
        // that follows its last read)
        lds_fence();
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
        static_assert(NF * 256 * 4 <= NBUF * KS * KT * KROW * 2, "exchange fits the K tiles");
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

// ---------------------------------------------------------------------------------------------
// d 512 with at most 32 query vectors per KV head (verify windows of a few rows): the
// channel-split kernel.  TensorFold PR #1620, per-tile follow-up (the head-dim-512 layer's
// verify rows, timed alone with a cold L2).
//
// With 16 or 32 query vectors the tile kernel above leaves two of its four waves idle, and each
// live wave takes both products over all 512 channels at one wave per SIMD, a chain of 64 MFMAs
// per 32-key tile, each waiting on its own LDS read.  Here wave w owns channels
// 128 w .. 128 w + 127 of the queries, keys and values:
//  * S^T = K Q^T over the wave's channels, with K loaded from memory straight into the A-operand
//    registers (lane: key 16 nb + col, 8 channels of its lane group), no LDS;
//  * the four waves' partial scores are added through LDS in one fixed order, so every wave
//    holds the same full scores, runs the same online softmax on them and gets the same bits;
//  * O^T += V^T P^T for the wave's 128 output channels: each wave loads its own 256-byte slice
//    of the tile's V rows straight into LDS (rows of 256 bytes, 16-byte pieces permuted as in the
//    d 128 direct-to-LDS layout) and reads V^T back with transposing reads.
// Tiles stream through a ring of three buffers, the next one in flight while one is computed.
// Pages hold at least 32 keys, so a tile lies in at most two pages: one division and two cached
// table entries per tile.  MODE 0: P % 32 == 0, one page per tile.
// Measured on the 4-row verify at 9,000 keys over pages of 37 (188 workgroups, one per CU): cold
// part kernel 20.9-21.0 us with nontemporal loads (26.9-27.2 with plain ones) against
// 27.4-27.8 for the tile kernel.  Each workgroup streams 192 KB of K/V; a plain read of the same
// bytes with the same grid and bytes per workgroup takes 17.4-18.1 us cold, so at this shape
// the CU's streaming rate (about 21 GB/s per CU with every workgroup loading) bounds the call,
// not the math.

template <int QB, int MODE>
__global__ __launch_bounds__(256) void part_narrow_kernel(const PartArgs a) {
    constexpr int D = 512, KT = 32, CW = 128;   // keys per tile, channels per wave
    constexpr int NKB = CW / 32;                // QK k-steps per wave
    constexpr int NCB = CW / 16;                // PV output blocks per wave
    constexpr int NBT = kNarrowTiles;
    constexpr int TC = kTableCache;
    constexpr int NF = 2 * QB;                  // score fragments per lane (query x key blocks)
    __shared__ __attribute__((aligned(16))) char v_lds[NBT][4][KT * CW * 2];
    __shared__ __attribute__((aligned(16))) f32x4_t xch[2][4][NF][64];
    __shared__ int32_t t_lds[TC];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int col = lane & 15, grp = lane >> 4;
    // work items (stream, KV head, split) in XCD order, as in the tile kernel
    const int item = (blockIdx.x & 7) * a.per_xcd + (blockIdx.x >> 3);
    if (item >= a.S * a.Hkv * a.n_splits) return;
    const int split = item % a.n_splits;
    const int kvh = (item / a.n_splits) % a.Hkv;
    const int s = item / (a.n_splits * a.Hkv);
    const int R = a.R, W = a.window, CH = a.chunk;
    const int G = a.Hq / a.Hkv;
    const int NQ = R * G;
    const int32_t *trow = a.table + (size_t)s * a.stride;

    // queries of this wave's channels as the B operand (column 16 b + col, channels
    // 128 wave + 32 kb + 8 grp .. + 8), issued together with the length and, for a full layer
    // whose table fits the cache, the table entries
    const bool whole = whole_table(MODE, a.ring_pages, a.stride);
    const int Lv = load_uniform_i32(a.seq_len + s);
    bool col_ok[QB];
    int rq[QB], hq[QB];
    uint32_t anc[QB];
    bf16x8_t qf[QB][NKB];
#pragma unroll
    for (int b = 0; b < QB; ++b) {
        const int vq = 16 * b + col;
        col_ok[b] = vq < NQ;
        rq[b] = col_ok[b] ? vq / G : 0;
        hq[b] = kvh * G + (col_ok[b] ? vq % G : 0);
        anc[b] = a.tree ? a.tree[s * R + rq[b]] : 0xFFFFFFFFu;
        const uint16_t *qrow = a.q + ((size_t)(s * R + rq[b]) * a.Hq + hq[b]) * D + CW * wave + 8 * grp;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
            u32x4 x = *reinterpret_cast<const u32x4 *>(qrow + 32 * kb);
            if (!col_ok[b]) x = u32x4{0, 0, 0, 0};
            qf[b][kb] = __builtin_bit_cast(bf16x8_t, x);
        }
    }
    constexpr int TPT = (TC + 255) / 256;
    int tv[TPT];
    if (whole) {
#pragma unroll
        for (int k = 0; k < TPT; ++k) {
            const int i = tid + k * 256;
            tv[k] = i < a.stride ? trow[i] : -1;
        }
    }
    const int L = kernel_len(__builtin_amdgcn_readfirstlane(Lv), a.max_len);
    if (whole) {
#pragma unroll
        for (int k = 0; k < TPT; ++k) {
            const int i = tid + k * 256;
            if (i < TC) t_lds[i] = ((unsigned)tv[k] < (unsigned)a.num_pages) ? tv[k] : -1;
        }
    }
    const int p_first = L - R, p_last = L - 1;
    const KeyRange keys = mfma_keys(L, R, W, CH, split, false, 0, R - 1);
    const int kbeg = keys.kbeg, kend = keys.kend;
    if (kbeg >= kend) return;   // no row sees this chunk: nothing to merge
    const int lo_full = W > 0 ? p_last - W + 1 : 0;
    const int hi_full = a.tree ? min(p_first, L - R - 1) : p_first;
    const int win0 = L - R;
    int p_col[QB], lo_col[QB];
#pragma unroll
    for (int b = 0; b < QB; ++b) {
        p_col[b] = L - R + rq[b];
        lo_col[b] = W > 0 ? p_col[b] - W + 1 : 0;
    }
    const int P = a.P;
    const int kt_first = (kbeg / KT) * KT;
    const int nt = (kend - kt_first + KT - 1) / KT;
    const int idx0 = whole ? 0 : kt_first / P;
    if (!whole) {
        for (int i = tid; i < TC; i += 256) {
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
    // Issue the loads of tile t (absolute start kt_first + 32 t) into K register set kr and V
    // buffer vb: rows r < sp lie in page pa at offset off0 + r, the others in page pb at r - sp.
    // 8 K loads (this lane's two key rows x four k-steps), then 8 V loads into LDS, all
    // nontemporal: every K/V byte of the call is read once (4-row verify at 9,000 keys, cold
    // part kernel 26.7-26.8 -> 20.9-21.0 us, whole call 32.0 -> 25.9 us; calls repeated back to
    // back on the same keys, whose K/V could stay in the caches, 21.4 -> 25.2 us).
    auto issue = [&](int t, u32x4 (&kr)[2][NKB], char *vb) {
        const int tb = kt_first + KT * t;
        const int idx = tb / P;
        const int off0 = tb - idx * P;
        const int pga = __builtin_amdgcn_readfirstlane(cached_page<TC>(t_lds, idx - idx0));
        const int pgb = MODE == 0 ? pga : __builtin_amdgcn_readfirstlane(cached_page<TC>(t_lds, idx + 1 - idx0));
        const size_t ea = (size_t)pga * page_elems + head_off + (size_t)off0 * D;
        const size_t eb = (size_t)pgb * page_elems + head_off;
        const int sp = MODE == 0 ? KT : P - off0;
        auto row = [&](int r) { return r < sp ? ea + (size_t)r * D : eb + (size_t)(r - sp) * D; };
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
            const uint16_t *kp = a.k_pages + row(16 * nb + col) + CW * wave + 8 * grp;
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) kr[nb][kb] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(kp + 32 * kb));
        }
#pragma unroll
        for (int j = 0; j < KT / 4; ++j) {
            const int r = 4 * j + grp;
            const int piece = (lane & 15) ^ (2 * (r & 7));
            const char *src = reinterpret_cast<const char *>(a.v_pages + row(r) + CW * wave) + 16 * piece;
            load_to_lds<true>(src, vb + 4 * j * 2 * CW);
        }
    };

    f32x4_t o[QB][NCB];
    float m_run[QB], l_run[QB];
#pragma unroll
    for (int b = 0; b < QB; ++b) {
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) o[b][cb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        m_run[b] = -INFINITY;
        l_run[b] = 0.f;
    }
    const float c2 = a.scale_log2;
    const float slack = fminf(8.0f / c2, 3.0e38f);
    const bf16x8_t ones8 = __builtin_bit_cast(bf16x8_t, u32x4{0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u});
    // V^T operand reads: rows 4 grp + (col >> 2) (+ 16), channels 16 cb + 4 (col & 3) of the
    // wave's slice (the d 128 direct-to-LDS layout)
    int v_rd[NCB];
    {
        const int vr = 4 * grp + (col >> 2);
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) v_rd[cb] = vr * 2 * CW + 32 * (cb ^ (vr & 7)) + 8 * (col & 3);
    }

    // one tile: scores over the wave's channels, their sum over the waves, mask, online softmax,
    // PV into the wave's output channels
    auto compute = [&](int t, const u32x4 (&kr)[2][NKB], const char *vb) {
        const int tb = kt_first + KT * t;
        f32x4_t sacc[QB][2];
#pragma unroll
        for (int b = 0; b < QB; ++b)
#pragma unroll
            for (int nb = 0; nb < 2; ++nb) {
                sacc[b][nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kb = 0; kb < NKB; ++kb)
                    sacc[b][nb] = mfma16(__builtin_bit_cast(bf16x8_t, kr[nb][kb]), qf[b][kb], sacc[b][nb]);
            }
        const int par = t & 1;
#pragma unroll
        for (int b = 0; b < QB; ++b)
#pragma unroll
            for (int nb = 0; nb < 2; ++nb) xch[par][wave][2 * b + nb][lane] = sacc[b][nb];
        // the waves' partial scores are in LDS (V loads stay in flight); with two exchange
        // buffers a wave writes buffer par again only after the next barrier, which every wave
        // passes after its reads of this one
        loader_barrier();
#pragma unroll
        for (int b = 0; b < QB; ++b)
#pragma unroll
            for (int nb = 0; nb < 2; ++nb) {
                const f32x4_t x0 = xch[par][0][2 * b + nb][lane], x1 = xch[par][1][2 * b + nb][lane];
                const f32x4_t x2 = xch[par][2][2 * b + nb][lane], x3 = xch[par][3][2 * b + nb][lane];
                sacc[b][nb] = (x0 + x1) + (x2 + x3);
            }
        const bool full = tb >= kbeg && tb + KT <= kend && tb + KT - 1 <= hi_full && tb >= lo_full;
        bf16x8_t pf[QB];
#pragma unroll
        for (int b = 0; b < QB; ++b) {
            float tmax = -INFINITY;
            if (full) {
#pragma unroll
                for (int nb = 0; nb < 2; ++nb)
#pragma unroll
                    for (int r = 0; r < 4; ++r) tmax = fmaxf(tmax, sacc[b][nb][r]);
            } else {
#pragma unroll
                for (int nb = 0; nb < 2; ++nb)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int j = tb + 16 * nb + 4 * grp + r;
                        const int tw = j - win0;
                        const bool vis = col_ok[b] & (j >= kbeg) & (j < kend) & (j <= p_col[b]) & (j >= lo_col[b]) &
                                         ((tw < 0) | (((anc[b] >> (tw & 31)) & 1u) != 0));
                        const float x = vis ? sacc[b][nb][r] : -INFINITY;
                        sacc[b][nb][r] = x;
                        tmax = fmaxf(tmax, x);
                    }
            }
            if (__builtin_amdgcn_ballot_w64(tmax > m_run[b] + slack)) {
                tmax = fmaxf(tmax, __shfl_xor(tmax, 16));
                tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
                const float m_new = fmaxf(m_run[b], tmax);
                const float mc_new = (m_new == -INFINITY) ? 0.f : m_new * c2;
                const float alpha = fast_exp2(m_run[b] * c2 - mc_new);
                m_run[b] = m_new;
                l_run[b] *= alpha;
                if (alpha != 1.f) {
#pragma unroll
                    for (int cb = 0; cb < NCB; ++cb) o[b][cb] *= alpha;
                }
            }
            const float mc = (m_run[b] == -INFINITY) ? 0.f : m_run[b] * c2;
#pragma unroll
            for (int hh = 0; hh < 2; ++hh)
#pragma unroll
                for (int r = 0; r < 4; ++r) pf[b][4 * hh + r] = (__bf16)fast_exp2(__builtin_fmaf(sacc[b][hh][r], c2, -mc));
            const f32x4_t ls = mfma16(ones8, pf[b], f32x4_t{0.f, 0.f, 0.f, 0.f});
            l_run[b] += ls[0];
        }
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) {
            const v4i16_t lo = lds_read_tr16(vb + v_rd[cb]);
            const v4i16_t hi = lds_read_tr16(vb + v_rd[cb] + 16 * 2 * CW);
            const uint2 l2 = __builtin_bit_cast(uint2, lo), h2 = __builtin_bit_cast(uint2, hi);
            const bf16x8_t vv = __builtin_bit_cast(bf16x8_t, u32x4{l2.x, l2.y, h2.x, h2.y});
#pragma unroll
            for (int b = 0; b < QB; ++b) o[b][cb] = mfma16(vv, pf[b], o[b][cb]);
        }
    };
    // zero the rows of V buffer vb (tile t, loaded by this lane) outside [kbeg, kend): unused
    // slots may hold NaN, which a zero weight would not cancel
    auto vfix = [&](int t, char *vb) {
        const int tb = kt_first + KT * t;
        if (tb >= kbeg && tb + KT <= kend) return;
#pragma unroll
        for (int j = 0; j < KT / 4; ++j) {
            const int key = tb + 4 * j + grp;
            if (key < kbeg || key >= kend) *reinterpret_cast<u32x4 *>(vb + 4 * j * 2 * CW + 16 * lane) = u32x4{0u, 0u, 0u, 0u};
        }
    };

    // A ring of three tiles (K register sets k0..k2, V buffers vb0..vb2; tile t in set t mod 3).
    // Tile t + 2 is issued right after tile t is computed, into the set tile t - 1 used, so one
    // tile streams in while one is computed.  A wave whose loads fill the CU's memory queue
    // stalls at issue until data returns, and the score exchange makes every wave wait for the
    // slowest one: issuing further ahead only moves the compute behind the stream (tile t + 2
    // issued before tile t is computed: cold part kernel of the 4-row verify at 9,000 keys
    // 26.9-27.2 us).  The main loop issues only tiles inside the chunk and waits for a fixed
    // count (the 16 loads of the next tile stay in flight); the tail (at most four tiles)
    // spells out its waits.
    u32x4 k0[2][NKB], k1[2][NKB], k2[2][NKB];
    char *const vb0 = v_lds[0][wave], *const vb1 = v_lds[1][wave], *const vb2 = v_lds[2][wave];
    auto fence = [] { asm volatile("" ::: "memory"); };
    issue(0, k0, vb0);
    fence();
    issue(min(1, nt - 1), k1, vb1);   // a chunk of one tile rereads it
    fence();
    int t = 0;
    for (; t + 5 <= nt; t += 3) {
        wait_vmcnt<16>();
        fence();
        vfix(t, vb0);
        compute(t, k0, vb0);
        issue(t + 2, k2, vb2);
        fence();
        wait_vmcnt<16>();
        fence();
        vfix(t + 1, vb1);
        compute(t + 1, k1, vb1);
        issue(t + 3, k0, vb0);
        fence();
        wait_vmcnt<16>();
        fence();
        vfix(t + 2, vb2);
        compute(t + 2, k2, vb2);
        issue(t + 4, k1, vb1);
        fence();
    }
    // tail: tiles t .. nt - 1 (1 to 4 of them); t and t + 1 (or t again) are issued
    const int rem = nt - t;
    wait_vmcnt<16>();
    fence();
    vfix(t, vb0);
    compute(t, k0, vb0);
    if (rem >= 3) issue(t + 2, k2, vb2);
    fence();
    if (rem >= 2) {
        if (rem >= 3) wait_vmcnt<16>(); else wait_vmem();
        fence();
        vfix(t + 1, vb1);
        compute(t + 1, k1, vb1);
    }
    if (rem >= 4) issue(t + 3, k0, vb0);
    fence();
    if (rem >= 3) {
        if (rem >= 4) wait_vmcnt<16>(); else wait_vmem();
        fence();
        vfix(t + 2, vb2);
        compute(t + 2, k2, vb2);
    }
    if (rem >= 4) {
        wait_vmem();
        fence();
        vfix(t + 3, vb0);
        compute(t + 3, k0, vb0);
    }
    wait_vmem();   // a one-tile chunk's reread
    fence();

    // partials: this wave's 128 channels of each column, (m, l) from wave 0
#pragma unroll
    for (int b = 0; b < QB; ++b) {
        if (!col_ok[b]) continue;
        const size_t slot = ((size_t)(s * R + rq[b]) * a.Hq + hq[b]) * a.n_splits + split;
        float *dst = a.ws_acc + slot * D + CW * wave + 4 * grp;
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb)
            *reinterpret_cast<float4 *>(dst + 16 * cb) = make_float4(o[b][cb][0], o[b][cb][1], o[b][cb][2], o[b][cb][3]);
        if (wave == 0 && grp == 0) {
            const float m2 = m_run[b] == -INFINITY ? -INFINITY : m_run[b] * c2;
            *reinterpret_cast<float2 *>(a.ws_ml + slot * 2) = make_float2(m2, l_run[b]);
        }
    }
}

template <int D, int G, int QW, int KS, bool NTL>
static hipError_t launch_dgq(const PartArgs &a, hipStream_t st) {
    using Geo = MfmaGeom<D>;
    const dim3 grid(8 * a.per_xcd);
    switch (table_mode(a.P, a.chunk, Geo::KT, 1)) {
        case 0:
            // at d 128, pages holding whole tiles: loads straight into LDS
            if constexpr (D == 128) {
                // split calls (verify windows) stream their keys from HBM: deeper prefetch
                if (a.direct)
                    hipLaunchKernelGGL((part_mfma_kernel<D, G, QW, 0, KS, NTL, true>), grid, dim3(256 * KS + 64 * kLoadWaves),
                                       0, st, a);
                else
                    hipLaunchKernelGGL((part_mfma_kernel<D, G, QW, 0, KS, NTL, true, true>), grid,
                                       dim3(256 * KS + 64 * kLoadWaves), 0, st, a);
            }
            else
                hipLaunchKernelGGL((part_mfma_kernel<D, G, QW, 0, KS, NTL, false>), grid, dim3(256 * KS), 0, st, a);
            break;
        case 1: hipLaunchKernelGGL((part_mfma_kernel<D, G, QW, 1, KS, NTL, false>), grid, dim3(256 * KS), 0, st, a); break;
        default: hipLaunchKernelGGL((part_mfma_kernel<D, G, QW, 2, KS, NTL, false>), grid, dim3(256 * KS), 0, st, a); break;
    }
    return hipGetLastError();
}

template <int D, int G, int KS>
static hipError_t launch_dg(const PartArgs &a, hipStream_t st) {
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
    if (!p.direct && narrow_shape(D, a.R * G, a.P) && table_mode(a.P, a.chunk, 32, 32) != 2) {
        if (p.tiles != 1) return hipErrorInvalidValue;
        const dim3 grid(8 * a.per_xcd);
        const bool one = a.R * G <= 16;
        if (a.P % 32 == 0) {
            if (one) hipLaunchKernelGGL((part_narrow_kernel<1, 0>), grid, dim3(256), 0, st, a);
            else hipLaunchKernelGGL((part_narrow_kernel<2, 0>), grid, dim3(256), 0, st, a);
        } else {
            if (one) hipLaunchKernelGGL((part_narrow_kernel<1, 1>), grid, dim3(256), 0, st, a);
            else hipLaunchKernelGGL((part_narrow_kernel<2, 1>), grid, dim3(256), 0, st, a);
        }
        return hipGetLastError();
    }
    if (D == 128 && G == 4) return launch_dg<128, 4, 2>(a, st);
    if (D == 128 && G == 8) return launch_dg<128, 8, 2>(a, st);
    if (D == 128 && G == 12) return launch_dg<128, 12, 2>(a, st);
    if (D == 128 && G == 16) return launch_dg<128, 16, 2>(a, st);
    if (D == 256 && G == 4) return launch_dg<256, 4, 1>(a, st);
    if (D == 256 && G == 8) return launch_dg<256, 8, 1>(a, st);
    if (D == 256 && G == 12) return launch_dg<256, 12, 1>(a, st);
    if (D == 256 && G == 16) return launch_dg<256, 16, 1>(a, st);
    if (D == 512 && G == 4) return launch_dg<512, 4, 1>(a, st);
    if (D == 512 && G == 8) return launch_dg<512, 8, 1>(a, st);
    if (D == 512 && G == 12) return launch_dg<512, 12, 1>(a, st);
    if (D == 512 && G == 16) return launch_dg<512, 16, 1>(a, st);
    return hipErrorInvalidValue;
}

}  // namespace kvp
