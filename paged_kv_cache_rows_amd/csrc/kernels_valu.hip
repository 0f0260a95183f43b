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
    static constexpr int CHUNK = 16 * NB;     // keys per workgroup
    static constexpr int RS = D + 8;          // LDS row stride (bf16 elements)
    static constexpr int TC = 72;             // page-table entries cached per chunk
};

int valu_chunk(int D) { return D == 512 ? ValuGeom<512>::CHUNK : ValuGeom<128>::CHUNK; }

// Loads of one batch (16 rows per lane group, 16 bytes per lane per row).  Every load reads
// inside the pool: an absent page reads page 0 and an out-of-range row keeps its slot; rows
// outside the chunk are zeroed later, when V is staged.  The three modes are chosen by a
// wave-uniform value so that each loop is straight-line code.
template <int D>
struct BatchLoader {
    const uint16_t *k_pages, *v_pages;
    const int32_t *trow;
    const int32_t *t_lds;      // page-table entries of the chunk from logical page idx0 on
    size_t page_elems, head_off;
    int P, idx0, lrow, ring_pages, stride, num_pages;

    template <int MODE>
    __device__ __forceinline__ void load(int b, u32x4 (&kr)[16], u32x4 (&vr)[16]) const {
        constexpr int RPI = ValuGeom<D>::RPI;
        if constexpr (MODE == 0) {
            // the whole batch lies in one page: one lookup
            const int idx = b / P;
            const int pg = max(t_lds[idx - idx0], 0);
            const size_t base = (size_t)pg * page_elems + head_off + (size_t)(b - idx * P + lrow) * D;
#pragma unroll
            for (int t = 0; t < 16; ++t) {
                kr[t] = *reinterpret_cast<const u32x4 *>(k_pages + base + (size_t)(t * RPI) * D);
                vr[t] = *reinterpret_cast<const u32x4 *>(v_pages + base + (size_t)(t * RPI) * D);
            }
        } else if constexpr (MODE == 1) {
            // rows straddle pages: step RPI rows at a time, crossing at most one page boundary
            const int j0 = b + lrow;
            int idx = j0 / P;
            int off = j0 - idx * P;
#pragma unroll
            for (int t = 0; t < 16; ++t) {
                const int pg = max(t_lds[idx - idx0], 0);
                const size_t e = (size_t)pg * page_elems + head_off + (size_t)off * D;
                kr[t] = *reinterpret_cast<const u32x4 *>(k_pages + e);
                vr[t] = *reinterpret_cast<const u32x4 *>(v_pages + e);
                off += RPI;
                const bool wrap = off >= P;
                off = wrap ? off - P : off;
                idx += wrap ? 1 : 0;
            }
        } else {
            // tiny pages: divide per row and read the table from global memory
#pragma unroll
            for (int t = 0; t < 16; ++t) {
                const int j = b + t * RPI + lrow;
                int idx = j / P;
                const int off = j - idx * P;
                if (ring_pages) idx %= ring_pages;
                const int tp = trow[min(idx, stride - 1)];
                const int pg = (idx < stride && (unsigned)tp < (unsigned)num_pages) ? tp : 0;
                const size_t e = (size_t)pg * page_elems + head_off + (size_t)off * D;
                kr[t] = *reinterpret_cast<const u32x4 *>(k_pages + e);
                vr[t] = *reinterpret_cast<const u32x4 *>(v_pages + e);
            }
        }
    }
};

// Load modes, fixed per launch from P: 0 when P is a multiple of the batch, 1 when rows
// straddle pages but the chunk's table entries fit the LDS cache, 2 for tiny pages.
template <int D>
int valu_mode(int P) {
    using Geo = ValuGeom<D>;
    if (P % Geo::NB == 0) return 0;
    if ((Geo::CHUNK + Geo::NB) / P + 2 <= Geo::TC && Geo::RPI <= P) return 1;
    return 2;
}

template <int D, int G, int NQ, int MODE>
__global__ __launch_bounds__(64) void part_valu_kernel(const PartArgs a) {
    using Geo = ValuGeom<D>;
    constexpr int LPR = Geo::LPR, RPI = Geo::RPI, NB = Geo::NB, QL = Geo::QL, SEG = Geo::SEG;
    constexpr int CHUNK = Geo::CHUNK, RS = Geo::RS, TC = Geo::TC;
    constexpr int R = NQ / G;
    static_assert(NQ % G == 0 && NQ % 4 == 0, "query vectors come in whole rows of 4 or 8");

    __shared__ __attribute__((aligned(16))) uint16_t k_lds[NB * RS];
    __shared__ __attribute__((aligned(16))) uint16_t v_lds[NB * RS];
    __shared__ __attribute__((aligned(16))) uint16_t q_lds[NQ * RS];
    __shared__ __attribute__((aligned(16))) uint32_t p_lds[(NB / 2) * NQ];
    __shared__ int32_t t_lds[TC];

    const int lane = threadIdx.x;
    const int split = blockIdx.x, kvh = blockIdx.y, s = blockIdx.z;
    const int L = a.seq_len[s];
    const int W = a.window;
    const int lo = W > 0 ? max(0, L - R - W + 1) : 0;
    const int c0 = (lo / CHUNK + split) * CHUNK;
    if (L <= 0 || c0 >= L || split >= a.n_splits) return;
    const int kbeg = max(c0, lo);
    const int kend = min(c0 + CHUNK, L);

    // Queries of this KV head: vector v = r * G + g is row r, query head kvh * G + g.
    for (int i = lane; i < NQ * (D / 8); i += 64) {
        const int v = i / (D / 8), c = i - (i / (D / 8)) * (D / 8);
        const int r = v / G, g = v - (v / G) * G;
        const uint4 *src = reinterpret_cast<const uint4 *>(
            a.q + ((size_t)(s * R + r) * a.Hq + kvh * G + g) * D) + c;
        *reinterpret_cast<uint4 *>(q_lds + v * RS + c * 8) = *src;
    }

    const uint16_t *q_rows[NQ];
#pragma unroll
    for (int v = 0; v < NQ; ++v)
        q_rows[v] = a.q + ((size_t)(s * R + v / G) * a.Hq + kvh * G + (v % G)) * D;

    const int lrow = lane / LPR;            // row inside a group of RPI rows (load and PV)
    const int lch = lane - lrow * LPR;      // 16-byte piece of the row
    const size_t page_elems = (size_t)a.Hkv * a.P * D;
    const size_t head_off = (size_t)kvh * a.P * D + (size_t)lch * 8;
    const int32_t *trow = a.table + (size_t)s * a.stride;
    const int P = a.P;
    const int b_first = (kbeg / NB) * NB;

    // The chunk's page-table entries, looked up once per chunk into LDS (logical page index
    // idx0 + i); entries past the table or outside the pool become -1.
    const int idx0 = b_first / P;
    if (MODE != 2) {
        for (int i = lane; i < TC; i += 64) {
            int idx = idx0 + i;
            if (a.ring_pages) idx %= a.ring_pages;
            int pg = -1;
            if (idx < a.stride) pg = trow[idx];
            t_lds[i] = ((unsigned)pg < (unsigned)a.num_pages) ? pg : -1;
        }
    }
    lds_fence();
    BatchLoader<D> ld{a.k_pages, a.v_pages, trow, t_lds, page_elems, head_off, P, idx0, lrow,
                      a.ring_pages, a.stride, a.num_pages};
    u32x4 kr[16], vr[16];

    float m_run[NQ], l_run[NQ], acc[NQ][8];
#pragma unroll
    for (int v = 0; v < NQ; ++v) {
        m_run[v] = -INFINITY;
        l_run[v] = 0.f;
#pragma unroll
        for (int c = 0; c < 8; ++c) acc[v][c] = 0.f;
    }

    const int nb = (kend - b_first + NB - 1) / NB;
    const int kk = (QL == 1) ? lane : (lane % NB);     // key of this lane in the QK stage
    const int seg = (QL == 1) ? 0 : (lane / NB);       // its channel segment
    const float scale_log2 = a.scale_log2;

    ld.template load<MODE>(b_first, kr, vr);
    for (int ib = 0; ib < nb; ++ib) {
        const int b = b_first + ib * NB;
        lds_fence();
#pragma unroll
        for (int t = 0; t < 16; ++t)
            *reinterpret_cast<u32x4 *>(k_lds + (t * RPI + lrow) * RS + lch * 8) = kr[t];
        if (b >= kbeg && b + NB <= kend) {
#pragma unroll
            for (int t = 0; t < 16; ++t)
                *reinterpret_cast<u32x4 *>(v_lds + (t * RPI + lrow) * RS + lch * 8) = vr[t];
        } else {
            // a batch at the chunk's edge: V rows outside [kbeg, kend) become zeros, so that a
            // zero weight never meets a NaN in an unused slot
#pragma unroll
            for (int t = 0; t < 16; ++t) {
                const int j = b + t * RPI + lrow;
                const uint32_t keep = (j >= kbeg && j < kend) ? 0xFFFFFFFFu : 0u;
                *reinterpret_cast<u32x4 *>(v_lds + (t * RPI + lrow) * RS + lch * 8) = vr[t] & keep;
            }
        }
        if (ib + 1 < nb) ld.template load<MODE>(b + NB, kr, vr);
        lds_fence();

        // ---- scores: this lane's key against every query vector of the KV head
        float sc[NQ];
#pragma unroll
        for (int v = 0; v < NQ; ++v) sc[v] = 0.f;
        const uint16_t *krow = k_lds + kk * RS + seg * SEG;
        const uint16_t *qb = q_lds + seg * SEG;
#pragma unroll
        for (int cb = 0; cb < SEG / 8; ++cb) {
            const uint4 kv = *reinterpret_cast<const uint4 *>(krow + cb * 8);
#pragma unroll
            for (int v = 0; v < NQ; ++v) {
                // one lane per key: the query is wave-uniform and read through the scalar cache
                // into SGPRs; with four lanes per key each lane reads its segment from LDS
                const uint4 qv = (QL == 1) ? *reinterpret_cast<const uint4 *>(q_rows[v] + cb * 8)
                                           : *reinterpret_cast<const uint4 *>(qb + v * RS + cb * 8);
                float x = sc[v];
                x = dot2_bf16(qv.x, kv.x, x);
                x = dot2_bf16(qv.y, kv.y, x);
                x = dot2_bf16(qv.z, kv.z, x);
                x = dot2_bf16(qv.w, kv.w, x);
                sc[v] = x;
            }
        }
        if (QL > 1) {
#pragma unroll
            for (int v = 0; v < NQ; ++v) {
                sc[v] = sc[v] + __shfl_xor(sc[v], 16);
                sc[v] = sc[v] + __shfl_xor(sc[v], 32);
            }
        }

        // ---- online softmax (log2 domain)
        const int j = b + kk;
        float pv[NQ], alpha[NQ];
        bool rescale = false;
#pragma unroll
        for (int v = 0; v < NQ; ++v) {
            const int pr = L - R + v / G;                 // position of this vector's row
            const int lor = W > 0 ? pr - W + 1 : 0;
            const bool vis = j >= kbeg && j < kend && j <= pr && j >= lor;
            const float x = vis ? sc[v] * scale_log2 : -INFINITY;
            const float bm = wave_max(x);
            const float mn = fmaxf(m_run[v], bm);
            const float al = (mn == -INFINITY) ? 1.f : fast_exp2(m_run[v] - mn);
            pv[v] = vis ? fast_exp2(x - mn) : 0.f;
            m_run[v] = mn;
            alpha[v] = al;
            rescale |= (al != 1.f);
            l_run[v] = l_run[v] * al + (seg == 0 ? pv[v] : 0.f);
        }
        // pack (p[key], p[key + RPI]) as bf16 pairs for the PV dot2
        const bool writer = seg == 0 && ((kk / RPI) & 1) == 0;
        const int pid = (kk / (2 * RPI)) * RPI + (kk % RPI);
#pragma unroll
        for (int v4 = 0; v4 < NQ / 4; ++v4) {
            uint32_t w[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float partner = __shfl_down(pv[v4 * 4 + i], RPI);
                w[i] = pack_bf16x2(pv[v4 * 4 + i], partner);
            }
            if (writer)
                *reinterpret_cast<uint4 *>(p_lds + pid * NQ + v4 * 4) = make_uint4(w[0], w[1], w[2], w[3]);
        }
        if (rescale) {
#pragma unroll
            for (int v = 0; v < NQ; ++v)
#pragma unroll
                for (int c = 0; c < 8; ++c) acc[v][c] *= alpha[v];
        }
        lds_fence();

        // ---- PV: lane owns channels lch*8..+8 of keys t*RPI + lrow
#pragma unroll
        for (int tp = 0; tp < 8; ++tp) {
            const uint4 va = *reinterpret_cast<const uint4 *>(v_lds + ((2 * tp) * RPI + lrow) * RS + lch * 8);
            const uint4 vb = *reinterpret_cast<const uint4 *>(v_lds + ((2 * tp + 1) * RPI + lrow) * RS + lch * 8);
            uint32_t vp[8];
            vp[0] = (va.x & 0xFFFFu) | (vb.x << 16);
            vp[1] = (va.x >> 16) | (vb.x & 0xFFFF0000u);
            vp[2] = (va.y & 0xFFFFu) | (vb.y << 16);
            vp[3] = (va.y >> 16) | (vb.y & 0xFFFF0000u);
            vp[4] = (va.z & 0xFFFFu) | (vb.z << 16);
            vp[5] = (va.z >> 16) | (vb.z & 0xFFFF0000u);
            vp[6] = (va.w & 0xFFFFu) | (vb.w << 16);
            vp[7] = (va.w >> 16) | (vb.w & 0xFFFF0000u);
            const int prd = tp * RPI + lrow;
#pragma unroll
            for (int v4 = 0; v4 < NQ / 4; ++v4) {
                const uint4 pp = *reinterpret_cast<const uint4 *>(p_lds + prd * NQ + v4 * 4);
                const uint32_t pw[4] = {pp.x, pp.y, pp.z, pp.w};
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int c = 0; c < 8; ++c) acc[v4 * 4 + i][c] = dot2_bf16(pw[i], vp[c], acc[v4 * 4 + i][c]);
            }
        }
    }

    // ---- epilogue: combine lanes, write the partial of this chunk
    float l_tot[NQ];
#pragma unroll
    for (int v = 0; v < NQ; ++v) l_tot[v] = wave_sum(l_run[v]);
    if (RPI > 1) {
#pragma unroll
        for (int v = 0; v < NQ; ++v)
#pragma unroll
            for (int c = 0; c < 8; ++c) {
                acc[v][c] = acc[v][c] + __shfl_xor(acc[v][c], 16);
                if (RPI > 2) acc[v][c] = acc[v][c] + __shfl_xor(acc[v][c], 32);
            }
    }
#pragma unroll
    for (int v = 0; v < NQ; ++v) {
        if ((v % RPI) != lrow) continue;
        const int r = v / G, h = kvh * G + (v % G);
        const size_t slot = (((size_t)(s * R + r) * a.Hq + h) * a.n_splits + split);
        float4 *dst = reinterpret_cast<float4 *>(a.ws_acc + slot * D + lch * 8);
        dst[0] = make_float4(acc[v][0], acc[v][1], acc[v][2], acc[v][3]);
        dst[1] = make_float4(acc[v][4], acc[v][5], acc[v][6], acc[v][7]);
        if (lch == 0) *reinterpret_cast<float2 *>(a.ws_ml + slot * 2) = make_float2(m_run[v], l_tot[v]);
    }
}

bool valu_supported(int D, int G, int NQ) {
    if (D != 128 && D != 512) return false;
    if (G == 4) return NQ == 4 || NQ == 8 || NQ == 12;
    if (G == 8) return NQ == 8;
    return false;
}

template <int D, int G, int NQ>
static hipError_t launch_one(const PartArgs &a, int S, hipStream_t st) {
    const dim3 grid(a.n_splits, a.Hkv, S);
    switch (valu_mode<D>(a.P)) {
        case 0: hipLaunchKernelGGL((part_valu_kernel<D, G, NQ, 0>), grid, dim3(64), 0, st, a); break;
        case 1: hipLaunchKernelGGL((part_valu_kernel<D, G, NQ, 1>), grid, dim3(64), 0, st, a); break;
        default: hipLaunchKernelGGL((part_valu_kernel<D, G, NQ, 2>), grid, dim3(64), 0, st, a); break;
    }
    return hipGetLastError();
}

hipError_t launch_part_valu(int D, int G, int NQ, const PartArgs &a, int S, hipStream_t st) {
#define KVP_VALU_CASE(d, g, nq) \
    if (D == d && G == g && NQ == nq) return launch_one<d, g, nq>(a, S, st);
    KVP_VALU_CASE(128, 4, 4) KVP_VALU_CASE(128, 4, 8) KVP_VALU_CASE(128, 4, 12) KVP_VALU_CASE(128, 8, 8)
    KVP_VALU_CASE(512, 4, 4) KVP_VALU_CASE(512, 4, 8) KVP_VALU_CASE(512, 4, 12) KVP_VALU_CASE(512, 8, 8)
#undef KVP_VALU_CASE
    return hipErrorInvalidValue;
}

}  // namespace kvp
