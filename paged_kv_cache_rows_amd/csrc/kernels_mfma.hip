// Paged GQA attention part kernel for many query vectors per KV head (rows * group >= 16):
// speculative verify windows and prompt chunks, on MFMA.
//
// TensorFold PR #1620, opening description (Reads bullet: prompts and drafted verify read keys
// through the page table) and TensorFold PR #2730 (verify windows of up to eight rows).
//
// Design for gfx950.  A workgroup of 4 waves takes a tile of 64 query vectors of one KV head
// (rows x GQA heads, row-major) and one chunk of keys; each wave owns 16 query vectors.
//  * K and V tiles of KT keys are loaded cooperatively through the page table (entries of the
//    chunk cached in LDS) into LDS; K row-major, V transposed (keys contiguous per channel).
//  * Scores are computed transposed, S^T = K Q^T, with v_mfma_f32_16x16x32_bf16: the wave's
//    queries are the B operand, held in registers for the whole chunk.  In the C layout a lane
//    owns one query column and 4 keys per 16-key block, which is exactly the B-operand layout
//    that O^T = V^T P^T needs, so the softmax weights feed the second MFMA from registers.
//  * Online softmax per query column in the log2 domain; masked keys are selected out and V
//    rows outside the chunk are zeroed, so NaN in unused slots never reaches the sums.
//  * The workgroup writes an unnormalised partial (acc, m, l) per query vector, merged later
//    in fixed chunk order.
#include "internal.h"
#include "device_common.h"

namespace kvp {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

template <int D>
struct MfmaGeom {
    static constexpr int KT = D == 128 ? 64 : 32;       // keys per tile
    static constexpr int CHUNK = D == 128 ? 256 : 128;  // keys per workgroup
    static constexpr int KRS = D + 8;                   // K tile row stride (bf16)
    static constexpr int VRS = KT + 4;                  // V^T row stride (bf16)
    static constexpr int M = 64;                        // query vectors per workgroup
    static constexpr int NT = 256;                      // threads
    static constexpr int LC = KT * D / 8 / NT;          // 16-byte pieces per thread per operand
    static constexpr int TC = 72;                       // cached page-table entries
};

int mfma_chunk(int D) { return D == 512 ? MfmaGeom<512>::CHUNK : MfmaGeom<128>::CHUNK; }

bool mfma_supported(int D, int G, int R) {
    return (D == 128 || D == 512) && (G == 4 || G == 8) && R >= 1 && R * G >= 16;
}

int mfma_query_tiles(int D, int G, int R) {
    (void)D;
    return (R * G + 63) / 64;
}

template <int D>
static bool mfma_cached(int P) {
    using Geo = MfmaGeom<D>;
    return (Geo::CHUNK + Geo::KT) / P + 2 <= Geo::TC;
}

__device__ __forceinline__ f32x4_t mfma16(const bf16x8_t &a, const bf16x8_t &b, const f32x4_t &c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

template <int D, int G, bool CACHED>
__global__ __launch_bounds__(256) void part_mfma_kernel(const PartArgs a) {
    using Geo = MfmaGeom<D>;
    constexpr int KT = Geo::KT, CHUNK = Geo::CHUNK, KRS = Geo::KRS, VRS = Geo::VRS, M = Geo::M;
    constexpr int LC = Geo::LC, TC = Geo::TC;
    constexpr int NB = KT / 16;      // 16-key blocks per tile
    constexpr int NKB = D / 32;      // 32-channel blocks (QK k-steps)
    constexpr int NCB = D / 16;      // 16-channel blocks (PV output blocks)
    constexpr int NPM = KT / 32;     // 32-key PV k-steps

    __shared__ __attribute__((aligned(16))) uint16_t k_lds[KT * KRS];
    __shared__ __attribute__((aligned(16))) uint16_t vt_lds[D * VRS];
    __shared__ int32_t t_lds[TC];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int col = lane & 15, grp = lane >> 4;
    const int split = blockIdx.x, s = blockIdx.z;
    const int kvh = blockIdx.y % a.Hkv, tile = blockIdx.y / a.Hkv;
    const int R = a.R, W = a.window;
    const int L = a.seq_len[s];
    const int NQ = R * G;
    const int v0 = tile * M;
    if (L <= 0 || v0 >= NQ || split >= a.n_splits) return;
    const int r_first = v0 / G;
    const int r_last = (min(NQ, v0 + M) - 1) / G;
    const int p_first = L - R + r_first, p_last = L - R + r_last;
    const int lo_stream = W > 0 ? max(0, L - R - W + 1) : 0;
    const int c0 = (lo_stream / CHUNK + split) * CHUNK;
    const int lo_tile = W > 0 ? max(0, p_first - W + 1) : 0;
    const int kbeg = max(c0, lo_tile);
    const int kend = min(c0 + CHUNK, p_last + 1);
    if (kbeg >= kend) return;        // no row of the tile sees this chunk: nothing to merge

    // this lane's query column
    const int vq = v0 + wave * 16 + col;
    const bool col_ok = vq < NQ;
    const int rq = col_ok ? vq / G : 0;
    const int hq = kvh * G + (col_ok ? vq % G : 0);
    const int p_col = L - R + rq;
    const int lo_col = W > 0 ? p_col - W + 1 : 0;

    // queries as the B operand of S^T = K Q^T: lane holds channels 32 kb + 8 grp .. + 8
    bf16x8_t qf[NKB];
    {
        const uint16_t *qrow = a.q + ((size_t)(s * R + rq) * a.Hq + hq) * D + 8 * grp;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
            u32x4 x = *reinterpret_cast<const u32x4 *>(qrow + 32 * kb);
            if (!col_ok) x = u32x4{0, 0, 0, 0};
            qf[kb] = __builtin_bit_cast(bf16x8_t, x);
        }
    }

    const int P = a.P;
    const int kt_first = (kbeg / KT) * KT;
    const int nt = (kend - kt_first + KT - 1) / KT;
    const int idx0 = kt_first / P;
    const int32_t *trow = a.table + (size_t)s * a.stride;
    if (CACHED) {
        for (int i = tid; i < TC; i += Geo::NT) {
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
    // piece u of this thread: key row kr[u] of the tile, channels 8 * kc[u] .. + 8
    u32x4 kreg[LC], vreg[LC];
    auto load_tile = [&](int tb, u32x4 (&kq)[LC], u32x4 (&vq_)[LC]) {
#pragma unroll
        for (int u = 0; u < LC; ++u) {
            const int c = tid + Geo::NT * u;
            const int kr = c / (D / 8), kc = c % (D / 8);
            const int j = tb + kr;
            int idx = j / P;
            const int off = j - idx * P;
            int pg;
            if (CACHED) {
                pg = t_lds[idx - idx0];
            } else {
                if (a.ring_pages) idx %= a.ring_pages;
                const int tp = trow[min(idx, a.stride - 1)];
                pg = (idx < a.stride && (unsigned)tp < (unsigned)a.num_pages) ? tp : -1;
            }
            const size_t e = (size_t)max(pg, 0) * page_elems + head_off + (size_t)off * D + 8 * kc;
            kq[u] = *reinterpret_cast<const u32x4 *>(a.k_pages + e);
            vq_[u] = *reinterpret_cast<const u32x4 *>(a.v_pages + e);
        }
    };

    f32x4_t o[NCB];
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) o[cb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY, l_run = 0.f;
    const float scale_log2 = a.scale_log2;

    load_tile(kt_first, kreg, vreg);
    for (int it = 0; it < nt; ++it) {
        const int tb = kt_first + it * KT;
        lds_fence();
#pragma unroll
        for (int u = 0; u < LC; ++u) {
            const int c = tid + Geo::NT * u;
            const int kr = c / (D / 8), kc = c % (D / 8);
            const int j = tb + kr;
            *reinterpret_cast<u32x4 *>(k_lds + kr * KRS + 8 * kc) = kreg[u];
            const uint32_t keep = (j >= kbeg && j < kend) ? 0xFFFFFFFFu : 0u;
            const u32x4 x = vreg[u] & keep;
            const uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                vt_lds[(8 * kc + 2 * i) * VRS + kr] = (uint16_t)(w[i] & 0xFFFFu);
                vt_lds[(8 * kc + 2 * i + 1) * VRS + kr] = (uint16_t)(w[i] >> 16);
            }
        }
        if (it + 1 < nt) load_tile(tb + KT, kreg, vreg);
        lds_fence();

        // S^T for this wave's 16 query columns
        f32x4_t sacc[NB];
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            sacc[nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) {
                const bf16x8_t kf = *reinterpret_cast<const bf16x8_t *>(k_lds + (16 * nb + col) * KRS + 32 * kb + 8 * grp);
                sacc[nb] = mfma16(kf, qf[kb], sacc[nb]);
            }
        }
        // mask, tile max, new running max
        float tmax = -INFINITY;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int j = tb + 16 * nb + 4 * grp + r;
                const bool vis = col_ok && j >= kbeg && j < kend && j <= p_col && j >= lo_col;
                const float x = vis ? sacc[nb][r] * scale_log2 : -INFINITY;
                sacc[nb][r] = x;
                tmax = fmaxf(tmax, x);
            }
        tmax = fmaxf(tmax, __shfl_xor(tmax, 16));
        tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
        const float m_new = fmaxf(m_run, tmax);
        const float alpha = (m_new == -INFINITY) ? 1.f : fast_exp2(m_run - m_new);
        m_run = m_new;
        float psum = 0.f;
        bf16x8_t pf[NPM];
#pragma unroll
        for (int pm = 0; pm < NPM; ++pm) {
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float x = sacc[2 * pm + h][r];
                    const float p = (x == -INFINITY) ? 0.f : fast_exp2(x - m_new);
                    psum += p;
                    pf[pm][4 * h + r] = (__bf16)p;
                }
        }
        l_run = l_run * alpha + psum;
        if (alpha != 1.f) {
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb) o[cb] *= alpha;
        }
        // O^T += V^T P^T: A = V^T rows (channels), keys 32 pm + 4 grp + {0..3} and + 16
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) {
#pragma unroll
            for (int pm = 0; pm < NPM; ++pm) {
                const uint16_t *vrow = vt_lds + (16 * cb + col) * VRS + 32 * pm + 4 * grp;
                const uint2 lo = *reinterpret_cast<const uint2 *>(vrow);
                const uint2 hi = *reinterpret_cast<const uint2 *>(vrow + 16);
                const u32x4 vv = u32x4{lo.x, lo.y, hi.x, hi.y};
                o[cb] = mfma16(__builtin_bit_cast(bf16x8_t, vv), pf[pm], o[cb]);
            }
        }
    }

    // combine the four key groups' partial sums of each column, write the partials
    float l_tot = l_run + __shfl_xor(l_run, 16);
    l_tot = l_tot + __shfl_xor(l_tot, 32);
    if (col_ok) {
        const int h = hq;
        const size_t slot = ((size_t)(s * R + rq) * a.Hq + h) * a.n_splits + split;
        float *dst = a.ws_acc + slot * D + 4 * grp;
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb)
            *reinterpret_cast<float4 *>(dst + 16 * cb) = make_float4(o[cb][0], o[cb][1], o[cb][2], o[cb][3]);
        if (grp == 0) *reinterpret_cast<float2 *>(a.ws_ml + slot * 2) = make_float2(m_run, l_tot);
    }
}

template <int D, int G>
static hipError_t launch_d_g(const PartArgs &a, int S, hipStream_t st) {
    const dim3 grid(a.n_splits, a.Hkv * mfma_query_tiles(D, G, a.R), S);
    if (mfma_cached<D>(a.P))
        hipLaunchKernelGGL((part_mfma_kernel<D, G, true>), grid, dim3(256), 0, st, a);
    else
        hipLaunchKernelGGL((part_mfma_kernel<D, G, false>), grid, dim3(256), 0, st, a);
    return hipGetLastError();
}

hipError_t launch_part_mfma(int D, int G, const PartArgs &a, int S, hipStream_t st) {
    if (D == 128 && G == 4) return launch_d_g<128, 4>(a, S, st);
    if (D == 128 && G == 8) return launch_d_g<128, 8>(a, S, st);
    if (D == 512 && G == 4) return launch_d_g<512, 4>(a, S, st);
    if (D == 512 && G == 8) return launch_d_g<512, 8>(a, S, st);
    return hipErrorInvalidValue;
}

}  // namespace kvp
