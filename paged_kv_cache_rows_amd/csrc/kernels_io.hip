// Row write into page slots, and the fixed-order merge of split-context partials.
//
// Row write: TensorFold PR #1620, opening description, Writes bullet (the K/V rows a layer
// produces are copied into their page slots).  Merge: the same PR's follow-up discussion, where the
// tree-attention parts are combined by a merge kernel that reads no pages; here the partials
// are combined in increasing chunk order, so the result depends only on logical positions.
#include "internal.h"
#include "device_common.h"

namespace kvp {

// One workgroup per (stream, row); each thread moves 16-byte pieces of the row's Hkv*D values.
// The page lookup happens once per row, not per value.
__global__ __launch_bounds__(256) void rows_put_kernel(const RowsArgs a) {
    const int row = blockIdx.x;            // s * R + r
    const int s = row / a.R;
    const int r = row - s * a.R;
    const int pos = kernel_len(a.seq_len[s], a.max_len) - a.R + r;
    if (pos < 0) return;
    int idx = pos / a.P;
    const int off = pos - idx * a.P;
    if (a.ring_pages) idx %= a.ring_pages;
    if (idx >= a.stride) return;
    const int pg = a.table[(size_t)s * a.stride + idx];
    if ((unsigned)pg >= (unsigned)a.num_pages) return;
    const int per_head = a.D / 8;
    const int n = a.Hkv * per_head;
    const uint4 *ks = reinterpret_cast<const uint4 *>(a.k_new + (size_t)row * a.Hkv * a.D);
    const uint4 *vs = reinterpret_cast<const uint4 *>(a.v_new + (size_t)row * a.Hkv * a.D);
    for (int c = threadIdx.x; c < n; c += blockDim.x) {
        const int kvh = c / per_head;
        const int w = c - kvh * per_head;
        const size_t dst = (((size_t)pg * a.Hkv + kvh) * a.P + off) * a.D + (size_t)w * 8;
        *reinterpret_cast<uint4 *>(a.k_pages + dst) = ks[c];
        *reinterpret_cast<uint4 *>(a.v_pages + dst) = vs[c];
    }
}

// Page copy (TensorFold PR #1620, opening description, Kept states bullet: a stream's state is
// kept by copying the pages its table walks).  Block (x, y) copies the x-th run of
// 256 * PPT 16-byte pieces of pair y, K and V, with streaming loads and stores: the bytes are
// touched once.
constexpr int COPY_PPT = 8;

__global__ __launch_bounds__(256) void pages_copy_kernel(const CopyArgs a) {
    const int i = blockIdx.y;
    const int sp = a.src[i], dp = a.dst[i];
    if ((unsigned)sp >= (unsigned)a.num_pages || (unsigned)dp >= (unsigned)a.num_pages || sp == dp) return;
    const size_t pieces = a.page_elems / 8;
    const u32x4 *ks = reinterpret_cast<const u32x4 *>(a.k_pages + (size_t)sp * a.page_elems);
    const u32x4 *vs = reinterpret_cast<const u32x4 *>(a.v_pages + (size_t)sp * a.page_elems);
    u32x4 *kd = reinterpret_cast<u32x4 *>(a.k_pages + (size_t)dp * a.page_elems);
    u32x4 *vd = reinterpret_cast<u32x4 *>(a.v_pages + (size_t)dp * a.page_elems);
    const size_t p0 = (size_t)blockIdx.x * (256 * COPY_PPT) + threadIdx.x;
    u32x4 kx[COPY_PPT], vx[COPY_PPT];
#pragma unroll
    for (int u = 0; u < COPY_PPT; ++u) {
        const size_t pc = min(p0 + (size_t)u * 256, pieces - 1);
        kx[u] = __builtin_nontemporal_load(ks + pc);
        vx[u] = __builtin_nontemporal_load(vs + pc);
    }
#pragma unroll
    for (int u = 0; u < COPY_PPT; ++u) {
        const size_t pc = p0 + (size_t)u * 256;
        if (pc < pieces) {
            __builtin_nontemporal_store(kx[u], kd + pc);
            __builtin_nontemporal_store(vx[u], vd + pc);
        }
    }
}

hipError_t launch_pages_copy(const CopyArgs &args, hipStream_t st) {
    if (args.n <= 0) return hipSuccess;
    const size_t pieces = args.page_elems / 8;
    const unsigned bx = (unsigned)((pieces + 256 * COPY_PPT - 1) / (256 * COPY_PPT));
    // gridDim.y is limited to 65535: launch the pairs in slices
    for (int i0 = 0; i0 < args.n; i0 += 65535) {
        CopyArgs a = args;
        a.src = args.src + i0;
        a.dst = args.dst + i0;
        a.n = min(args.n - i0, 65535);
        hipLaunchKernelGGL(pages_copy_kernel, dim3(bx, a.n), dim3(256), 0, st, a);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

hipError_t launch_rows_put(const RowsArgs &a, hipStream_t st) {
    const int blocks = a.S * a.R;
    if (blocks == 0) return hipSuccess;
    hipLaunchKernelGGL(rows_put_kernel, dim3(blocks), dim3(256), 0, st, a);
    return hipGetLastError();
}

// One wave per (stream, row, query head) and slice of CW channels, CW chosen per call so that a
// wave holds all of a row's splits in one pass where it can (launch_merge).  Lane = (split group sg, channel block cb):
// it owns channels [8 cb, 8 cb + 8) of its slice for the splits i = sg, sg + SG, ...; the split
// groups are summed at the end in a fixed order, so the result depends only on the partials,
// not on timing.
template <int D, int CW>
__global__ __launch_bounds__(64) void merge_kernel(const MergeArgs a) {
    constexpr int NCW = D / CW;             // waves per (stream, row, query head)
    constexpr int CB = CW / 8;              // channel blocks of 8
    constexpr int SG = 64 / CB;             // split groups
    const int vec = blockIdx.x / NCW;       // (s * R + r) * Hq + h
    const int cw = blockIdx.x % NCW;        // channel slice
    const int s = vec / (a.R * a.Hq);
    const int r = (vec / a.Hq) % a.R;
    const int lane = threadIdx.x;
    const int cb = lane % CB, sg = lane / CB;
    const float2 *ml = reinterpret_cast<const float2 *>(a.ws_ml) + (size_t)vec * a.n_splits;
    const float *acc = a.ws_acc + (size_t)vec * a.n_splits * D + cw * CW + cb * 8;
    // Without a window every row's splits start at split 0, so when they fit one pass the
    // partials are loaded before the stream's length is known (slots the row turns out not to
    // read are discarded by select below): the merge then costs one round trip to memory.
    const bool early = a.window <= 0 && a.n_splits <= 4 * SG;
    float4 xe[4][2];
    float2 mle[4];
    if (early) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int i = u * SG + sg;
            const int ic = i < a.n_splits ? i : 0;
            mle[u] = ml[ic];
            const float4 *src = reinterpret_cast<const float4 *>(acc + (size_t)ic * D);
            xe[u][0] = src[0];
            xe[u][1] = src[1];
        }
    }
    const int L = kernel_len(a.seq_len[s], a.max_len);
    const int pos = L - a.R + r;
    float num[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) num[c] = 0.f;
    float den = 0.f, M = -INFINITY;
    if (pos >= 0) {
        // this row reads only the splits holding its own keys [lo_r, pos]: the even pieces of
        // the stream, or the chunks counted from the first chunk any row of the stream sees
        const SplitSpan sp = row_splits(L, a.R, a.window, pos, a.n_splits, a.chunk, a.even != 0, a.align);
        const int i_begin = sp.first, n = sp.end;
        if (n - i_begin <= 4 * SG) {
            // one pass (every decode and verify plan here): the partials and their (m, l) are
            // loaded together, before the max is known
            float4 x[4][2];
            float2 m_l[4];
            if (early) {
                // i_begin is 0 here; a slot past the row's splits may never have been written
                // (possibly NaN): it becomes an empty split, so that a zero weight never meets it
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const bool in = u * SG + sg < n;
                    m_l[u] = in ? mle[u] : make_float2(-INFINITY, 0.f);
                    const float4 z = make_float4(0.f, 0.f, 0.f, 0.f);
                    x[u][0] = in ? xe[u][0] : z;
                    x[u][1] = in ? xe[u][1] : z;
                }
            } else {
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const int i = i_begin + u * SG + sg;
                    // a padded slot rereads the row's first split, which is always written (a
                    // zero weight must never meet an unwritten, possibly NaN, split)
                    const int ic = i < n ? i : i_begin;
                    m_l[u] = ml[ic];
                    const float4 *src = reinterpret_cast<const float4 *>(acc + (size_t)ic * D);
                    x[u][0] = src[0];
                    x[u][1] = src[1];
                }
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) M = fmaxf(M, m_l[u].x);
            M = wave_max(M);
            if (M != -INFINITY) {
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const bool in = i_begin + u * SG + sg < n;
                    const float w = (in && m_l[u].x != -INFINITY) ? fast_exp2(m_l[u].x - M) : 0.f;
                    if (cb == 0) den += w * m_l[u].y;
                    num[0] += w * x[u][0].x; num[1] += w * x[u][0].y;
                    num[2] += w * x[u][0].z; num[3] += w * x[u][0].w;
                    num[4] += w * x[u][1].x; num[5] += w * x[u][1].y;
                    num[6] += w * x[u][1].z; num[7] += w * x[u][1].w;
                }
            }
        } else {
            for (int i = i_begin + lane; i < n; i += 64) M = fmaxf(M, ml[i].x);
            M = wave_max(M);
            if (M != -INFINITY) {
                for (int i0 = i_begin; i0 < n; i0 += 4 * SG) {
                    float4 x[4][2];
                    float w[4];
    #pragma unroll
                    for (int u = 0; u < 4; ++u) {
                        const int i = i0 + u * SG + sg;
                        const bool in = i < n;
                        // a padded slot rereads the row's first split, which is always written
                        // (a zero weight must never meet an unwritten, possibly NaN, split)
                        const int ic = in ? i : i_begin;
                        const float2 m_l = ml[ic];
                        const float4 *src = reinterpret_cast<const float4 *>(acc + (size_t)ic * D);
                        x[u][0] = src[0];
                        x[u][1] = src[1];
                        w[u] = (in && m_l.x != -INFINITY) ? fast_exp2(m_l.x - M) : 0.f;
                        if (cb == 0) den += w[u] * m_l.y;
                    }
    #pragma unroll
                    for (int u = 0; u < 4; ++u) {
                        num[0] += w[u] * x[u][0].x; num[1] += w[u] * x[u][0].y;
                        num[2] += w[u] * x[u][0].z; num[3] += w[u] * x[u][0].w;
                        num[4] += w[u] * x[u][1].x; num[5] += w[u] * x[u][1].y;
                        num[6] += w[u] * x[u][1].z; num[7] += w[u] * x[u][1].w;
                    }
                }
            }
        }
    }
    // sum the split groups (lanes cb, cb + CB, ...) and the denominators (lanes 0, CB, ...)
#pragma unroll
    for (int d = CB; d < 64; d *= 2)
#pragma unroll
        for (int c = 0; c < 8; ++c) num[c] = num[c] + __shfl_xor(num[c], d);
    den = wave_sum(den);
    if (sg == 0) {
        const float inv = den > 0.f ? 1.0f / den : 0.f;
        uint32_t o[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) o[c] = pack_bf16x2(num[2 * c] * inv, num[2 * c + 1] * inv);
        *reinterpret_cast<uint4 *>(a.out + (size_t)vec * D + cw * CW + cb * 8) = make_uint4(o[0], o[1], o[2], o[3]);
    }
}

hipError_t launch_merge(const MergeArgs &a, hipStream_t st) {
    const int blocks = a.S * a.R * a.Hq;
    if (blocks == 0) return hipSuccess;
    if (a.D != 128 && a.D != 256 && a.D != 512) return hipErrorInvalidValue;
    // The widest channel slice whose wave holds every split of a row in one pass (4 per lane,
    // 64 / (CW / 8) split groups: 2048 / CW splits), down to 32 channels; past 64 splits,
    // 64-channel slices in several passes.  One pass with the loads issued before the
    // stream's length is one round trip to memory: the 2,048-key d 512 decode (64 splits) in
    // 32-channel slices, cold whole call 15.3-15.5 -> 14.5-14.8 us.  16-channel slices (2,048
    // one-wave workgroups for the d 512 verify's 94 splits) measured slower than several
    // passes over 64 channels: 27.8 against 26.0 us.
    int cw = 64;
    for (int c = 128; c >= 32; c /= 2)
        if (c <= a.D && a.n_splits <= 2048 / c) {
            cw = c;
            break;
        }
#define KVP_MERGE(d, c)                                                                                  \
    if (a.D == d && cw == c) {                                                                           \
        hipLaunchKernelGGL((merge_kernel<d, c>), dim3(blocks * (d / c)), dim3(64), 0, st, a);            \
        return hipGetLastError();                                                                        \
    }
    KVP_MERGE(128, 128) KVP_MERGE(128, 64) KVP_MERGE(128, 32)
    KVP_MERGE(256, 128) KVP_MERGE(256, 64) KVP_MERGE(256, 32)
    KVP_MERGE(512, 128) KVP_MERGE(512, 64) KVP_MERGE(512, 32)
#undef KVP_MERGE
    return hipErrorInvalidValue;
}

}  // namespace kvp
