// Row write into page slots, and the fixed-order merge of split-context partials.
//
// Row write: TensorFold PR #1620, opening description, "Writes" bullet (the rows kernel's new
// K/V rows are copied into the pages).  Merge: the same PR's follow-up discussion, where the
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
    const int pos = a.seq_len[s] - a.R + r;
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

hipError_t launch_rows_put(const RowsArgs &a, hipStream_t st) {
    const int blocks = a.S * a.R;
    if (blocks == 0) return hipSuccess;
    hipLaunchKernelGGL(rows_put_kernel, dim3(blocks), dim3(256), 0, st, a);
    return hipGetLastError();
}

// One wave per (stream, row, query head).  Lane c owns channels [c*CPL, (c+1)*CPL).
template <int CPL>
__global__ __launch_bounds__(64) void merge_kernel(const MergeArgs a) {
    const int vec = blockIdx.x;            // (s * R + r) * Hq + h
    const int s = vec / (a.R * a.Hq);
    const int r = (vec / a.Hq) % a.R;
    const int L = a.seq_len[s];
    const int lane = threadIdx.x;
    uint16_t *o = a.out + (size_t)vec * a.D + lane * CPL;
    const int pos = L - a.R + r;
    float res[CPL];
    for (int c = 0; c < CPL; ++c) res[c] = 0.f;
    if (pos >= 0) {
        const int lo = a.window > 0 ? max(0, L - a.R - a.window + 1) : 0;
        const int first = lo / a.chunk;
        int n = (L + a.chunk - 1) / a.chunk - first;
        if (n > a.n_splits) n = a.n_splits;
        const float *ml = a.ws_ml + (size_t)vec * a.n_splits * 2;
        const float *acc = a.ws_acc + (size_t)vec * a.n_splits * a.D + lane * CPL;
        float M = -INFINITY;
        for (int i = 0; i < n; ++i) M = fmaxf(M, ml[2 * i]);
        float den = 0.f;
        float num[CPL];
        for (int c = 0; c < CPL; ++c) num[c] = 0.f;
        if (M != -INFINITY) {
            for (int i = 0; i < n; ++i) {
                const float mi = ml[2 * i];
                const float w = (mi == -INFINITY) ? 0.f : fast_exp2(mi - M);
                den += w * ml[2 * i + 1];
                const float *ai = acc + (size_t)i * a.D;
#pragma unroll
                for (int c = 0; c < CPL; ++c) num[c] += w * ai[c];
            }
        }
        if (den > 0.f) {
            const float inv = 1.0f / den;
#pragma unroll
            for (int c = 0; c < CPL; ++c) res[c] = num[c] * inv;
        }
    }
#pragma unroll
    for (int c = 0; c < CPL; c += 2) {
        *reinterpret_cast<uint32_t *>(o + c) = pack_bf16x2(res[c], res[c + 1]);
    }
}

hipError_t launch_merge(const MergeArgs &a, hipStream_t st) {
    const int blocks = a.S * a.R * a.Hq;
    if (blocks == 0) return hipSuccess;
    switch (a.D) {
        case 128: hipLaunchKernelGGL(merge_kernel<2>, dim3(blocks), dim3(64), 0, st, a); break;
        case 512: hipLaunchKernelGGL(merge_kernel<8>, dim3(blocks), dim3(64), 0, st, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace kvp
