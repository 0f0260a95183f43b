// Device helpers shared by the gfx950 kernels: bf16 packing, the bf16 dot2 instruction and
// wave64 reductions built on DPP row operations plus lane reads.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvp {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// c + a.lo * b.lo + a.hi * b.hi, bf16 inputs, fp32 accumulate (v_dot2c_f32_bf16).
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                           __builtin_bit_cast(bf16x2_t, b), c, false);
}

// Two fp32 values rounded to bf16 (nearest even) and packed lo | hi << 16.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    bf16x2_t v;
    v[0] = (__bf16)lo;
    v[1] = (__bf16)hi;
    return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ uint16_t to_bf16_bits(float x) {
    __bf16 b = (__bf16)x;
    return __builtin_bit_cast(uint16_t, b);
}

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x),
                                                                 CTRL, 0xF, 0xF, false));
}

// DPP controls (GFX9 encoding).
constexpr int DPP_QUAD_XOR1 = 0xB1;   // quad_perm [1,0,3,2]
constexpr int DPP_QUAD_XOR2 = 0x4E;   // quad_perm [2,3,0,1]
constexpr int DPP_ROW_MIRROR = 0x140;
constexpr int DPP_ROW_HALF_MIRROR = 0x141;

// Reduce within each row of 16 lanes; every lane of the row ends with the same value
// (max and + are commutative, so both partners of each step compute identical bits).
__device__ __forceinline__ float row_max16(float x) {
    x = fmaxf(x, dpp<DPP_QUAD_XOR1>(x));
    x = fmaxf(x, dpp<DPP_QUAD_XOR2>(x));
    x = fmaxf(x, dpp<DPP_ROW_HALF_MIRROR>(x));
    x = fmaxf(x, dpp<DPP_ROW_MIRROR>(x));
    return x;
}

__device__ __forceinline__ float row_sum16(float x) {
    x = x + dpp<DPP_QUAD_XOR1>(x);
    x = x + dpp<DPP_QUAD_XOR2>(x);
    x = x + dpp<DPP_ROW_HALF_MIRROR>(x);
    x = x + dpp<DPP_ROW_MIRROR>(x);
    return x;
}

__device__ __forceinline__ float lane_read(float x, int lane) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), lane));
}

// Wave-uniform max / sum over all 64 lanes (fixed order, so bit-reproducible).
__device__ __forceinline__ float wave_max(float x) {
    x = row_max16(x);
    return fmaxf(fmaxf(lane_read(x, 0), lane_read(x, 16)), fmaxf(lane_read(x, 32), lane_read(x, 48)));
}

__device__ __forceinline__ float wave_sum(float x) {
    x = row_sum16(x);
    return (lane_read(x, 0) + lane_read(x, 16)) + (lane_read(x, 32) + lane_read(x, 48));
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// A wave-uniform int32 read from global memory with a vector load, so that it is issued
// together with the other loads at the start of a kernel and one wait covers them all (a
// scalar load is scheduled on its own, after the vector loads have been waited for).  The
// lane-dependent zero from mbcnt makes the address look per-lane to the compiler.
__device__ __forceinline__ int load_uniform_i32(const int32_t *p) {
    const int z = __builtin_amdgcn_mbcnt_lo(0u, 0u);
    return *(p + z);
}

// Page id of entry i of a workgroup's cached page-table entries (TC of them, -1 for an absent
// page).  An index outside the cache counts as absent: only rows past the keys a workgroup
// uses produce one (the tail of its last load step), and those rows are masked out.  Absent
// pages read page 0, which is always inside the pool.
template <int TC>
__device__ __forceinline__ int cached_page(const int32_t *t, int i) {
    return (unsigned)i < (unsigned)TC ? max(t[i], 0) : 0;
}

// A 16-byte load of K/V page data with the nontemporal hint, for the decode kernel, which reads
// every K/V byte of a call once: streaming it through the caches rather than keeping it there
// raises the achieved HBM rate of the 12-stream decode from about 5.6 to 5.9-6.3 TB/s.  (The
// MFMA kernel uses it at d 128 where a key tile has one reader; where several query tiles
// reread a tile from L2, and at d 512, its loads stay plain.)
__device__ __forceinline__ u32x4 stream_load(const uint16_t *p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
}

// Orders this wave's LDS accesses for the compiler without emitting any wait: within one wave
// the LDS unit executes DS instructions in issue order, so data exchanged between the lanes of
// one wave through LDS needs no barrier, only that the compiler keep the order.
__device__ __forceinline__ void wave_lds_fence() {
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront", "local");
}

// Workgroup barrier whose fences cover LDS only: it waits for this wave's LDS operations
// (lgkmcnt) but leaves global loads in flight, so prefetches survive it.
__device__ __forceinline__ void lds_fence() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

}  // namespace kvp
