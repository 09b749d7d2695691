// Shared device helpers for the gfx950 kernels of the compressed KV cache.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#define MKV_D 128
#define MKV_SEG 64
#define MKV_WAVE 64
#define MKV_MAX_GROUP_DEV 8

namespace mkv {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;

// ---- scalar conversions -------------------------------------------------------------------------------
__device__ __forceinline__ float bf16_to_f32(uint32_t b16) { return __uint_as_float(b16 << 16); }

// float32 -> bf16 bit pattern, round to nearest, ties to even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// Order-preserving key of a float32 score: larger float -> larger key; -0 is folded onto +0 so that the
// two zeros tie like they do numerically.
__device__ __forceinline__ uint32_t score_key(float s) {
    uint32_t u = __float_as_uint(s);
    if (u == 0x80000000u) u = 0u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// ---- wave-level reductions (DPP within rows of 16 lanes, scalar reads or row broadcasts beyond) ---------
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
// Sum over each group of 8 consecutive lanes; every lane of the group gets the total.
__device__ __forceinline__ float sum8(float v) {
    v += dpp_f<0xB1>(v);    // quad_perm [1,0,3,2]
    v += dpp_f<0x4E>(v);    // quad_perm [2,3,0,1]
    v += dpp_f<0x141>(v);   // row_half_mirror: lane i <-> 7-i inside each group of 8
    return v;
}
__device__ __forceinline__ float shfl_xor_f(float v, int m) {
    return __shfl_xor(v, m, MKV_WAVE);
}
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ uint32_t dpp_u(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, ROW_MASK, 0xF, false);
}
__device__ __forceinline__ float lane_f(float v, int lane) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), lane));
}
// Whole-wave max and sum: DPP inside each row of 16 lanes (every lane of a row ends with the row's result), then
// the four rows' results read into scalar registers and combined.  Every lane returns the same value.
__device__ __forceinline__ float wave_max(float v) {
    v = fmaxf(v, dpp_f<0xB1>(v));
    v = fmaxf(v, dpp_f<0x4E>(v));
    v = fmaxf(v, dpp_f<0x141>(v));
    v = fmaxf(v, dpp_f<0x140>(v));   // row_mirror: lane i <-> 15-i inside each row
    return fmaxf(fmaxf(lane_f(v, 0), lane_f(v, 16)), fmaxf(lane_f(v, 32), lane_f(v, 48)));
}
__device__ __forceinline__ float wave_sum(float v) {
    v += dpp_f<0xB1>(v);
    v += dpp_f<0x4E>(v);
    v += dpp_f<0x141>(v);
    v += dpp_f<0x140>(v);
    return (lane_f(v, 0) + lane_f(v, 16)) + (lane_f(v, 32) + lane_f(v, 48));
}
// Inclusive prefix sum over the 64 lanes of a wave: shifts inside each row of 16, then row 0's total is added to
// row 1 and row 2's to row 3 (row_bcast:15), and rows 0-1's total to rows 2 and 3 (row_bcast:31).
__device__ __forceinline__ uint32_t wave_incl_u32(uint32_t v) {
    const int r = threadIdx.x & 15;
    uint32_t y = dpp_u<0x111>(v);
    if (r >= 1) v += y;
    y = dpp_u<0x112>(v);
    if (r >= 2) v += y;
    y = dpp_u<0x114>(v);
    if (r >= 4) v += y;
    y = dpp_u<0x118>(v);
    if (r >= 8) v += y;
    v += dpp_u<0x142, 0xA>(v);
    v += dpp_u<0x143, 0xC>(v);
    return v;
}

// Orders LDS accesses of one wave (all lanes) without a workgroup barrier.
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// ---- device-scope atomics -----------------------------------------------------------------------------
__device__ __forceinline__ uint32_t atomic_add_dev(uint32_t* p, uint32_t v) {
    return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Index r with base[r] <= b < base[r+1] for a non-decreasing base[0..n] with base[0] == 0 <= b < base[n].
__device__ __forceinline__ int find_slot(const int32_t* base, int n, int b) {
    int lo = 0, hi = n;
    while (hi - lo > 1) {
        int mid = (lo + hi) >> 1;
        if (base[mid] <= b) lo = mid; else hi = mid;
    }
    return lo;
}

// Workgroup-wide exclusive scan of one uint32 per thread (blockDim.x a multiple of 64, <= 1024).
// `tmp` must hold blockDim.x/64 + 1 words of LDS.  Returns the exclusive prefix; *total gets the sum.
__device__ __forceinline__ uint32_t block_exscan(uint32_t v, uint32_t* tmp, uint32_t* total) {
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6, nw = blockDim.x >> 6;
    const uint32_t x = wave_incl_u32(v);
    if (lane == 63) tmp[wid] = x;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t run = 0;
        for (int w = 0; w < nw; ++w) { uint32_t t = tmp[w]; tmp[w] = run; run += t; }
        tmp[nw] = run;
    }
    __syncthreads();
    uint32_t res = tmp[wid] + x - v;
    *total = tmp[nw];
    __syncthreads();
    return res;
}

}  // namespace mkv
