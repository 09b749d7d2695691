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

// ---- wave-level reductions (DPP within rows of 16 lanes, permute beyond) -------------------------------
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
__device__ __forceinline__ float wave_max(float v) {
    for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m, MKV_WAVE));
    return v;
}
__device__ __forceinline__ float wave_sum(float v) {
    for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, MKV_WAVE);
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
    uint32_t x = v;
    for (int d = 1; d < 64; d <<= 1) {
        uint32_t y = __shfl_up(x, d, MKV_WAVE);
        if (lane >= d) x += y;
    }
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
