// Uncompressed decode attention over bf16 K/V: the baseline the compressed path is compared with.
//
// MosaicKV (§1, Observation & Approach 2) measures its compressed attention against uncompressed decode
// attention, which it profiles as memory-bound.  This kernel is that baseline on gfx950: every token of every
// KV head is read once, K then V, 16 bytes per lane; a workgroup covers one to eight chunks of 512 tokens of
// one (request, KV head) for its whole query group, merging them with a running maximum, and leaves a
// log-sum-exp partial that the combine kernel merges (more chunks per workgroup on long contexts keep the
// number of partials, and so the combine, small).
#include "common.cuh"
#include "kernels.h"

namespace mkv {

constexpr int kDenseRing = 8;   // loads in flight per lane

__device__ __forceinline__ void unpack8(const u32x4& w, float* x) {
    const uint32_t v[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        x[2 * i] = __uint_as_float(v[i] << 16);
        x[2 * i + 1] = __uint_as_float(v[i] & 0xFFFF0000u);
    }
}

// Lane layout: a wave reads 4 tokens per load (lane group grp = lane / 16 takes one token), each lane 8 channels
// (cs = lane % 16 owns channels 8cs .. 8cs+7).  Wave w covers tokens [128 w, 128 w + 128) of the chunk; a
// group's tokens are grp, grp + 4, ...  Loads past the chunk's last token re-read that token (branch-free, so the
// ring stays in flight) and are masked out of the softmax.
// MULTI: the workgroup covers a.cpw chunks (else one, with the loop and its running maximum folded away).
template <int G, bool MULTI>
__global__ __launch_bounds__(256) void k_dense_attend(DenseArgs a) {
    const int cpw = MULTI ? a.cpw : 1;
    constexpr int TPW = kDenseChunk / 4;   // tokens per wave
    constexpr int NIT = TPW / 4;           // loads per lane per tensor
    __shared__ float sl[kDenseChunk][G];   // logits (log2 units), then softmax numerators
    __shared__ float red[2][4][G];
    __shared__ float wacc[4][G][MKV_D];
    const int b = blockIdx.x;
    const int r = find_slot(a.t_dblk, a.B, b);
    const int n = a.t_n[r], span = kDenseChunk * cpw, nch = (n + span - 1) / span;
    const int local = b - a.t_dblk[r];
    const int g = local / nch, wchunk = local - g * nch;
    const int tid = threadIdx.x, lane = tid & 63, wid = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int grp = lane >> 4, cs = lane & 15;
    const int Hq = a.G * a.Hkv;
    const float scale = 1.4426950408889634f * 0.08838834764831845f;   // log2(e) / sqrt(128)

    float qv[G][8];
#pragma unroll
    for (int h = 0; h < G; ++h) {
        const u32x4 w = *reinterpret_cast<const u32x4*>(a.q + ((size_t)r * Hq + g * G + h) * MKV_D + 8 * cs);
        unpack8(w, qv[h]);
#pragma unroll
        for (int i = 0; i < 8; ++i) qv[h][i] *= scale;
    }
    const size_t rs = (size_t)a.Hkv * MKV_D;   // elements between consecutive tokens of one KV head
    const int tw0 = wid * TPW + grp;
    // running maximum, sum of exponentials and weighted value sums over this workgroup's chunks
    float M[G], L[G], o[G][8];
#pragma unroll
    for (int h = 0; h < G; ++h) {
        M[h] = -INFINITY;
        L[h] = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) o[h][i] = 0.f;
    }
    for (int sc = 0; sc < cpw; ++sc) {
        const int t0 = (wchunk * cpw + sc) * kDenseChunk;
        if (t0 >= n) break;   // the same in every thread
        const int cnt = min(kDenseChunk, n - t0);
        const size_t first = ((size_t)(a.t_tok0[r] + t0) * a.Hkv + g) * MKV_D + 8 * cs;
        const uint16_t* Kp = a.K + first;
        const uint16_t* Vp = a.V + first;
        auto ld = [&](const uint16_t* P, int it) -> u32x4 {
            const int t = min(tw0 + 4 * it, cnt - 1);
            // read once: non-temporal, so that the stream does not displace the step's small tables from the
            // caches
            return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(P + (size_t)t * rs));
        };

        // ---- logits ----
        u32x4 ring[kDenseRing];
#pragma unroll
        for (int j = 0; j < kDenseRing; ++j) ring[j] = ld(Kp, j);
        for (int it0 = 0; it0 < NIT; it0 += kDenseRing) {
#pragma unroll
            for (int j = 0; j < kDenseRing; ++j) {
                const int it = it0 + j;
                float x[8];
                unpack8(ring[j], x);
                if (it + kDenseRing < NIT) ring[j] = ld(Kp, it + kDenseRing);
                float d[G];
#pragma unroll
                for (int h = 0; h < G; ++h) {
                    float s = 0.f;
#pragma unroll
                    for (int i = 0; i < 8; ++i) s = fmaf(qv[h][i], x[i], s);
                    s += dpp_f<0xB1>(s);
                    s += dpp_f<0x4E>(s);
                    s += dpp_f<0x141>(s);
                    s += dpp_f<0x140>(s);
                    d[h] = s;
                }
                const int t = tw0 + 4 * it;
                if (cs == 0) {
#pragma unroll
                    for (int h = 0; h < G; ++h) sl[t][h] = t < cnt ? d[h] : -INFINITY;
                }
            }
        }
        __syncthreads();

        // ---- softmax over the chunk against the running maximum (thread tid holds tokens tid, tid + 256) ----
#pragma unroll
        for (int h = 0; h < G; ++h) {
            const float m = wave_max(fmaxf(sl[tid][h], sl[tid + 256][h]));
            if (lane == 0) red[0][wid][h] = m;
        }
        __syncthreads();
        float alpha[G];
#pragma unroll
        for (int h = 0; h < G; ++h) {
            const float mc = fmaxf(fmaxf(red[0][0][h], red[0][1][h]), fmaxf(red[0][2][h], red[0][3][h]));
            const float mn = fmaxf(M[h], mc);   // finite: the chunk holds at least one token
            alpha[h] = exp2f(M[h] - mn);        // 0 for the first chunk
            M[h] = mn;
            const float e0 = exp2f(sl[tid][h] - mn), e1 = exp2f(sl[tid + 256][h] - mn);
            sl[tid][h] = e0;
            sl[tid + 256][h] = e1;
            const float s = wave_sum(e0 + e1);
            if (lane == 0) red[1][wid][h] = s;
        }
        __syncthreads();
#pragma unroll
        for (int h = 0; h < G; ++h) {
            L[h] = L[h] * alpha[h] + ((red[1][0][h] + red[1][1][h]) + (red[1][2][h] + red[1][3][h]));
#pragma unroll
            for (int i = 0; i < 8; ++i) o[h][i] *= alpha[h];
        }

        // ---- weighted sum of the value rows ----
#pragma unroll
        for (int j = 0; j < kDenseRing; ++j) ring[j] = ld(Vp, j);
        for (int it0 = 0; it0 < NIT; it0 += kDenseRing) {
#pragma unroll
            for (int j = 0; j < kDenseRing; ++j) {
                const int it = it0 + j;
                float x[8];
                unpack8(ring[j], x);
                if (it + kDenseRing < NIT) ring[j] = ld(Vp, it + kDenseRing);
                const int t = tw0 + 4 * it;
#pragma unroll
                for (int h = 0; h < G; ++h) {
                    const float p = sl[t][h];
#pragma unroll
                    for (int i = 0; i < 8; ++i) o[h][i] = fmaf(p, x[i], o[h][i]);
                }
            }
        }
        if (MULTI) __syncthreads();   // the next chunk's logits overwrite sl and red
    }
    // the four lane groups hold disjoint tokens of the same channels
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            float v = o[h][i];
            v += __shfl_xor(v, 16, MKV_WAVE);
            v += __shfl_xor(v, 32, MKV_WAVE);
            o[h][i] = v;
        }
    if (grp == 0) {
#pragma unroll
        for (int h = 0; h < G; ++h)
#pragma unroll
            for (int i = 0; i < 8; ++i) wacc[wid][h][8 * cs + i] = o[h][i];
    }
    __syncthreads();
    for (int i = tid; i < G * MKV_D; i += 256) {
        const int h = i >> 7, ch = i & 127;
        float* dst = a.part + ((size_t)b * G + h) * (MKV_D + 2);
        if (ch == 0) { dst[0] = M[h]; dst[1] = L[h]; }
        dst[2 + ch] = (wacc[0][h][ch] + wacc[1][h][ch]) + (wacc[2][h][ch] + wacc[3][h][ch]);
    }
}

hipError_t launch_dense_attend(const DenseArgs& a, int n_blocks, hipStream_t s) {
    if (n_blocks == 0) return hipSuccess;
    const dim3 grid(n_blocks), block(256);
    if (a.cpw > 1) {
        switch (a.G) {
            case 1: launch_kernel(k_dense_attend<1, true>, grid, block, 0, s, a); break;
            case 2: launch_kernel(k_dense_attend<2, true>, grid, block, 0, s, a); break;
            case 4: launch_kernel(k_dense_attend<4, true>, grid, block, 0, s, a); break;
            default: launch_kernel(k_dense_attend<8, true>, grid, block, 0, s, a); break;
        }
    } else {
        switch (a.G) {
            case 1: launch_kernel(k_dense_attend<1, false>, grid, block, 0, s, a); break;
            case 2: launch_kernel(k_dense_attend<2, false>, grid, block, 0, s, a); break;
            case 4: launch_kernel(k_dense_attend<4, false>, grid, block, 0, s, a); break;
            default: launch_kernel(k_dense_attend<8, false>, grid, block, 0, s, a); break;
        }
    }
    return hipGetLastError();
}

}  // namespace mkv
