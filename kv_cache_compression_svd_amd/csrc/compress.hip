// Dynamic two-D compression on gfx950 (arXiv 2607.00760, section 1, Observation & Approach 1: per-vector
// element selection after an SVD rotation, one compression strategy per KV-cache segment; Observation &
// Approach 2: the sparse cache is packed into a dense format in GPU memory).
//
// Two passes over each 64-token segment tile of one (request, KV head, tensor) stream:
//   decide: rotate (MFMA), find per-vector magnitude thresholds of the c largest channels, test the energy
//           rule in float64, pick the segment's kept-channel count, record its payload size;
//   scan:   exclusive scan of the segment sizes -> payload offsets;
//   pack:   rotate again, keep the channels above each vector's threshold (ties: lower channel first), and
//           write the segment as one contiguous block (values, then uint8 channel indices).
// The rotation of bf16 data multiplies the bf16 tile by the fp32 basis split into three bf16 parts
// (hi + mid + lo carries 24 significant bits), accumulating in fp32; fp32 data is rotated in float64 on the
// vector ALUs.
#include "common.cuh"
#include "kernels.h"

namespace mkv {

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

__global__ void k_upload(Upload u) {
    for (int i = threadIdx.x; i < u.n; i += blockDim.x) u.dst[i] = u.w[i];
}

hipError_t launch_upload(const Upload& u, hipStream_t s) {
    hipLaunchKernelGGL(k_upload, dim3(1), dim3(256), 0, s, u);
    return hipGetLastError();
}

struct Tile {
    int X, r, h, s0, s1, n;
    int64_t tok0;   // first token of the request
    int64_t seg0;   // global id of segment 0 of this stream
};

__device__ __forceinline__ Tile cmp_tile(const CmpArgs& a) {
    const int32_t* tokbase = a.tab;
    const int32_t* nn = a.tab + a.B;
    const int32_t* segbase = a.tab + 2 * a.B;
    const int32_t* cblk = a.tab + 3 * a.B;
    Tile t;
    t.X = blockIdx.x / a.nblk;
    const int b = blockIdx.x - t.X * a.nblk;
    t.r = find_slot(cblk, a.B, b);
    t.n = nn[t.r];
    const int Sr = (t.n + MKV_SEG - 1) / MKV_SEG;
    const int nch = (Sr + a.spw - 1) / a.spw;
    const int local = b - cblk[t.r];
    t.h = local / nch;
    const int chunk = local - t.h * nch;
    t.s0 = chunk * a.spw;
    t.s1 = min(Sr, t.s0 + a.spw);
    t.tok0 = tokbase[t.r];
    t.seg0 = (int64_t)t.X * a.S + (int64_t)a.Hkv * segbase[t.r] + (int64_t)t.h * Sr;
    return t;
}

__device__ __forceinline__ size_t thr_index(const CmpArgs& a, const Tile& t, int64_t tok) {
    return ((((size_t)t.X * a.total_tokens + tok) * a.Hkv + t.h) << 2);
}

// ---- magnitude counting helpers -----------------------------------------------------------------------
// Number of the 32 bf16 magnitudes (15-bit patterns, two per word) that are >= cand (0 <= cand <= 0x8000).
__device__ __forceinline__ int count_ge_bf16(const uint32_t* w, uint32_t cand) {
    const u16x2 cc = {(unsigned short)cand, (unsigned short)cand};
    u16x2 acc = {0, 0};
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        const u16x2 m = __builtin_bit_cast(u16x2, w[j] & 0x7FFF7FFFu);
        const u16x2 d = m - cc;          // bit 15 set exactly when m < cand
        acc += d >> (unsigned short)15;
    }
    return 32 - (int)(acc.x + acc.y);
}

__device__ __forceinline__ int count_ge_f32(const uint32_t* w, uint32_t cand) {
    int c = 0;
#pragma unroll
    for (int j = 0; j < 32; ++j) c += ((w[j] & 0x7FFFFFFFu) >= cand) ? 1 : 0;
    return c;
}

__device__ __forceinline__ int sum4i(int v) {
    v += __shfl_xor(v, 1, MKV_WAVE);
    v += __shfl_xor(v, 2, MKV_WAVE);
    return v;
}
__device__ __forceinline__ double sum4d(double v) {
    v += __shfl_xor(v, 1, MKV_WAVE);
    v += __shfl_xor(v, 2, MKV_WAVE);
    return v;
}
// exclusive prefix over the 4 lanes of a vector (lane order = channel order)
__device__ __forceinline__ int excl4(int v, int p) {
    int x = v;
    int y = __shfl_up(x, 1, MKV_WAVE);
    if (p >= 1) x += y;
    y = __shfl_up(x, 2, MKV_WAVE);
    if (p >= 2) x += y;
    return x - v;
}

__device__ __forceinline__ uint32_t lowest_bits(uint32_t m, int k) {
    uint32_t r = 0;
    for (int i = 0; i < k; ++i) { const uint32_t lb = m & (0u - m); r |= lb; m ^= lb; }
    return r;
}

// Value of a magnitude pattern.
__device__ __forceinline__ double mag_value(uint32_t t, bool bf16) {
    return bf16 ? (double)bf16_to_f32(t) : (double)__uint_as_float(t);
}

// ---- per-vector decision: 4 lanes own 32 channels each of one vector ----------------------------------
// Returns the largest code k (smallest count keep[k]) the vector admits; thr[k] gets keep[k]'s threshold.
template <bool BF16>
__device__ __forceinline__ int vector_decide(const uint32_t* w, const CmpArgs& a, uint32_t* thr) {
    double e = 0.0;
    if (BF16) {
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const double lo = bf16_to_f32(w[j] & 0xFFFFu), hi = bf16_to_f32(w[j] >> 16);
            e += lo * lo;
            e += hi * hi;
        }
    } else {
#pragma unroll
        for (int j = 0; j < 32; ++j) { const double x = __uint_as_float(w[j]); e += x * x; }
    }
    const double e_all = sum4d(e);
    const double bound = __dmul_rn(a.frac, e_all);
    int best = 0;
    for (int k = 1; k < a.n_keep; ++k) {
        const int c = a.keep[k];
        uint32_t t = 0;
        const int top = BF16 ? 14 : 30;
        for (int bit = top; bit >= 0; --bit) {
            const uint32_t cand = t | (1u << bit);
            const int ge = sum4i(BF16 ? count_ge_bf16(w, cand) : count_ge_f32(w, cand));
            if (ge >= c) t = cand;
        }
        // energy of the c largest: everything strictly above t, plus (c - gt) copies of t
        double part = 0.0;
        int gt = 0;
        if (BF16) {
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                const uint32_t lo = w[j] & 0xFFFFu, hi = w[j] >> 16;
                if ((lo & 0x7FFFu) > t) { const double x = bf16_to_f32(lo); part += x * x; ++gt; }
                if ((hi & 0x7FFFu) > t) { const double x = bf16_to_f32(hi); part += x * x; ++gt; }
            }
        } else {
#pragma unroll
            for (int j = 0; j < 32; ++j) {
                if ((w[j] & 0x7FFFFFFFu) > t) { const double x = __uint_as_float(w[j]); part += x * x; ++gt; }
            }
        }
        const double tv = mag_value(t, BF16);
        const double ec = sum4d(part) + (double)(c - sum4i(gt)) * (tv * tv);
        thr[k] = t;
        if (ec >= bound) best = k;
    }
    return best;
}

// ---- pack one vector's kept channels into the staging block -------------------------------------------
template <bool BF16>
__device__ __forceinline__ void vector_pack(const uint32_t* w, uint32_t t, int c, int v, int p, int ns,
                                            uint8_t* stg) {
    uint32_t gtm = 0, eqm = 0;
    if (BF16) {
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const uint32_t lo = w[j] & 0x7FFFu, hi = (w[j] >> 16) & 0x7FFFu;
            gtm |= (lo > t ? 1u : 0u) << (2 * j);
            gtm |= (hi > t ? 1u : 0u) << (2 * j + 1);
            eqm |= (lo == t ? 1u : 0u) << (2 * j);
            eqm |= (hi == t ? 1u : 0u) << (2 * j + 1);
        }
    } else {
#pragma unroll
        for (int j = 0; j < 32; ++j) {
            const uint32_t m = w[j] & 0x7FFFFFFFu;
            gtm |= (m > t ? 1u : 0u) << j;
            eqm |= (m == t ? 1u : 0u) << j;
        }
    }
    const int need = c - sum4i(__popc(gtm));
    const int eqc = __popc(eqm);
    const int take = min(max(need - excl4(eqc, p), 0), eqc);
    const uint32_t keepm = gtm | lowest_bits(eqm, take);
    int pos = excl4(__popc(keepm), p);
    const int bv = BF16 ? 2 : 4;
    uint8_t* vals = stg + (size_t)v * c * bv;
    uint8_t* idx = stg + (size_t)ns * c * bv + (size_t)v * c;
    for (int j = 0; j < 32; ++j) {
        if (!((keepm >> j) & 1u)) continue;
        if (BF16) {
            const uint32_t u = (j & 1) ? (w[j >> 1] >> 16) : (w[j >> 1] & 0xFFFFu);
            reinterpret_cast<uint16_t*>(vals)[pos] = (uint16_t)u;
        } else {
            reinterpret_cast<uint32_t*>(vals)[pos] = w[j];
        }
        idx[pos] = (uint8_t)(32 * p + j);
        ++pos;
    }
}

// Segment code: minimum over the valid vectors of the tile (4 waves x 16 vectors).
__device__ __forceinline__ int segment_code(int best, bool valid, int* s_code) {
    int v = valid ? best : 255;
    for (int m = 32; m >= 1; m >>= 1) v = min(v, __shfl_xor(v, m, MKV_WAVE));
    if ((threadIdx.x & 63) == 0) s_code[threadIdx.x >> 6] = v;
    __syncthreads();
    const int code = min(min(s_code[0], s_code[1]), min(s_code[2], s_code[3]));
    return code;
}

// =====================================================================================================
// bf16 kernel: 256 threads; wave w rotates output channels [32w, 32w+32) of a 64x128 tile with MFMA.
// =====================================================================================================
constexpr int XS = 136;   // LDS row stride in u16 (272 B: 16-B aligned, skews banks between rows)

template <bool PACK>
__global__ __launch_bounds__(256) void k_cmp_bf16(CmpArgs a) {
    __shared__ __attribute__((aligned(16))) uint16_t xs[64 * XS];
    __shared__ __attribute__((aligned(16))) uint16_t xh[64 * XS];
    __shared__ __attribute__((aligned(16))) uint8_t stg[64 * 64 * 3];
    __shared__ int s_code[4];

    const Tile t = cmp_tile(a);
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const uint16_t* src = reinterpret_cast<const uint16_t*>(t.X ? a.V : a.K);
    const float* Bm = a.basis ? a.basis + ((((size_t)t.r * a.Hkv + t.h) * 2 + t.X) << 14) : nullptr;

    // basis fragments of this wave's 32 output channels, split into three bf16 parts
    bf16x8 bh[2][4], bmid[2][4], blo[2][4];
    if (Bm) {
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
#pragma unroll
            for (int ks = 0; ks < 4; ++ks)
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const int k = 32 * ks + (lane >> 4) * 8 + i;
                    const int col = 32 * wid + 16 * nt + (lane & 15);
                    const float v = Bm[k * MKV_D + col];
                    const uint32_t hb = f32_to_bf16_rne(v);
                    const float r1 = v - bf16_to_f32(hb);
                    const uint32_t mb = f32_to_bf16_rne(r1);
                    const float r2 = r1 - bf16_to_f32(mb);
                    const uint32_t lb = f32_to_bf16_rne(r2);
                    bh[nt][ks][i] = __builtin_bit_cast(__bf16, (unsigned short)hb);
                    bmid[nt][ks][i] = __builtin_bit_cast(__bf16, (unsigned short)mb);
                    blo[nt][ks][i] = __builtin_bit_cast(__bf16, (unsigned short)lb);
                }
    }
    const uint16_t* rot = Bm ? xh : xs;

    for (int s = t.s0; s < t.s1; ++s) {
        const int ns = min(MKV_SEG, t.n - s * MKV_SEG);
        const int64_t tokS = t.tok0 + (int64_t)s * MKV_SEG;
        const int64_t gs = t.seg0 + s;
        {   // x tile -> LDS (rows past the segment end are zero)
            const int row = tid >> 2, q = tid & 3;
            u32x4* dst = reinterpret_cast<u32x4*>(&xs[row * XS + q * 32]);
            if (row < ns) {
                const u32x4* p = reinterpret_cast<const u32x4*>(src + ((((tokS + row) * a.Hkv + t.h)) << 7) + q * 32);
                const u32x4 v0 = p[0], v1 = p[1], v2 = p[2], v3 = p[3];
                dst[0] = v0; dst[1] = v1; dst[2] = v2; dst[3] = v3;
            } else {
                const u32x4 z = {0, 0, 0, 0};
                dst[0] = z; dst[1] = z; dst[2] = z; dst[3] = z;
            }
        }
        __syncthreads();
        if (Bm) {
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) {
                f32x4 am[2] = {{0, 0, 0, 0}, {0, 0, 0, 0}}, ac[2] = {{0, 0, 0, 0}, {0, 0, 0, 0}};
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) {
                    const bf16x8 A = *reinterpret_cast<const bf16x8*>(&xs[(16 * mt + (lane & 15)) * XS + 32 * ks + (lane >> 4) * 8]);
#pragma unroll
                    for (int nt = 0; nt < 2; ++nt) {
                        am[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, bh[nt][ks], am[nt], 0, 0, 0);
                        ac[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, blo[nt][ks], ac[nt], 0, 0, 0);
                        ac[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, bmid[nt][ks], ac[nt], 0, 0, 0);
                    }
                }
#pragma unroll
                for (int nt = 0; nt < 2; ++nt)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int row = 16 * mt + (lane >> 4) * 4 + i;
                        const int col = 32 * wid + 16 * nt + (lane & 15);
                        xh[row * XS + col] = (uint16_t)f32_to_bf16_rne(am[nt][i] + ac[nt][i]);
                    }
            }
            __syncthreads();
        }

        const int v = tid >> 2, p = tid & 3;
        const bool valid = v < ns;
        uint32_t w[16];
        {
            const u32x4* rp = reinterpret_cast<const u32x4*>(&rot[v * XS + p * 32]);
#pragma unroll
            for (int j = 0; j < 4; ++j) { const u32x4 x = rp[j]; w[4*j] = x.x; w[4*j+1] = x.y; w[4*j+2] = x.z; w[4*j+3] = x.w; }
        }
        if (!PACK) {
            uint32_t thr[4] = {0, 0, 0, 0};
            const int best = vector_decide<true>(w, a, thr);
            const int code = segment_code(best, valid, s_code);
            if (valid && p == 0) {
                uint16_t* tp = a.thr + thr_index(a, t, tokS + v);
                for (int k = 1; k < a.n_keep; ++k) tp[k] = (uint16_t)thr[k];
            }
            if (tid == 0) {
                const int c = a.keep[code];
                a.codes[gs] = (uint8_t)code;
                a.seg_off[gs] = (uint64_t)ns * c * (2 + (c < MKV_D ? 1 : 0));
            }
        } else {
            const int code = a.codes[gs];
            const int c = a.keep[code];
            uint8_t* dst = a.payload + a.seg_off[gs];
            if (c == MKV_D) {
                const int nq = ns * 16;   // 16-byte pieces of ns rows of 256 bytes
                for (int qd = tid; qd < nq; qd += 256) {
                    const int row = qd >> 4, col = (qd & 15) * 8;
                    *reinterpret_cast<u32x4*>(dst + (size_t)qd * 16) = *reinterpret_cast<const u32x4*>(&rot[row * XS + col]);
                }
            } else {
                if (valid) {
                    const uint32_t tt = a.thr[thr_index(a, t, tokS + v) + code];
                    vector_pack<true>(w, tt, c, v, p, ns, stg);
                }
                __syncthreads();
                const int nq = ns * c * 3 / 16;
                for (int qd = tid; qd < nq; qd += 256)
                    *reinterpret_cast<u32x4*>(dst + (size_t)qd * 16) = *reinterpret_cast<const u32x4*>(stg + (size_t)qd * 16);
            }
        }
        __syncthreads();
    }
}

// =====================================================================================================
// fp32 kernel: rotation in float64 on the vector ALUs (one rounding to fp32 at the end).
// =====================================================================================================
constexpr int XF = 132;

template <bool PACK>
__global__ __launch_bounds__(256) void k_cmp_f32(CmpArgs a) {
    extern __shared__ __attribute__((aligned(16))) float lds[];
    float* xs = lds;                  // [64][132]
    float* xh = xs + 64 * XF;         // [64][132]
    float* bs = xh + 64 * XF;         // [128][128]
    __shared__ int s_code[4];

    const Tile t = cmp_tile(a);
    const int tid = threadIdx.x;
    const float* src = reinterpret_cast<const float*>(t.X ? a.V : a.K);
    const float* Bm = a.basis ? a.basis + ((((size_t)t.r * a.Hkv + t.h) * 2 + t.X) << 14) : nullptr;
    if (Bm)
        for (int i = tid; i < MKV_D * MKV_D; i += 256) bs[i] = Bm[i];
    const float* rot = Bm ? xh : xs;
    uint8_t* stg = reinterpret_cast<uint8_t*>(xs);   // reused after the rotation (20 KB <= 33 KB)

    for (int s = t.s0; s < t.s1; ++s) {
        const int ns = min(MKV_SEG, t.n - s * MKV_SEG);
        const int64_t tokS = t.tok0 + (int64_t)s * MKV_SEG;
        const int64_t gs = t.seg0 + s;
        {
            const int row = tid >> 2, q = tid & 3;
            u32x4* dst = reinterpret_cast<u32x4*>(&xs[row * XF + q * 32]);
            if (row < ns) {
                const u32x4* p = reinterpret_cast<const u32x4*>(src + ((((tokS + row) * a.Hkv + t.h)) << 7) + q * 32);
#pragma unroll
                for (int j = 0; j < 8; ++j) dst[j] = p[j];
            } else {
                const u32x4 z = {0, 0, 0, 0};
#pragma unroll
                for (int j = 0; j < 8; ++j) dst[j] = z;
            }
        }
        __syncthreads();
        if (Bm) {
            const int col = tid & 127, r0 = tid >> 7;
            double acc[32];
#pragma unroll
            for (int k = 0; k < 32; ++k) acc[k] = 0.0;
            for (int kk = 0; kk < MKV_D; ++kk) {
                const double b = bs[kk * MKV_D + col];
#pragma unroll
                for (int k = 0; k < 32; ++k) acc[k] = fma((double)xs[(r0 + 2 * k) * XF + kk], b, acc[k]);
            }
#pragma unroll
            for (int k = 0; k < 32; ++k) xh[(r0 + 2 * k) * XF + col] = (float)acc[k];
            __syncthreads();
        }
        const int v = tid >> 2, p = tid & 3;
        const bool valid = v < ns;
        uint32_t w[32];
        {
            const u32x4* rp = reinterpret_cast<const u32x4*>(&rot[v * XF + p * 32]);
#pragma unroll
            for (int j = 0; j < 8; ++j) { const u32x4 x = rp[j]; w[4*j] = x.x; w[4*j+1] = x.y; w[4*j+2] = x.z; w[4*j+3] = x.w; }
        }
        __syncthreads();   // xs is reused as staging below
        if (!PACK) {
            uint32_t thr[4] = {0, 0, 0, 0};
            const int best = vector_decide<false>(w, a, thr);
            const int code = segment_code(best, valid, s_code);
            // an fp32 magnitude threshold takes two of the vector's four 16-bit scratch slots, so fp32 stores
            // support at most two kept counts below 128
            if (valid && p == 0) {
                uint16_t* tp = a.thr + thr_index(a, t, tokS + v);
                for (int k = 1; k < a.n_keep && k < 3; ++k) {
                    tp[2 * (k - 1)] = (uint16_t)(thr[k] & 0xFFFFu);
                    tp[2 * (k - 1) + 1] = (uint16_t)(thr[k] >> 16);
                }
            }
            if (tid == 0) {
                const int c = a.keep[code];
                a.codes[gs] = (uint8_t)code;
                a.seg_off[gs] = (uint64_t)ns * c * (4 + (c < MKV_D ? 1 : 0));
            }
        } else {
            const int code = a.codes[gs];
            const int c = a.keep[code];
            uint8_t* dst = a.payload + a.seg_off[gs];
            if (c == MKV_D) {
                const int nq = ns * 32;   // 16-byte pieces of ns rows of 512 bytes
                for (int qd = tid; qd < nq; qd += 256) {
                    const int row = qd >> 5, col = (qd & 31) * 4;
                    *reinterpret_cast<u32x4*>(dst + (size_t)qd * 16) = *reinterpret_cast<const u32x4*>(&rot[row * XF + col]);
                }
            } else {
                if (valid) {
                    const uint16_t* tp = a.thr + thr_index(a, t, tokS + v);
                    const uint32_t tt = (uint32_t)tp[2 * (code - 1)] | ((uint32_t)tp[2 * (code - 1) + 1] << 16);
                    vector_pack<false>(w, tt, c, v, p, ns, stg);
                }
                __syncthreads();
                const int nq = ns * c * 5 / 16;
                for (int qd = tid; qd < nq; qd += 256)
                    *reinterpret_cast<u32x4*>(dst + (size_t)qd * 16) = *reinterpret_cast<const u32x4*>(stg + (size_t)qd * 16);
            }
        }
        __syncthreads();
    }
}

constexpr size_t kF32Lds = (size_t)(2 * 64 * XF + MKV_D * MKV_D) * sizeof(float);

template <bool PACK>
static hipError_t launch_cmp(const CmpArgs& a, int dtype, hipStream_t s) {
    const dim3 grid(2 * a.nblk), block(256);
    if (a.nblk == 0) return hipSuccess;
    if (dtype == 1) {
        hipLaunchKernelGGL(k_cmp_bf16<PACK>, grid, block, 0, s, a);
    } else {
        static bool attr_set = false;
        if (!attr_set) {
            hipFuncSetAttribute((const void*)k_cmp_f32<PACK>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)kF32Lds);
            attr_set = true;
        }
        hipLaunchKernelGGL(k_cmp_f32<PACK>, grid, block, kF32Lds, s, a);
    }
    return hipGetLastError();
}

hipError_t launch_cmp_decide(const CmpArgs& a, int dtype, hipStream_t s) { return launch_cmp<false>(a, dtype, s); }
hipError_t launch_cmp_pack(const CmpArgs& a, int dtype, hipStream_t s) { return launch_cmp<true>(a, dtype, s); }

// =====================================================================================================
// exclusive scan of the segment sizes (one workgroup; each thread owns a contiguous run)
// =====================================================================================================
__global__ __launch_bounds__(1024) void k_cmp_scan(uint64_t* a, int64_t n, uint64_t* total) {
    __shared__ uint64_t tmp[17];
    const int64_t per = (n + 1023) / 1024;
    const int64_t lo = min((int64_t)threadIdx.x * per, n), hi = min(lo + per, n);
    uint64_t sum = 0;
    for (int64_t i = lo; i < hi; ++i) sum += a[i];
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    uint64_t x = sum;
    for (int d = 1; d < 64; d <<= 1) {
        const uint64_t y = __shfl_up(x, d, MKV_WAVE);
        if (lane >= d) x += y;
    }
    if (lane == 63) tmp[wid] = x;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint64_t run = 0;
        for (int w = 0; w < 16; ++w) { const uint64_t q = tmp[w]; tmp[w] = run; run += q; }
        tmp[16] = run;
    }
    __syncthreads();
    uint64_t run = tmp[wid] + x - sum;
    for (int64_t i = lo; i < hi; ++i) { const uint64_t v = a[i]; a[i] = run; run += v; }
    if (threadIdx.x == 0) *total = tmp[16];
}

hipError_t launch_cmp_scan(uint64_t* seg_off, int64_t count, uint64_t* total, hipStream_t s) {
    hipLaunchKernelGGL(k_cmp_scan, dim3(1), dim3(1024), 0, s, seg_off, count, total);
    return hipGetLastError();
}

}  // namespace mkv
