// Dynamic two-D compression on gfx950 (arXiv 2607.00760, section 1, Observation & Approach 1: per-vector
// element selection after an SVD rotation, one compression strategy per KV-cache segment; Observation &
// Approach 2: the sparse cache is packed into a dense format in GPU memory).
//
// Each workgroup walks a run of consecutive 64-token segment tiles of one (request, KV head, tensor) stream.
// bf16 stores of fixed size take one pass:
//   rotate (MFMA), find per-vector magnitude thresholds of the c largest channels, test the energy rule in
//   float64, pick the segment's kept-channel count, keep the channels above each vector's threshold (ties:
//   lower channel first) and write the segment as one contiguous block (values, then uint8 channel indices)
//   right after the run's previous segment.  Each run starts at the payload position of its first segment
//   slot at full size (64 x 128 values), so runs never overlap and need no scan; the bytes between the end of
//   a run and the next run's start stay unused.
// Growable stores, paged pools and float32 stores take two passes, which pack every run back to back:
//   decide: the same decisions, storing the thresholds; each workgroup records its payload bytes;
//   scan:   exclusive scan of the workgroup totals -> each workgroup's payload offset (pools: pages instead);
//   pack:   rotate again and write the segments as above at the scanned offsets.
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
    launch_kernel(k_upload, dim3(1), dim3(256), 0, s, u);
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
    const int32_t* scap = a.tab + 3 * a.B;
    const int32_t* cblk = a.tab + 4 * a.B;
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
    t.seg0 = (int64_t)t.X * a.S + (int64_t)a.Hkv * segbase[t.r] + (int64_t)t.h * scap[t.r];
    return t;
}

__device__ __forceinline__ size_t thr_index(const CmpArgs& a, const Tile& t, int64_t tok) {
    return ((((size_t)t.X * a.total_tokens + tok) * a.Hkv + t.h) << 2);
}

// =====================================================================================================
// fp32 path: 4 lanes per vector, each owning 32 channels
// =====================================================================================================
// Number of this lane's 32 float32 magnitudes that are >= cand.
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

// Largest code k (smallest count keep[k]) the vector admits; thr[k] gets the magnitude pattern of its keep[k]-th
// largest value, found bit by bit over the 31-bit float32 magnitude.
__device__ __forceinline__ int vector_decide_f32(const uint32_t* w, const CmpArgs& a, uint32_t* thr) {
    double e = 0.0;
#pragma unroll
    for (int j = 0; j < 32; ++j) { const double x = __uint_as_float(w[j]); e += x * x; }
    const double e_all = sum4d(e);
    const double bound = __dmul_rn(a.frac, e_all);
    int best = 0;
    for (int k = 1; k < a.n_keep; ++k) {
        const int c = a.keep[k];
        uint32_t t = 0;
        for (int bit = 30; bit >= 0; --bit) {
            const uint32_t cand = t | (1u << bit);
            if (sum4i(count_ge_f32(w, cand)) >= c) t = cand;
        }
        // energy of the c largest: everything strictly above t, plus (c - gt) copies of t
        double part = 0.0;
        int gt = 0;
#pragma unroll
        for (int j = 0; j < 32; ++j) {
            if ((w[j] & 0x7FFFFFFFu) > t) { const double x = __uint_as_float(w[j]); part += x * x; ++gt; }
        }
        const double tv = (double)__uint_as_float(t);
        const double ec = sum4d(part) + (double)(c - sum4i(gt)) * (tv * tv);
        thr[k] = t;
        if (ec >= bound) best = k;
    }
    return best;
}

// This lane's kept channels of one vector into the staging block (values [ns][c] then indices [ns][c]); among
// values equal to the threshold the lower channels are kept.
__device__ __forceinline__ void vector_pack_f32(const uint32_t* w, uint32_t t, int c, int v, int p, int ns,
                                                uint8_t* stg) {
    uint32_t gtm = 0, eqm = 0;
#pragma unroll
    for (int j = 0; j < 32; ++j) {
        const uint32_t m = w[j] & 0x7FFFFFFFu;
        gtm |= (m > t ? 1u : 0u) << j;
        eqm |= (m == t ? 1u : 0u) << j;
    }
    const int need = c - sum4i(__popc(gtm));
    const int eqc = __popc(eqm);
    const int take = min(max(need - excl4(eqc, p), 0), eqc);
    const uint32_t keepm = gtm | lowest_bits(eqm, take);
    int pos = excl4(__popc(keepm), p);
    uint8_t* vals = stg + (size_t)v * c * 4;
    uint8_t* idx = stg + (size_t)ns * c * 4 + (size_t)v * c;
    for (int j = 0; j < 32; ++j) {
        if (!((keepm >> j) & 1u)) continue;
        reinterpret_cast<uint32_t*>(vals)[pos] = w[j];
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
// bf16 path: 8 lanes per vector, each owning 16 channels (8 words of packed 16-bit magnitudes)
// =====================================================================================================
__device__ __forceinline__ int uni(int x) { return __builtin_amdgcn_readfirstlane(x); }

template <int CTRL>
__device__ __forceinline__ int dpp_i(int v) { return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false); }
__device__ __forceinline__ int sum8i(int v) {
    v += dpp_i<0xB1>(v);
    v += dpp_i<0x4E>(v);
    v += dpp_i<0x141>(v);
    return v;
}
__device__ __forceinline__ uint32_t max8u(uint32_t v) {
    v = max(v, (uint32_t)dpp_i<0xB1>((int)v));
    v = max(v, (uint32_t)dpp_i<0x4E>((int)v));
    v = max(v, (uint32_t)dpp_i<0x141>((int)v));
    return v;
}
__device__ __forceinline__ uint32_t min8u(uint32_t v) {
    v = min(v, (uint32_t)dpp_i<0xB1>((int)v));
    v = min(v, (uint32_t)dpp_i<0x4E>((int)v));
    v = min(v, (uint32_t)dpp_i<0x141>((int)v));
    return v;
}
// 64-bit values move between lanes as two 32-bit DPP moves (no LDS round trip)
template <int CTRL>
__device__ __forceinline__ double dpp_d(double v) {
    const uint64_t u = (uint64_t)__double_as_longlong(v);
    const uint32_t lo = (uint32_t)dpp_i<CTRL>((int)(uint32_t)u), hi = (uint32_t)dpp_i<CTRL>((int)(uint32_t)(u >> 32));
    return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}
__device__ __forceinline__ double sum8d(double v) {
    v += dpp_d<0xB1>(v);
    v += dpp_d<0x4E>(v);
    v += dpp_d<0x141>(v);
    return v;
}
// exclusive prefix over the 8 lanes of a vector (lane order = channel order): DPP row shifts by 1, 2, 4, each
// added only where the source lane belongs to the same vector
__device__ __forceinline__ int excl8(int v, int p) {
    int x = v;
    int y = dpp_i<0x111>(x);
    if (p >= 1) x += y;
    y = dpp_i<0x112>(x);
    if (p >= 2) x += y;
    y = dpp_i<0x114>(x);
    if (p >= 4) x += y;
    return x - v;
}
// This lane's 16 magnitudes (mw: 15-bit patterns, two per word) as 7-bit search keys, four per word with the top
// bit of every byte set: key = min((m - base) >> sh, 127), and 0 for m < base.
__device__ __forceinline__ void swar_keys(const uint32_t* mw, uint32_t base, int sh, uint32_t (&kw)[4]) {
    typedef __attribute__((ext_vector_type(2))) unsigned short u16v2;
    const u16v2 b2 = {(unsigned short)base, (unsigned short)base};
    const u16v2 cap = {127, 127};
    const u16v2 sh2 = {(unsigned short)sh, (unsigned short)sh};
    uint32_t u[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        u16v2 x = __builtin_bit_cast(u16v2, mw[j]);
        x = __builtin_elementwise_sub_sat(x, b2);
        x = x >> sh2;
        x = __builtin_elementwise_min(x, cap);
        u[j] = __builtin_bit_cast(uint32_t, x);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) kw[j] = __builtin_amdgcn_perm(u[2 * j + 1], u[2 * j], 0x06040200u) | 0x80808080u;
}
// Number of this lane's 16 keys >= t (0 <= t <= 127), given tt = t in every byte: per byte, (key | 0x80) - t
// keeps its top bit iff key >= t, and no byte borrows from its neighbour.
__device__ __forceinline__ int swar_count_ge(const uint32_t (&kw)[4], uint32_t tt) {
    int n = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) n += __popc((kw[j] - tt) & 0x80808080u);
    return n;
}

// Magnitude pattern of the c-th largest of the vector's 128 values, given lo_end with at least c values >= lo_end
// and the largest value mx: the largest t with count(m >= t) >= c, found by halving the integer range
// [lo_end, lo_end + 2^L) with L bits, enough for every vector of the wave (a wider range than a vector needs
// gives the same t, since no t above mx has c values at or above it; one L per wave keeps the loops uniform).
// The range is cut into phases of up to 7 bits (the top phase takes what is left over): each phase turns the
// magnitudes into 7-bit keys relative to the range's low end and searches the key bit by bit, counting four keys
// per 32-bit word; values above the phase's range saturate at key 127 and still count.
__device__ __forceinline__ uint32_t vector_threshold8(const uint32_t* mw, uint32_t lo_end, uint32_t mx, int c) {
    uint32_t base = lo_end;
    uint32_t wdt = mx - lo_end;
    wdt = max(wdt, (uint32_t)dpp_i<0xB1>((int)wdt));
    wdt = max(wdt, (uint32_t)dpp_i<0x4E>((int)wdt));
    wdt = max(wdt, (uint32_t)dpp_i<0x141>((int)wdt));
    wdt = max(wdt, (uint32_t)dpp_i<0x140>((int)wdt));   // the largest of each row of 16 lanes
    wdt = max(max((uint32_t)__builtin_amdgcn_readlane((int)wdt, 0), (uint32_t)__builtin_amdgcn_readlane((int)wdt, 16)),
              max((uint32_t)__builtin_amdgcn_readlane((int)wdt, 32), (uint32_t)__builtin_amdgcn_readlane((int)wdt, 48)));
    int L = wdt ? 32 - __clz(wdt) : 0;
    while (L > 0) {
        const int sh = ((L - 1) / 7) * 7;
        uint32_t kw[4];
        swar_keys(mw, base, sh, kw);
        uint32_t tt = 0;   // the key found so far, in every byte
        for (int bit = L - sh - 1; bit >= 0; --bit) {
            const uint32_t cand = tt | (0x01010101u << bit);
            if (sum8i(swar_count_ge(kw, cand)) >= c) tt = cand;
        }
        base += (tt & 0x7Fu) << sh;
        L = sh;
    }
    return base;
}

// Largest code k the vector admits (keep[k] channels hold >= frac of its energy); thr[k] <- the magnitude of its
// keep[k]-th largest value.  Thresholds come from vector_threshold8 over the range [smallest magnitude, largest]
// for the first count; smaller counts are searched above the previous threshold.
// Called by every thread of the workgroup (64 vectors of one segment): before searching level k >= 2 the
// workgroup checks whether some valid vector already cannot reach it, either because it failed level k-1 or
// because an upper bound on its top keep[k] energy is below the target.  Two bounds, both from level k-1:
// E_{k-1} - (keep[k-1] - keep[k]) * t_{k-1}^2 (each of the dropped values is at least t_{k-1}), and, with
// u = 2 t_{k-1} and m = the number of values >= u, E(values >= u) + (keep[k] - m) * u^2 when m <= keep[k] (the
// top keep[k] are those m values and keep[k] - m values below u).  Then no vector's result at level k can
// change the segment's code, and the search stops for the whole workgroup.  s_fail: per-level flags, zero on
// entry.
__device__ __forceinline__ int vector_decide8(const uint32_t* w, const CmpArgs& a, uint32_t* thr, bool valid,
                                              int* s_fail) {
    double e = 0.0;
    u16x2 mx2 = {0, 0}, mn2 = {0x7FFF, 0x7FFF};
    uint32_t mw[8];   // magnitude patterns
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        mw[j] = w[j] & 0x7FFF7FFFu;
        const double lo = bf16_to_f32(w[j] & 0xFFFFu), hi = bf16_to_f32(w[j] >> 16);
        e += lo * lo;
        e += hi * hi;
        const u16x2 m = __builtin_bit_cast(u16x2, mw[j]);
        mx2 = __builtin_elementwise_max(mx2, m);
        mn2 = __builtin_elementwise_min(mn2, m);
    }
    const double e_all = sum8d(e);
    const double bound = __dmul_rn(a.frac, e_all);
    const uint32_t mx = max8u(max((uint32_t)mx2.x, (uint32_t)mx2.y));
    uint32_t lo_end = min8u(min((uint32_t)mn2.x, (uint32_t)mn2.y));
    int best = 0;
    double ec_prev = e_all, tv_prev = 0.0, ub2_prev = INFINITY;
    for (int k = 1; k < a.n_keep; ++k) {
        const int c = a.keep[k];
        if (k >= 2) {
            // the margin keeps fp64 rounding of the bound from ever flagging a vector that reaches level k
            const double ub = fmin(ec_prev - (double)(a.keep[k - 1] - c) * (tv_prev * tv_prev), ub2_prev);
            if (valid && (best < k - 1 || ub + 1e-10 * e_all < bound)) s_fail[k] = 1;
            __syncthreads();
            if (s_fail[k]) break;
        }
        const uint32_t t = vector_threshold8(mw, lo_end, mx, c);
        // kept energy from the magnitudes, squared in float64 (exact for every bf16 value, subnormals and values
        // beyond 2^64 included); recomputed from the magnitude words rather than kept from the total (the signed
        // words): holding the 16 float64 values across the search costs registers
        // u: the magnitude pattern one exponent step above t (a larger value; at least twice t for normal t)
        const uint32_t u = t + 128u;
        double part = 0.0, eu = 0.0;
        int gt = 0, mu = 0;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const uint32_t lo = mw[j] & 0xFFFFu, hi = mw[j] >> 16;
            const double xl = bf16_to_f32(lo), xh = bf16_to_f32(hi);
            if (lo > t) { part += xl * xl; ++gt; }
            if (hi > t) { part += xh * xh; ++gt; }
            if (lo >= u) { eu += xl * xl; ++mu; }
            if (hi >= u) { eu += xh * xh; ++mu; }
        }
        const double tv = bf16_to_f32(t);
        const double ec = sum8d(part) + (double)(c - sum8i(gt)) * (tv * tv);
        if (k + 1 < a.n_keep) {
            const int cn = a.keep[k + 1], m = sum8i(mu);
            const double es = sum8d(eu), uv = bf16_to_f32(u);
            ub2_prev = (u < 0x7F80u && m <= cn) ? es + (double)(cn - m) * (uv * uv) : INFINITY;
        }
        thr[k] = t;
        if (ec >= bound) best = k;
        lo_end = t;
        ec_prev = ec;
        tv_prev = tv;
    }
    return best;
}

// This lane's kept channels of one vector into the staging block (values [ns][c] then indices [ns][c]).
__device__ __forceinline__ void vector_pack8(const uint32_t* w, uint32_t t, int c, int v, int p, int ns, uint8_t* stg) {
    uint32_t gtm = 0, eqm = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const uint32_t lo = w[j] & 0x7FFFu, hi = (w[j] >> 16) & 0x7FFFu;
        gtm |= (lo > t ? 1u : 0u) << (2 * j);
        gtm |= (hi > t ? 1u : 0u) << (2 * j + 1);
        eqm |= (lo == t ? 1u : 0u) << (2 * j);
        eqm |= (hi == t ? 1u : 0u) << (2 * j + 1);
    }
    const int need = c - sum8i(__popc(gtm));
    const int eqc = __popc(eqm);
    const int take = min(max(need - excl8(eqc, p), 0), eqc);
    const uint32_t keepm = gtm | lowest_bits(eqm, take);
    int pos = excl8(__popc(keepm), p);
    uint16_t* vals = reinterpret_cast<uint16_t*>(stg) + (size_t)v * c;
    uint8_t* idx = stg + (size_t)ns * c * 2 + (size_t)v * c;
    for (int j = 0; j < 16; ++j) {
        if (!((keepm >> j) & 1u)) continue;
        vals[pos] = (uint16_t)((j & 1) ? (w[j >> 1] >> 16) : (w[j >> 1] & 0xFFFFu));
        idx[pos] = (uint8_t)(16 * p + j);
        ++pos;
    }
}

// Segment code: minimum over the valid vectors of the tile (8 waves x 8 vectors).
__device__ __forceinline__ int segment_code8(int best, bool valid, int* s_code) {
    // best is the same on the 8 lanes of a vector: the two vectors of each row of 16 lanes meet by a row mirror,
    // the four rows through scalar reads
    int v = valid ? best : 255;
    v = min(v, dpp_i<0x140>(v));
    v = min(min(__builtin_amdgcn_readlane(v, 0), __builtin_amdgcn_readlane(v, 16)),
            min(__builtin_amdgcn_readlane(v, 32), __builtin_amdgcn_readlane(v, 48)));
    if ((threadIdx.x & 63) == 0) s_code[threadIdx.x >> 6] = v;
    __syncthreads();
    int code = s_code[0];
#pragma unroll
    for (int w = 1; w < 8; ++w) code = min(code, s_code[w]);
    return code;
}

// =====================================================================================================
// bf16 kernel: 512 threads; wave w rotates output channels [16w, 16w+16) of each 64x128 tile with MFMA
// (16x16x32 bf16, the fp32 basis split into three bf16 parts held in registers); tiles are double-buffered
// in LDS, the next one loaded while the current one is rotated and selected.
// =====================================================================================================
constexpr int XS = 136;   // LDS row stride in u16 (272 B: 16-B aligned, skews banks between rows)
// kernel modes: the decide pass, the pack pass, or both in one pass (segment runs at their slot positions)
constexpr int kCmpDecide = 0, kCmpPack = 1, kCmpFused = 2;

// MFMA B fragments of basis columns [16 wid, 16 wid + 16): the float32 basis split into three bf16 parts
// (hi + mid + lo), so that the bf16 products summed in float32 reproduce the float32 basis.  The same
// arithmetic, in the same order, as the compressor's inline copy (so appended segments match compressed ones).
__device__ __forceinline__ void basis_frags(const float* Bm, int wid, int lane, bf16x8 (&bh)[4], bf16x8 (&bmid)[4],
                                            bf16x8 (&blo)[4]) {
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int k = 32 * ks + (lane >> 4) * 8 + i;
            const int col = 16 * wid + (lane & 15);
            const float v = Bm[k * MKV_D + col];
            const uint32_t hb = f32_to_bf16_rne(v);
            const float r1 = v - bf16_to_f32(hb);
            const uint32_t mb = f32_to_bf16_rne(r1);
            const float r2 = r1 - bf16_to_f32(mb);
            const uint32_t lb = f32_to_bf16_rne(r2);
            bh[ks][i] = __builtin_bit_cast(__bf16, (unsigned short)hb);
            bmid[ks][i] = __builtin_bit_cast(__bf16, (unsigned short)mb);
            blo[ks][i] = __builtin_bit_cast(__bf16, (unsigned short)lb);
        }
}

// Two float32 values rounded to bf16 (nearest, ties to even) and packed low | high << 16: the casts compile to
// gfx950's conversion instruction, which rounds the same way as f32_to_bf16_rne for every finite value.
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2v;
__device__ __forceinline__ uint32_t pack2_bf16(float lo, float hi) {
    bf16x2v r;
    r.x = (__bf16)lo;
    r.y = (__bf16)hi;
    return __builtin_bit_cast(uint32_t, r);
}

// Output channels [16 wid, 16 wid + 16) of a 64 x 128 tile: xh = round_bf16(X @ B) (LDS, row stride XS).
__device__ __forceinline__ void rotate_tile(const uint16_t* X, uint16_t* xh, const bf16x8 (&bh)[4],
                                            const bf16x8 (&bmid)[4], const bf16x8 (&blo)[4], int wid, int lane) {
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
        f32x4 am = {0, 0, 0, 0}, ac = {0, 0, 0, 0};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const bf16x8 A = *reinterpret_cast<const bf16x8*>(&X[(16 * mt + (lane & 15)) * XS + 32 * ks + (lane >> 4) * 8]);
            am = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bh[ks], A, am, 0, 0, 0);
            ac = __builtin_amdgcn_mfma_f32_16x16x32_bf16(blo[ks], A, ac, 0, 0, 0);
            ac = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bmid[ks], A, ac, 0, 0, 0);
        }
        // the product is taken transposed (basis rows times tile columns): this lane holds channels
        // 16 wid + 4 (lane / 16) .. + 3 of row 16 mt + lane % 16, stored as one 8-byte write
        u32x2 pk;
        pk.x = pack2_bf16(am[0] + ac[0], am[1] + ac[1]);
        pk.y = pack2_bf16(am[2] + ac[2], am[3] + ac[3]);
        *reinterpret_cast<u32x2*>(&xh[(16 * mt + (lane & 15)) * XS + 16 * wid + 4 * (lane >> 4)]) = pk;
    }
}

// Four waves per SIMD (128 registers) so that two workgroups share a CU and one's MFMA rotation overlaps the
// other's threshold search; with the lo basis parts in LDS (decide and one-pass modes) a few registers still
// spill to scratch, with all three parts in registers (pack pass) none.
template <int MODE>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(4, 4))) void k_cmp_bf16(CmpArgs a) {
    constexpr bool PACK = MODE == kCmpPack, DECIDE = MODE != kCmpPack, WRITE = MODE != kCmpDecide;
    // decide and one-pass modes keep the lo parts of the basis fragments in LDS (8 waves x 4 KB) instead of
    // registers, and then use one tile buffer: with a basis the input tile is read only by the rotation, so the
    // next tile can land in the same buffer at the end of the segment.  Without a basis (the decision reads the
    // input tile itself) the lo area is the second tile buffer; the pack pass keeps two buffers and registers.
    constexpr bool LO_LDS = MODE != kCmpPack;
    __shared__ __attribute__((aligned(16))) uint16_t xs0[64 * XS];
    __shared__ __attribute__((aligned(16))) uint16_t xsB[LO_LDS ? 8 * 4 * 64 * 8 : 64 * XS];
    __shared__ __attribute__((aligned(16))) uint16_t xh[64 * XS];
    __shared__ __attribute__((aligned(16))) uint8_t stg[64 * 64 * 3];
    __shared__ int s_code[8];
    __shared__ int s_fail[2][4];   // per segment parity: levels some vector cannot reach

    const Tile t = cmp_tile(a);
    const int tid = threadIdx.x, lane = tid & 63, wid = uni(tid >> 6);
    const uint16_t* src = reinterpret_cast<const uint16_t*>(t.X ? a.V : a.K);
    const float* Bm = a.basis ? a.basis + ((((size_t)t.r * a.Hkv + t.h) * 2 + t.X) << 14) : nullptr;

    // the basis fragments and the rotation below are written out here rather than through basis_frags() and
    // rotate_tile(): with the helpers the compiler spills more of this kernel's registers (measured slower)
    bf16x8 bh[4], bmid[4], blo[4];
    if (Bm) {
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int k = 32 * ks + (lane >> 4) * 8 + i;
                const int col = 16 * wid + (lane & 15);
                const float v = Bm[k * MKV_D + col];
                const uint32_t hb = f32_to_bf16_rne(v);
                const float r1 = v - bf16_to_f32(hb);
                const uint32_t mb = f32_to_bf16_rne(r1);
                const float r2 = r1 - bf16_to_f32(mb);
                const uint32_t lb = f32_to_bf16_rne(r2);
                bh[ks][i] = __builtin_bit_cast(__bf16, (unsigned short)hb);
                bmid[ks][i] = __builtin_bit_cast(__bf16, (unsigned short)mb);
                blo[ks][i] = __builtin_bit_cast(__bf16, (unsigned short)lb);
            }
        if (LO_LDS) {   // each wave's own 4 KB, read back by the same lanes only
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) reinterpret_cast<bf16x8*>(xsB)[(wid * 4 + ks) * 64 + lane] = blo[ks];
        }
    }
    const bool dbl = !LO_LDS || !Bm;   // two tile buffers
    uint16_t* const xb0 = xs0;
    uint16_t* const xb1 = dbl ? xsB : xs0;
    // tile rows: thread -> row tid/8, 16 channels (32 bytes) starting at 16 * (tid % 8)
    const int lrow = tid >> 3, lq = tid & 7;
    u32x4 r0 = {0, 0, 0, 0}, r1 = {0, 0, 0, 0};
    auto load_tile = [&](int s) {
        const int ns = min(MKV_SEG, t.n - s * MKV_SEG);
        if (lrow < ns) {
            const int64_t tok = t.tok0 + (int64_t)s * MKV_SEG + lrow;
            const u32x4* p = reinterpret_cast<const u32x4*>(src + ((tok * a.Hkv + t.h) << 7) + lq * 16);
            r0 = p[0];
            r1 = p[1];
        } else {
            r0 = u32x4{0, 0, 0, 0};
            r1 = u32x4{0, 0, 0, 0};
        }
    };
    auto store_tile = [&](uint16_t* X) {
        u32x4* d = reinterpret_cast<u32x4*>(&X[lrow * XS + lq * 16]);
        d[0] = r0;
        d[1] = r1;
    };
    if (t.s0 < t.s1) {
        load_tile(t.s0);
        store_tile(xb0);
    }
    if (tid < 8) s_fail[tid >> 2][tid & 3] = 0;
    uint64_t wg_bytes = 0;   // decide, one pass: payload bytes of this workgroup
    // offset of this workgroup's first segment: scanned (pack) or its full-size slot position (one pass)
    uint64_t wg_off = PACK ? a.wg_total[blockIdx.x]
                    : MODE == kCmpFused ? (uint64_t)(t.seg0 + t.s0) * (MKV_SEG * MKV_D * 2) : 0;
    // pack: the segment code and this thread's vector's thresholds are loaded one segment ahead, so that their
    // latency overlaps the previous segment
    int code_n = 0;
    u32x2 thr_n = {0u, 0u};
    auto load_meta = [&](int s) {
        code_n = a.codes[t.seg0 + s];
        if ((tid >> 3) < min(MKV_SEG, t.n - s * MKV_SEG))
            thr_n = *reinterpret_cast<const u32x2*>(a.thr + thr_index(a, t, t.tok0 + (int64_t)s * MKV_SEG + (tid >> 3)));
    };
    if (PACK && t.s0 < t.s1) load_meta(t.s0);

    for (int s = t.s0; s < t.s1; ++s) {
        const int cur = (s - t.s0) & 1;
        const int ns = min(MKV_SEG, t.n - s * MKV_SEG);
        const int64_t tokS = t.tok0 + (int64_t)s * MKV_SEG;
        const int64_t gs = t.seg0 + s;
        __syncthreads();
        // the other parity's flags were last read in the previous segment, before this barrier
        if (tid < 4) s_fail[cur ^ 1][tid] = 0;
        const bool more = s + 1 < t.s1;
        const int code_c = code_n;
        const u32x2 thr_c = thr_n;
        if (more) {
            load_tile(s + 1);
            if (PACK) load_meta(s + 1);
        }
        const uint16_t* X = cur ? xb1 : xb0;
        if (Bm) {
            if (LO_LDS) {
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) blo[ks] = reinterpret_cast<const bf16x8*>(xsB)[(wid * 4 + ks) * 64 + lane];
            }
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) {
                f32x4 am = {0, 0, 0, 0}, ac = {0, 0, 0, 0};
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) {
                    const bf16x8 A = *reinterpret_cast<const bf16x8*>(&X[(16 * mt + (lane & 15)) * XS + 32 * ks + (lane >> 4) * 8]);
                    am = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bh[ks], A, am, 0, 0, 0);
                    ac = __builtin_amdgcn_mfma_f32_16x16x32_bf16(blo[ks], A, ac, 0, 0, 0);
                    ac = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bmid[ks], A, ac, 0, 0, 0);
                }
                // the product is taken transposed (basis rows times tile columns): this lane holds channels
                // 16 wid + 4 (lane / 16) .. + 3 of row 16 mt + lane % 16, stored as one 8-byte write
                u32x2 pk;
                pk.x = pack2_bf16(am[0] + ac[0], am[1] + ac[1]);
                pk.y = pack2_bf16(am[2] + ac[2], am[3] + ac[3]);
                *reinterpret_cast<u32x2*>(&xh[(16 * mt + (lane & 15)) * XS + 16 * wid + 4 * (lane >> 4)]) = pk;
            }
            __syncthreads();
        }
        const uint16_t* R = Bm ? xh : X;
        const int v = tid >> 3, p = tid & 7;
        const bool valid = v < ns;
        uint32_t w[8];
        auto read_vector = [&]() {
            const u32x4* rp = reinterpret_cast<const u32x4*>(&R[v * XS + p * 16]);
            const u32x4 x0 = rp[0], x1 = rp[1];
            w[0] = x0.x; w[1] = x0.y; w[2] = x0.z; w[3] = x0.w;
            w[4] = x1.x; w[5] = x1.y; w[6] = x1.z; w[7] = x1.w;
        };
        read_vector();
        int code_f = 0;
        uint32_t thr_f = 0;
        if (DECIDE) {
            uint32_t thr[4] = {0, 0, 0, 0};
            const int best = vector_decide8(w, a, thr, valid, s_fail[cur]);
            const int code = uni(segment_code8(best, valid, s_code));   // the same in every thread
            if (MODE == kCmpDecide && valid && p == 0) {
                uint16_t* tp = a.thr + thr_index(a, t, tokS + v);
                for (int k = 1; k < a.n_keep; ++k) tp[k] = (uint16_t)thr[k];
            }
            if (tid == 0) {
                const int c = a.keep[code];
                a.codes[gs] = (uint8_t)code;
                wg_bytes += (uint64_t)ns * c * (2 + (c < MKV_D ? 1 : 0));
            }
            code_f = code;
            thr_f = code == 1 ? thr[1] : code == 2 ? thr[2] : thr[3];
            // the vector again from LDS (past the barrier in segment_code8) rather than held across the search
            if (MODE == kCmpFused) read_vector();
        }
        if (WRITE) {
            const int code = PACK ? code_c : code_f;
            const int c = a.keep[code];
            uint8_t* dst = a.payload + (a.preplaced ? a.seg_off[gs] : wg_off);
            if (!a.preplaced && tid == 0) a.seg_off[gs] = wg_off;
            wg_off += (uint64_t)ns * c * (2 + (c < MKV_D ? 1 : 0));
            if (a.open_rows && ns < MKV_SEG && lrow < ns) {
                // growable store: the stream's unfinished last segment keeps its original rows for appends
                const int os = a.tab[5 * a.B + 1 + t.r];
                uint16_t* orow = a.open_rows + (((int64_t)os * a.Hkv + t.h) * 2 + t.X) * a.open_elems;
                u32x4* d = reinterpret_cast<u32x4*>(orow + lrow * MKV_D + lq * 16);
                const u32x4* q = reinterpret_cast<const u32x4*>(&X[lrow * XS + lq * 16]);
                d[0] = q[0];
                d[1] = q[1];
            }
            if (c == MKV_D) {
                const int nq = ns * 16;   // 16-byte pieces of ns rows of 256 bytes
                for (int qd = tid; qd < nq; qd += 512) {
                    const int row = qd >> 4, col = (qd & 15) * 8;
                    // written once and not read again in this pass: non-temporal
                    __builtin_nontemporal_store(*reinterpret_cast<const u32x4*>(&R[row * XS + col]), reinterpret_cast<u32x4*>(dst + (size_t)qd * 16));
                }
            } else {
                if (valid) {
                    const uint32_t tt = PACK ? ((code & 2) ? thr_c.y : thr_c.x) >> (16 * (code & 1)) & 0xFFFFu : thr_f;
                    vector_pack8(w, tt, c, v, p, ns, stg);
                }
                __syncthreads();
                const int nq = ns * c * 3 / 16;
                for (int qd = tid; qd < nq; qd += 512)
                    __builtin_nontemporal_store(*reinterpret_cast<const u32x4*>(stg + (size_t)qd * 16), reinterpret_cast<u32x4*>(dst + (size_t)qd * 16));
            }
        }
        if (more) store_tile(cur ? xb0 : xb1);
    }
    if (MODE == kCmpDecide && tid == 0) a.wg_total[blockIdx.x] = wg_bytes;
    if (MODE == kCmpFused && tid == 0 && wg_bytes) atomicAdd(reinterpret_cast<unsigned long long*>(a.total), wg_bytes);
}

// =====================================================================================================
// append: one token joins the open (last, unfinished) segment of each listed stream of a growable bf16 store
// =====================================================================================================
// One workgroup per (listed request, KV head, tensor).  The open segment's earlier rows (kept unrotated in the
// store) and the new row form the tile; the tile is rotated, decided and packed by the same code as the
// compressor, so the segment ends up exactly as compressing the extended context would leave it.  An open
// segment lives in its stream's open area; the append that completes it (64 tokens) seals it into the payload
// at a position taken from the payload counter, or (pools) at the position the host reserved for it.
__global__ __launch_bounds__(512) void k_cmp_append(CmpArgs a, AppendArgs x) {
    __shared__ __attribute__((aligned(16))) uint16_t xs[64 * XS];
    __shared__ __attribute__((aligned(16))) uint16_t xh[64 * XS];
    __shared__ __attribute__((aligned(16))) uint8_t stg[64 * 64 * 3];
    __shared__ int s_code[8];
    __shared__ int s_fail[4];
    __shared__ unsigned long long s_pos;
    const int tid = threadIdx.x, lane = tid & 63, wid = uni(tid >> 6);
    const int ai = blockIdx.x / (2 * x.Hkv), rem = blockIdx.x - ai * 2 * x.Hkv, h = rem >> 1, X = rem & 1;
    const int kr = x.tab[5 * ai], n_old = x.tab[5 * ai + 1], os = x.tab[5 * ai + 4];
    const int p = n_old & (MKV_SEG - 1), ns = p + 1;
    const int64_t g = (int64_t)X * x.S + x.tab[5 * ai + 2] + (int64_t)h * x.tab[5 * ai + 3] + (n_old >> 6);
    const int64_t st = ((int64_t)os * x.Hkv + h) * 2 + X;
    uint16_t* rows = x.open_rows + st * (int64_t)(x.open_bytes / 2);
    const uint16_t* nr = (X ? x.Vn : x.Kn) + ((int64_t)kr * x.Hkv + h) * MKV_D;
    const float* Bm = x.basis ? x.basis + ((((size_t)os * x.Hkv + h) * 2 + X) << 14) : nullptr;
    bf16x8 bh[4], bmid[4], blo[4];
    if (Bm) basis_frags(Bm, wid, lane, bh, bmid, blo);

    // tile: earlier rows of the open segment, the new row (also kept for later appends), zeros
    const int lrow = tid >> 3, lq = tid & 7;
    u32x4 r0 = {0, 0, 0, 0}, r1 = {0, 0, 0, 0};
    if (lrow < p) {
        const u32x4* q = reinterpret_cast<const u32x4*>(rows + lrow * MKV_D + lq * 16);
        r0 = q[0];
        r1 = q[1];
    } else if (lrow == p) {
        const u32x4* q = reinterpret_cast<const u32x4*>(nr + lq * 16);
        r0 = q[0];
        r1 = q[1];
        u32x4* d = reinterpret_cast<u32x4*>(rows + p * MKV_D + lq * 16);
        d[0] = r0;
        d[1] = r1;
    }
    {
        u32x4* d = reinterpret_cast<u32x4*>(&xs[lrow * XS + lq * 16]);
        d[0] = r0;
        d[1] = r1;
    }
    if (tid < 4) s_fail[tid] = 0;
    __syncthreads();
    if (Bm) {
        rotate_tile(xs, xh, bh, bmid, blo, wid, lane);
        __syncthreads();
    }
    const uint16_t* R = Bm ? xh : xs;
    const int v = tid >> 3, pl = tid & 7;
    const bool valid = v < ns;
    uint32_t w[8];
    {
        const u32x4* rp = reinterpret_cast<const u32x4*>(&R[v * XS + pl * 16]);
        const u32x4 x0 = rp[0], x1 = rp[1];
        w[0] = x0.x; w[1] = x0.y; w[2] = x0.z; w[3] = x0.w;
        w[4] = x1.x; w[5] = x1.y; w[6] = x1.z; w[7] = x1.w;
    }
    uint32_t thr[4] = {0, 0, 0, 0};
    const int best = vector_decide8(w, a, thr, valid, s_fail);
    const int code = segment_code8(best, valid, s_code);
    const int c = a.keep[code];
    if (tid == 0) {
        const uint64_t bytes = (uint64_t)ns * c * (2 + (c < MKV_D ? 1 : 0));
        s_pos = ns < MKV_SEG ? x.open_pack + st * x.open_bytes
              : x.seal_off ? x.seal_off[blockIdx.x] : atomicAdd(x.total, (unsigned long long)bytes);
        x.codes[g] = (uint8_t)code;
    }
    if (c < MKV_D && valid) vector_pack8(w, thr[code], c, v, pl, ns, stg);
    __syncthreads();
    const uint64_t pos = s_pos;
    uint8_t* dst = x.payload + pos;
    if (c == MKV_D) {
        for (int qd = tid; qd < ns * 16; qd += 512) {
            const int row = qd >> 4, col = (qd & 15) * 8;
            *reinterpret_cast<u32x4*>(dst + (size_t)qd * 16) = *reinterpret_cast<const u32x4*>(&R[row * XS + col]);
        }
    } else {
        const int nq = ns * c * 3 / 16;
        for (int qd = tid; qd < nq; qd += 512)
            *reinterpret_cast<u32x4*>(dst + (size_t)qd * 16) = *reinterpret_cast<const u32x4*>(stg + (size_t)qd * 16);
    }
    if (tid == 0) x.seg_off[g] = pos;
}

hipError_t launch_cmp_append(const CmpArgs& a, const AppendArgs& x, int n_requests, hipStream_t s) {
    if (n_requests == 0) return hipSuccess;
    launch_kernel(k_cmp_append, dim3(n_requests * 2 * x.Hkv), dim3(512), 0, s, a, x);
    return hipGetLastError();
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
    uint64_t wg_bytes = 0;                                  // decide: payload bytes of this workgroup
    uint64_t wg_off = PACK ? a.wg_total[blockIdx.x] : 0;    // pack: offset of this workgroup's first segment

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
            const int best = vector_decide_f32(w, a, thr);
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
                wg_bytes += (uint64_t)ns * c * (4 + (c < MKV_D ? 1 : 0));
            }
        } else {
            const int code = a.codes[gs];
            const int c = a.keep[code];
            uint8_t* dst = a.payload + (a.preplaced ? a.seg_off[gs] : wg_off);
            if (!a.preplaced && tid == 0) a.seg_off[gs] = wg_off;
            wg_off += (uint64_t)ns * c * (4 + (c < MKV_D ? 1 : 0));
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
                    vector_pack_f32(w, tt, c, v, p, ns, stg);
                }
                __syncthreads();
                const int nq = ns * c * 5 / 16;
                for (int qd = tid; qd < nq; qd += 256)
                    __builtin_nontemporal_store(*reinterpret_cast<const u32x4*>(stg + (size_t)qd * 16), reinterpret_cast<u32x4*>(dst + (size_t)qd * 16));
            }
        }
        __syncthreads();
    }
    if (!PACK && tid == 0) a.wg_total[blockIdx.x] = wg_bytes;
}

constexpr size_t kF32Lds = (size_t)(2 * 64 * XF + MKV_D * MKV_D) * sizeof(float);

template <bool PACK>
static hipError_t launch_cmp(const CmpArgs& a, int dtype, hipStream_t s) {
    const dim3 grid(2 * a.nblk), block(256);
    if (a.nblk == 0) return hipSuccess;
    if (dtype == 1) {
        launch_kernel(k_cmp_bf16<PACK ? kCmpPack : kCmpDecide>, grid, dim3(512), 0, s, a);
    } else {
        static bool attr_set = false;
        if (!attr_set) {
            hipFuncSetAttribute((const void*)k_cmp_f32<PACK>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)kF32Lds);
            attr_set = true;
        }
        launch_kernel(k_cmp_f32<PACK>, grid, block, kF32Lds, s, a);
    }
    return hipGetLastError();
}

hipError_t launch_cmp_decide(const CmpArgs& a, int dtype, hipStream_t s) { return launch_cmp<false>(a, dtype, s); }
hipError_t launch_cmp_pack(const CmpArgs& a, int dtype, hipStream_t s) { return launch_cmp<true>(a, dtype, s); }
hipError_t launch_cmp_fused(const CmpArgs& a, hipStream_t s) {
    if (a.nblk == 0) return hipSuccess;
    launch_kernel(k_cmp_bf16<kCmpFused>, dim3(2 * a.nblk), dim3(512), 0, s, a);
    return hipGetLastError();
}

// =====================================================================================================
// exclusive scan of the workgroup payload totals (one workgroup, tiles of 1024)
// =====================================================================================================
__global__ __launch_bounds__(1024) void k_cmp_scan(uint64_t* a, int64_t n, uint64_t* total) {
    __shared__ uint64_t tmp[17];
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    uint64_t carry = 0;
    for (int64_t b0 = 0; b0 < n; b0 += 1024) {
        const int64_t i = b0 + threadIdx.x;
        const uint64_t v = i < n ? a[i] : 0;
        uint64_t x = v;
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
        if (i < n) a[i] = carry + tmp[wid] + x - v;
        carry += tmp[16];
        __syncthreads();
    }
    if (threadIdx.x == 0) *total = carry;
}

hipError_t launch_cmp_scan(uint64_t* wg_total, int64_t count, uint64_t* total, hipStream_t s) {
    launch_kernel(k_cmp_scan, dim3(1), dim3(1024), 0, s, wg_total, count, total);
    return hipGetLastError();
}

// =====================================================================================================
// paged pools: segment placement into fixed-size pages
// =====================================================================================================
// One wave per (request, KV head, tensor) stream of the requests being added.  The stream's segments go into
// its pages in segment order, each segment whole (it never straddles two pages, so the decode kernels' per-
// segment reads stay contiguous): a segment that does not fit in the rest of the current page opens the next
// page.  Until the host has picked the pages, seg_off holds (page ordinal << 32) | byte offset in the page.
// The walk runs over the segment sizes of 64 segments at a time, held one per lane and read back in order.
__global__ __launch_bounds__(64) void k_pool_place(PoolArgs p) {
    const int st = blockIdx.x;                       // (r * Hkv + h) * 2 + X
    const int X = st & 1, rh = st >> 1, r = rh / p.Hkv, h = rh - r * p.Hkv;
    const int n = p.tab[p.B + r];
    const int nseg = (n + MKV_SEG - 1) / MKV_SEG;
    const int64_t g0 = X * p.S + (int64_t)p.Hkv * p.tab[2 * p.B + r] + (int64_t)h * p.tab[3 * p.B + r];
    const int lane = threadIdx.x;
    int ord = -1;                                    // current page ordinal (-1: none yet)
    uint32_t cur = 0;                                // bytes used in the current page
    uint64_t used = 0;
    for (int s0 = 0; s0 < nseg; s0 += 64) {
        const int s = s0 + lane;
        uint32_t bytes = 0;
        if (s < nseg) {
            const int c = p.keep[p.codes[g0 + s]];
            const int ns = min(MKV_SEG, n - s * MKV_SEG);
            bytes = (uint32_t)(ns * c * (p.bv + (c < MKV_D ? 1 : 0)));
        }
        uint64_t mine = 0;
        const int m = min(64, nseg - s0);
        for (int j = 0; j < m; ++j) {
            const uint32_t b = (uint32_t)__builtin_amdgcn_readlane((int)bytes, j);
            if (ord < 0 || (uint64_t)cur + b > p.page_bytes) { ++ord; cur = 0; }
            if (lane == j) mine = ((uint64_t)ord << 32) | cur;
            cur += b;
            used += b;
        }
        if (s < nseg) p.seg_off[g0 + s] = mine;
    }
    if (lane == 0) {
        p.pages[st] = ord + 1;
        p.used[st] = used;
    }
}

// Replaces each placed segment's (page ordinal, offset) by its payload offset in the page the host assigned.
__global__ __launch_bounds__(256) void k_pool_fix(PoolArgs p) {
    const int st = blockIdx.x;
    const int X = st & 1, rh = st >> 1, r = rh / p.Hkv, h = rh - r * p.Hkv;
    const int n = p.tab[p.B + r];
    const int nseg = (n + MKV_SEG - 1) / MKV_SEG;
    const int64_t g0 = X * p.S + (int64_t)p.Hkv * p.tab[2 * p.B + r] + (int64_t)h * p.tab[3 * p.B + r];
    const int first = p.list_base[st];
    for (int s = threadIdx.x; s < nseg; s += 256) {
        const uint64_t v = p.seg_off[g0 + s];
        p.seg_off[g0 + s] = (uint64_t)p.page_ids[first + (int)(v >> 32)] * p.page_bytes + (uint32_t)v;
    }
}

hipError_t launch_pool_place(const PoolArgs& p, int n_streams, hipStream_t s) {
    if (n_streams == 0) return hipSuccess;
    launch_kernel(k_pool_place, dim3(n_streams), dim3(64), 0, s, p);
    return hipGetLastError();
}

hipError_t launch_pool_fix(const PoolArgs& p, int n_streams, hipStream_t s) {
    if (n_streams == 0) return hipSuccess;
    launch_kernel(k_pool_fix, dim3(n_streams), dim3(256), 0, s, p);
    return hipGetLastError();
}

}  // namespace mkv
