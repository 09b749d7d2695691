// Decode-step attention over the compressed store on gfx950 (arXiv 2607.00760, section 1: query-aware
// token selection at run time, kept together with channel compression through selection and attention;
// Observation & Approach 2: compact sparse attention on the packed cache, on the vector ALUs rather than the
// matrix cores, without unpacking it).
//
// Kernels, in stream order, for every (request r, KV head g):
//   prep     q'_h = q_h @ B_K (fp32), Qbar = sum of the group's q'_h; clears the selection state.
//   score    s_j = sum over token j's stored channels of Qbar_i * k_j,i for every stored key (8 lanes per token,
//            coalesced 16-byte loads, Qbar gathered from LDS); writes an order-preserving 32-bit key per token and
//            a 4096-bin histogram of the key's top 12 bits.  The last workgroup of a stream finds the bin that
//            holds the T-th largest key.
//   count    per 4096-key block: keys in that bin or above.
//   write    the same keys, compacted in ascending token order (block offsets from the counts).
//   final    one workgroup per stream resolves the exact T-th key inside the boundary bin (two more 10-bit radix
//            levels) and emits the selected tokens in ascending order; ties go to the lower token index.
//   attend   256 selected tokens per workgroup: exact logits of the group's query heads against the sparse keys,
//            online softmax, weighted sum of the sparse values; emits (max, sum, partial output) per head.
//   combine  log-sum-exp merge of the partials, then out_h = o'_h @ B_V^T.
#include "common.cuh"
#include "kernels.h"

namespace mkv {

// ---- byte loads of 2..64 bytes into 32-bit words -------------------------------------------------------
template <int NB>
__device__ __forceinline__ void ldb(uint32_t* d, const uint8_t* p) {
    if constexpr (NB >= 16) {
#pragma unroll
        for (int i = 0; i < NB / 16; ++i) {
            const u32x4 x = reinterpret_cast<const u32x4*>(p)[i];
            d[4 * i] = x.x; d[4 * i + 1] = x.y; d[4 * i + 2] = x.z; d[4 * i + 3] = x.w;
        }
    } else if constexpr (NB == 8) {
        const u32x2 x = *reinterpret_cast<const u32x2*>(p);
        d[0] = x.x; d[1] = x.y;
    } else if constexpr (NB == 4) {
        d[0] = *reinterpret_cast<const uint32_t*>(p);
    } else {
        d[0] = *reinterpret_cast<const uint16_t*>(p);
    }
}

template <int BV>
__device__ __forceinline__ float val_at(const uint32_t* vw, int k) {
    if constexpr (BV == 2) return (k & 1) ? __uint_as_float(vw[k >> 1] & 0xFFFF0000u) : __uint_as_float(vw[k >> 1] << 16);
    else return __uint_as_float(vw[k]);
}
__device__ __forceinline__ int idx_at(const uint32_t* iw, int k) { return (iw[k >> 2] >> (8 * (k & 3))) & 0xFF; }

// =====================================================================================================
// prep
// =====================================================================================================
__global__ __launch_bounds__(128) void k_dec_prep(DecArgs a, Upload tab) {
    if (blockIdx.x == 0)
        for (int i = threadIdx.x; i < tab.n; i += 128) tab.dst[i] = tab.w[i];
    __shared__ float qs[MKV_MAX_GROUP_DEV][MKV_D];
    const int stream = blockIdx.x, r = stream / a.Hkv, g = stream - r * a.Hkv;
    const int i = threadIdx.x, G = a.G, Hq = a.G * a.Hkv;
    for (int h = 0; h < G; ++h) {
        const size_t qi = ((size_t)r * Hq + g * G + h) * MKV_D + i;
        qs[h][i] = a.dtype == 1 ? bf16_to_f32(reinterpret_cast<const uint16_t*>(a.q)[qi])
                                : reinterpret_cast<const float*>(a.q)[qi];
    }
    __syncthreads();
    float acc[MKV_MAX_GROUP_DEV];
    const float* Bk = a.basis ? a.basis + ((((size_t)r * a.Hkv + g) * 2) << 14) : nullptr;
    for (int h = 0; h < MKV_MAX_GROUP_DEV; ++h) acc[h] = 0.f;
    if (Bk) {
        for (int k = 0; k < MKV_D; ++k) {
            const float b = Bk[k * MKV_D + i];
#pragma unroll
            for (int h = 0; h < MKV_MAX_GROUP_DEV; ++h)
                if (h < G) acc[h] = fmaf(qs[h][k], b, acc[h]);
        }
    } else {
        for (int h = 0; h < G; ++h) acc[h] = qs[h][i];
    }
    float qb = 0.f;
    for (int h = 0; h < MKV_MAX_GROUP_DEV; ++h) {
        if (h < G) {
            a.qp[((size_t)r * Hq + g * G + h) * MKV_D + i] = acc[h];
            qb += acc[h];
        }
    }
    a.qbar[(size_t)stream * MKV_D + i] = qb;
    for (int j = i; j < kHistBins; j += 128) a.hist[(size_t)stream * kHistBins + j] = 0u;
    if (i < kStateWords) a.state[stream * kStateWords + i] = 0u;
}

hipError_t launch_dec_prep(const DecArgs& a, const Upload& tab, hipStream_t s) {
    hipLaunchKernelGGL(k_dec_prep, dim3(a.B * a.Hkv), dim3(128), 0, s, a, tab);
    return hipGetLastError();
}

// =====================================================================================================
// score
// =====================================================================================================
// One 64-token segment of stream keys with C kept channels: 8 lanes per token, 8 tokens per pass.  Lane
// (t8, sl) returns the score of token 8*sl + t8.
template <int BV, int C>
__device__ __forceinline__ float score_segment(const uint8_t* seg, int ns, const float* sq, int t8, int sl) {
    constexpr int VPL = C / 8;                 // values per lane
    constexpr int VB = VPL * BV;               // value bytes per lane
    constexpr int VW = (VB + 3) / 4;
    constexpr int IW = C < MKV_D ? (VPL + 3) / 4 : 1;
    const uint8_t* vbase = seg + sl * VB;
    const uint8_t* ibase = seg + (size_t)ns * C * BV + sl * VPL;
    float mine = 0.f;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
        uint32_t vw[4][VW], iw[4][IW];
#pragma unroll
        for (int pp = 0; pp < 4; ++pp) {
            const int tk = (half * 4 + pp) * 8 + t8;
            if (tk < ns) {
                ldb<VB>(vw[pp], vbase + (size_t)tk * C * BV);
                if constexpr (C < MKV_D) ldb<VPL>(iw[pp], ibase + (size_t)tk * C);
            } else {
#pragma unroll
                for (int x = 0; x < VW; ++x) vw[pp][x] = 0u;
#pragma unroll
                for (int x = 0; x < IW; ++x) iw[pp][x] = 0u;
            }
        }
#pragma unroll
        for (int pp = 0; pp < 4; ++pp) {
            float acc = 0.f;
#pragma unroll
            for (int k = 0; k < VPL; ++k) {
                const int ch = (C == MKV_D) ? sl * VPL + k : idx_at(iw[pp], k);
                acc = fmaf(sq[ch], val_at<BV>(vw[pp], k), acc);
            }
            acc = sum8(acc);
            if (sl == half * 4 + pp) mine = acc;
        }
    }
    return mine;
}

template <int BV>
__global__ __launch_bounds__(256) void k_score(DecArgs a) {
    __shared__ float sq[MKV_D];
    __shared__ uint32_t sh[kHistBins];
    __shared__ uint32_t tmp[8];
    __shared__ int s_last;
    const int b = blockIdx.x;
    const int r = find_slot(a.t_sblk, a.B, b);
    const int n = a.t_n[r], Sr = (n + MKV_SEG - 1) / MKV_SEG, nch = (Sr + a.spw - 1) / a.spw;
    const int local = b - a.t_sblk[r];
    const int g = local / nch, chunk = local - g * nch;
    const int stream = r * a.Hkv + g;
    const int64_t seg0 = (int64_t)a.Hkv * a.t_segbase[r] + (int64_t)g * Sr;
    const int64_t keybase = (int64_t)a.t_tokbase[r] * a.Hkv + (int64_t)g * n;
    const int tid = threadIdx.x;
    for (int i = tid; i < kHistBins; i += 256) sh[i] = 0u;
    if (tid < MKV_D) sq[tid] = a.qbar[(size_t)stream * MKV_D + tid];
    __syncthreads();

    const int wid = tid >> 6, lane = tid & 63, t8 = lane >> 3, sl = lane & 7;
    const int s0 = chunk * a.spw, s1 = min(Sr, s0 + a.spw);
    for (int s = s0 + wid; s < s1; s += 4) {
        const int64_t gs = seg0 + s;
        const int c = a.keep[a.codes[gs]];
        const uint8_t* seg = a.payload + a.seg_off[gs];
        const int ns = min(MKV_SEG, n - s * MKV_SEG);
        float sc;
        switch (c) {
            case 128: sc = score_segment<BV, 128>(seg, ns, sq, t8, sl); break;
            case 64: sc = score_segment<BV, 64>(seg, ns, sq, t8, sl); break;
            case 32: sc = score_segment<BV, 32>(seg, ns, sq, t8, sl); break;
            default: sc = score_segment<BV, 16>(seg, ns, sq, t8, sl); break;
        }
        const int tok = sl * 8 + t8;
        if (tok < ns) {
            const uint32_t key = score_key(sc);
            a.keys[keybase + (int64_t)s * MKV_SEG + tok] = key;
            atomicAdd(&sh[key >> 20], 1u);
        }
    }
    __syncthreads();
    uint32_t* gh = a.hist + (size_t)stream * kHistBins;
    for (int i = tid; i < kHistBins; i += 256) {
        const uint32_t v = sh[i];
        if (v) atomic_add_dev(&gh[i], v);
    }
    __threadfence();
    __syncthreads();
    if (tid == 0) {
        const uint32_t old = atomic_add_acqrel_dev(&a.state[stream * kStateWords + ST_DONE], 1u);
        s_last = (old == (uint32_t)(nch - 1));
    }
    __syncthreads();
    if (!s_last) return;
    __threadfence();

    // Last workgroup of the stream: the bin of the T-th largest key.  Thread t owns bins
    // [4095 - 16t - 15, 4095 - 16t], scanned from the top.
    const uint32_t T = (uint32_t)a.t_T[r];
    uint32_t cnt[16], loc = 0;
#pragma unroll
    for (int k = 0; k < 16; ++k) { cnt[k] = load_dev(&gh[kHistBins - 1 - (16 * tid + k)]); loc += cnt[k]; }
    uint32_t total;
    const uint32_t above = block_exscan(loc, tmp, &total);
    if (above < T && above + loc >= T) {
        uint32_t run = above;
#pragma unroll
        for (int k = 0; k < 16; ++k) {
            if (run + cnt[k] >= T) {
                uint32_t* st = a.state + stream * kStateWords;
                st[ST_P1] = (uint32_t)(kHistBins - 1 - (16 * tid + k));
                st[ST_NGT] = run;
                st[ST_NCAND] = cnt[k];
                st[ST_NEED] = T - run;
                break;
            }
            run += cnt[k];
        }
    }
}

hipError_t launch_score(const DecArgs& a, int n_blocks, hipStream_t s) {
    if (n_blocks == 0) return hipSuccess;
    if (a.dtype == 1) hipLaunchKernelGGL(k_score<2>, dim3(n_blocks), dim3(256), 0, s, a);
    else hipLaunchKernelGGL(k_score<4>, dim3(n_blocks), dim3(256), 0, s, a);
    return hipGetLastError();
}

// =====================================================================================================
// selection passes
// =====================================================================================================
struct KBlock { int r, g, kb, n, stream, first_blk; int64_t keybase; };

__device__ __forceinline__ KBlock kblock(const DecArgs& a) {
    KBlock k;
    const int b = blockIdx.x;
    k.r = find_slot(a.t_kblk, a.B, b);
    k.n = a.t_n[k.r];
    const int nkb = (k.n + kKeysPerBlock - 1) / kKeysPerBlock;
    const int local = b - a.t_kblk[k.r];
    k.g = local / nkb;
    k.kb = local - k.g * nkb;
    k.stream = k.r * a.Hkv + k.g;
    k.first_blk = b - k.kb;
    k.keybase = (int64_t)a.t_tokbase[k.r] * a.Hkv + (int64_t)k.g * k.n;
    return k;
}

__global__ __launch_bounds__(256) void k_sel_count(DecArgs a) {
    __shared__ uint32_t tmp[8];
    const KBlock k = kblock(a);
    const uint32_t p1 = a.state[k.stream * kStateWords + ST_P1];
    const int lo = k.kb * kKeysPerBlock, cnt = min(kKeysPerBlock, k.n - lo);
    const uint32_t* keys = a.keys + k.keybase + lo;
    uint32_t c = 0;
    for (int i = threadIdx.x; i < cnt; i += 256) c += ((keys[i] >> 20) >= p1) ? 1u : 0u;
    uint32_t total;
    block_exscan(c, tmp, &total);
    if (threadIdx.x == 0) a.bcnt[blockIdx.x] = total;
}

__global__ __launch_bounds__(256) void k_sel_write(DecArgs a) {
    __shared__ uint32_t tmp[8];
    __shared__ uint32_t sk[kKeysPerBlock];
    const KBlock k = kblock(a);
    const uint32_t p1 = a.state[k.stream * kStateWords + ST_P1];
    const int lo = k.kb * kKeysPerBlock, cnt = min(kKeysPerBlock, k.n - lo);
    const int tid = threadIdx.x;
    // offset of this block: entries of the earlier blocks of the stream
    uint32_t pre = 0;
    for (int i = tid; i < k.kb; i += 256) pre += a.bcnt[k.first_blk + i];
    uint32_t base;
    block_exscan(pre, tmp, &base);
    const uint32_t* keys = a.keys + k.keybase + lo;
    for (int i = tid; i < cnt; i += 256) sk[i] = keys[i];
    __syncthreads();
    uint32_t f = 0;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        const int i = tid * 16 + j;
        if (i < cnt && (sk[i] >> 20) >= p1) f |= 1u << j;
    }
    uint32_t total;
    uint32_t pos = base + block_exscan(__popc(f), tmp, &total);
    uint2* L = a.L + k.keybase;
    for (int j = 0; j < 16; ++j) {
        if ((f >> j) & 1u) {
            const int i = tid * 16 + j;
            L[pos++] = make_uint2((uint32_t)(lo + i), sk[i]);
        }
    }
}

hipError_t launch_sel_count(const DecArgs& a, int n_blocks, hipStream_t s) {
    if (n_blocks == 0) return hipSuccess;
    hipLaunchKernelGGL(k_sel_count, dim3(n_blocks), dim3(256), 0, s, a);
    return hipGetLastError();
}
hipError_t launch_sel_write(const DecArgs& a, int n_blocks, hipStream_t s) {
    if (n_blocks == 0) return hipSuccess;
    hipLaunchKernelGGL(k_sel_write, dim3(n_blocks), dim3(256), 0, s, a);
    return hipGetLastError();
}

// Largest bin b (of h[0..1023], one per thread) with (sum of bins >= b) >= need; returns b and the count
// still needed inside it through res[0], res[1].
__device__ __forceinline__ void find_bin1024(const uint32_t* h, uint32_t need, uint32_t* tmp, uint32_t* res) {
    const int tid = threadIdx.x;
    const uint32_t v = h[1023 - tid];
    uint32_t tot;
    const uint32_t above = block_exscan(v, tmp, &tot);
    if (above < need && above + v >= need) { res[0] = (uint32_t)(1023 - tid); res[1] = need - above; }
    __syncthreads();
}

__global__ __launch_bounds__(1024) void k_sel_final(DecArgs a) {
    __shared__ uint32_t h[1024];
    __shared__ uint32_t tmp[20];
    __shared__ uint32_t res[2];
    const int stream = blockIdx.x, r = stream / a.Hkv, g = stream - r * a.Hkv;
    const int n = a.t_n[r], T = a.t_T[r];
    const int tid = threadIdx.x;
    int32_t* urow = a.sel ? a.sel + (size_t)stream * a.sel_stride : nullptr;
    if (n > 0 && T > 0) {
        const uint32_t* st = a.state + stream * kStateWords;
        const uint32_t p1 = st[ST_P1], ngt = st[ST_NGT], ncand = st[ST_NCAND], need = st[ST_NEED];
        const uint32_t m = ngt + ncand;
        const int64_t keybase = (int64_t)a.t_tokbase[r] * a.Hkv + (int64_t)g * n;
        const uint2* L = a.L + keybase;
        const bool all = (need == ncand);
        uint32_t kstar = 0, need_eq = 0;
        if (!all) {
            h[tid] = 0u;
            __syncthreads();
            for (uint32_t i = tid; i < m; i += 1024) {
                const uint32_t key = L[i].y;
                if ((key >> 20) == p1) atomicAdd(&h[(key >> 10) & 1023u], 1u);
            }
            __syncthreads();
            find_bin1024(h, need, tmp, res);
            const uint32_t b2 = res[0], need2 = res[1];
            const uint32_t pre22 = (p1 << 10) | b2;
            h[tid] = 0u;
            __syncthreads();
            for (uint32_t i = tid; i < m; i += 1024) {
                const uint32_t key = L[i].y;
                if ((key >> 10) == pre22) atomicAdd(&h[key & 1023u], 1u);
            }
            __syncthreads();
            find_bin1024(h, need2, tmp, res);
            kstar = (pre22 << 10) | res[0];
            need_eq = res[1];
        }
        int32_t* srow = a.sel_int + (size_t)stream * a.sel_int_stride;
        uint32_t run_keep = 0, run_eq = 0;
        for (uint32_t b0 = 0; b0 < m; b0 += 1024) {
            const uint32_t i = b0 + tid;
            const bool valid = i < m;
            const uint2 e = valid ? L[i] : make_uint2(0u, 0u);
            const bool is_gt = valid && (all || e.y > kstar);
            const bool is_eq = valid && !all && e.y == kstar;
            uint32_t eqt, kt;
            const uint32_t eqx = block_exscan(is_eq ? 1u : 0u, tmp, &eqt);
            const bool keep = is_gt || (is_eq && run_eq + eqx < need_eq);
            const uint32_t kx = block_exscan(keep ? 1u : 0u, tmp, &kt);
            if (keep) {
                srow[run_keep + kx] = (int32_t)e.x;
                if (urow) urow[run_keep + kx] = (int32_t)e.x;
            }
            run_eq += eqt;
            run_keep += kt;
        }
    }
    if (urow) {
        const int start = (n > 0) ? min(T, n) : 0;
        for (int j = start + tid; j < a.sel_stride; j += 1024) urow[j] = -1;
    }
}

hipError_t launch_sel_final(const DecArgs& a, hipStream_t s) {
    hipLaunchKernelGGL(k_sel_final, dim3(a.B * a.Hkv), dim3(1024), 0, s, a);
    return hipGetLastError();
}

// =====================================================================================================
// sparse exact attention over the selected tokens
// =====================================================================================================
// Partial logits of the G query heads against this lane's slots of a key row with C kept channels.
template <int BV, int C, int G>
__device__ __forceinline__ void key_row(const uint8_t* seg, int ns, int tt, int sl, const float* qt, float* lg) {
    constexpr int VPL = C / 8, VB = VPL * BV, VW = (VB + 3) / 4, IW = C < MKV_D ? (VPL + 3) / 4 : 1;
    uint32_t vw[VW], iw[IW];
    ldb<VB>(vw, seg + (size_t)tt * C * BV + sl * VB);
    if constexpr (C < MKV_D) ldb<VPL>(iw, seg + (size_t)ns * C * BV + (size_t)tt * C + sl * VPL);
#pragma unroll
    for (int k = 0; k < VPL; ++k) {
        const int ch = (C == MKV_D) ? sl * VPL + k : idx_at(iw, k);
        const float v = val_at<BV>(vw, k);
#pragma unroll
        for (int h = 0; h < G; ++h) lg[h] = fmaf(qt[ch * G + h], v, lg[h]);
    }
}

// Scatter this lane's slots of a value row into a dense 128-float row.
template <int BV, int C>
__device__ __forceinline__ void value_row(const uint8_t* seg, int ns, int tt, int sl, float* dense) {
    constexpr int VPL = C / 8, VB = VPL * BV, VW = (VB + 3) / 4, IW = C < MKV_D ? (VPL + 3) / 4 : 1;
    uint32_t vw[VW], iw[IW];
    ldb<VB>(vw, seg + (size_t)tt * C * BV + sl * VB);
    if constexpr (C < MKV_D) ldb<VPL>(iw, seg + (size_t)ns * C * BV + (size_t)tt * C + sl * VPL);
#pragma unroll
    for (int k = 0; k < VPL; ++k) {
        const int ch = (C == MKV_D) ? sl * VPL + k : idx_at(iw, k);
        dense[ch] = val_at<BV>(vw, k);
    }
}

template <int BV, int G>
__global__ __launch_bounds__(256) void k_attend(DecArgs a) {
    __shared__ __attribute__((aligned(16))) float qt[MKV_D * G];
    __shared__ __attribute__((aligned(16))) float vb[4][8][MKV_D];
    __shared__ float pt[4][8][G];
    __shared__ float wm[4][G], wl[4][G];
    __shared__ float wacc[4][G][MKV_D];
    const int b = blockIdx.x;
    const int r = find_slot(a.t_ablk, a.B, b);
    const int n = a.t_n[r], T = a.t_T[r], Sr = (n + MKV_SEG - 1) / MKV_SEG;
    const int nach = (T + kAttnChunk - 1) / kAttnChunk;
    const int local = b - a.t_ablk[r];
    const int g = local / nach, chunk = local - g * nach;
    const int stream = r * a.Hkv + g, Hq = a.G * a.Hkv;
    const int tid = threadIdx.x, wid = tid >> 6, lane = tid & 63, t8 = lane >> 3, sl = lane & 7;
    for (int i = tid; i < MKV_D * G; i += 256) {
        const int h = i >> 7, ch = i & 127;
        qt[ch * G + h] = a.qp[((size_t)r * Hq + g * G + h) * MKV_D + ch];
    }
    __syncthreads();
    const int32_t* list = a.sel_int + (size_t)stream * a.sel_int_stride;
    const int64_t segK = (int64_t)a.Hkv * a.t_segbase[r] + (int64_t)g * Sr;
    const int64_t segV = a.S + segK;
    const float scale = 1.4426950408889634f * 0.08838834764831845f;   // log2(e) / sqrt(128)
    float m[G], l[G], acc[G][2];
#pragma unroll
    for (int h = 0; h < G; ++h) { m[h] = -INFINITY; l[h] = 0.f; acc[h][0] = 0.f; acc[h][1] = 0.f; }

    for (int pass = 0; pass < 8; ++pass) {
        const int li = chunk * kAttnChunk + wid * 64 + pass * 8 + t8;
        const int j = (li < T) ? list[li] : -1;
        float lg[G];
#pragma unroll
        for (int h = 0; h < G; ++h) lg[h] = 0.f;
        int s = 0, tt = 0, ns = 0;
        if (j >= 0) {
            s = j >> 6; tt = j & 63; ns = min(MKV_SEG, n - s * MKV_SEG);
            const int64_t gs = segK + s;
            const int c = a.keep[a.codes[gs]];
            const uint8_t* seg = a.payload + a.seg_off[gs];
            switch (c) {
                case 128: key_row<BV, 128, G>(seg, ns, tt, sl, qt, lg); break;
                case 64: key_row<BV, 64, G>(seg, ns, tt, sl, qt, lg); break;
                case 32: key_row<BV, 32, G>(seg, ns, tt, sl, qt, lg); break;
                default: key_row<BV, 16, G>(seg, ns, tt, sl, qt, lg); break;
            }
        }
        float sc[G], p[G];
#pragma unroll
        for (int h = 0; h < G; ++h) {
            lg[h] = sum8(lg[h]);
            lg[h] = (j >= 0) ? lg[h] * scale : -INFINITY;
            float pm = lg[h];
            pm = fmaxf(pm, __shfl_xor(pm, 8, MKV_WAVE));
            pm = fmaxf(pm, __shfl_xor(pm, 16, MKV_WAVE));
            pm = fmaxf(pm, __shfl_xor(pm, 32, MKV_WAVE));
            const float nm = fmaxf(m[h], pm);
            if (nm == -INFINITY) { sc[h] = 1.f; p[h] = 0.f; }
            else { sc[h] = exp2f(m[h] - nm); p[h] = exp2f(lg[h] - nm); }
            m[h] = nm;
        }
        float* dense = vb[wid][t8];
        *reinterpret_cast<f32x4*>(&dense[sl * 16 + 0]) = f32x4{0.f, 0.f, 0.f, 0.f};
        *reinterpret_cast<f32x4*>(&dense[sl * 16 + 4]) = f32x4{0.f, 0.f, 0.f, 0.f};
        *reinterpret_cast<f32x4*>(&dense[sl * 16 + 8]) = f32x4{0.f, 0.f, 0.f, 0.f};
        *reinterpret_cast<f32x4*>(&dense[sl * 16 + 12]) = f32x4{0.f, 0.f, 0.f, 0.f};
        wave_lds_sync();
        if (j >= 0) {
            const int64_t gs = segV + s;
            const int c = a.keep[a.codes[gs]];
            const uint8_t* seg = a.payload + a.seg_off[gs];
            switch (c) {
                case 128: value_row<BV, 128>(seg, ns, tt, sl, dense); break;
                case 64: value_row<BV, 64>(seg, ns, tt, sl, dense); break;
                case 32: value_row<BV, 32>(seg, ns, tt, sl, dense); break;
                default: value_row<BV, 16>(seg, ns, tt, sl, dense); break;
            }
        }
        if (sl == 0) {
#pragma unroll
            for (int h = 0; h < G; ++h) pt[wid][t8][h] = p[h];
        }
        wave_lds_sync();
#pragma unroll
        for (int h = 0; h < G; ++h) {
            float ps = 0.f;
#pragma unroll
            for (int t = 0; t < 8; ++t) ps += pt[wid][t][h];
            l[h] = l[h] * sc[h] + ps;
            acc[h][0] *= sc[h];
            acc[h][1] *= sc[h];
        }
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            const float2 v = *reinterpret_cast<const float2*>(&vb[wid][t][2 * lane]);
#pragma unroll
            for (int h = 0; h < G; ++h) {
                const float pp = pt[wid][t][h];
                acc[h][0] = fmaf(pp, v.x, acc[h][0]);
                acc[h][1] = fmaf(pp, v.y, acc[h][1]);
            }
        }
        wave_lds_sync();
    }
    if (lane == 0) {
#pragma unroll
        for (int h = 0; h < G; ++h) { wm[wid][h] = m[h]; wl[wid][h] = l[h]; }
    }
#pragma unroll
    for (int h = 0; h < G; ++h) { wacc[wid][h][2 * lane] = acc[h][0]; wacc[wid][h][2 * lane + 1] = acc[h][1]; }
    __syncthreads();
    for (int i = tid; i < G * MKV_D; i += 256) {
        const int h = i >> 7, ch = i & 127;
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < 4; ++w) M = fmaxf(M, wm[w][h]);
        float O = 0.f, Ls = 0.f;
        if (M != -INFINITY) {
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                if (wm[w][h] != -INFINITY) {
                    const float f = exp2f(wm[w][h] - M);
                    O = fmaf(wacc[w][h][ch], f, O);
                    Ls = fmaf(wl[w][h], f, Ls);
                }
            }
        }
        float* dst = a.part + ((size_t)b * G + h) * (MKV_D + 2);
        if (ch == 0) { dst[0] = M; dst[1] = Ls; }
        dst[2 + ch] = O;
    }
}

template <int G>
__global__ __launch_bounds__(256) void k_combine(DecArgs a) {
    __shared__ float o[G][MKV_D];
    __shared__ float bsh[MKV_D * (MKV_D + 1)];
    const int stream = blockIdx.x, r = stream / a.Hkv, g = stream - r * a.Hkv;
    const int n = a.t_n[r], T = (n > 0) ? a.t_T[r] : 0;
    const int nach = (T + kAttnChunk - 1) / kAttnChunk;
    const int first = a.t_ablk[r] + g * nach;
    const int tid = threadIdx.x, Hq = a.G * a.Hkv;
    for (int i = tid; i < G * MKV_D; i += 256) {
        const int h = i >> 7, ch = i & 127;
        float M = -INFINITY;
        for (int c = 0; c < nach; ++c) M = fmaxf(M, a.part[((size_t)(first + c) * G + h) * (MKV_D + 2)]);
        float O = 0.f, Ls = 0.f;
        if (M != -INFINITY) {
            for (int c = 0; c < nach; ++c) {
                const float* pp = a.part + ((size_t)(first + c) * G + h) * (MKV_D + 2);
                if (pp[0] != -INFINITY) {
                    const float f = exp2f(pp[0] - M);
                    O = fmaf(pp[2 + ch], f, O);
                    Ls = fmaf(pp[1], f, Ls);
                }
            }
        }
        o[h][ch] = (Ls > 0.f) ? O / Ls : 0.f;
    }
    const float* Bv = a.basis ? a.basis + ((((size_t)r * a.Hkv + g) * 2 + 1) << 14) : nullptr;
    if (Bv)
        for (int i = tid; i < MKV_D * MKV_D; i += 256) bsh[(i >> 7) * (MKV_D + 1) + (i & 127)] = Bv[i];
    __syncthreads();
    for (int i = tid; i < G * MKV_D; i += 256) {
        const int h = i >> 7, row = i & 127;
        float v;
        if (Bv) {
            v = 0.f;
            for (int k = 0; k < MKV_D; ++k) v = fmaf(o[h][k], bsh[row * (MKV_D + 1) + k], v);
        } else {
            v = o[h][row];
        }
        a.out[((size_t)r * Hq + g * G + h) * MKV_D + row] = v;
    }
}

template <int BV>
static void launch_attend_g(const DecArgs& a, int n_blocks, hipStream_t s) {
    switch (a.G) {
        case 1: hipLaunchKernelGGL((k_attend<BV, 1>), dim3(n_blocks), dim3(256), 0, s, a); break;
        case 2: hipLaunchKernelGGL((k_attend<BV, 2>), dim3(n_blocks), dim3(256), 0, s, a); break;
        case 4: hipLaunchKernelGGL((k_attend<BV, 4>), dim3(n_blocks), dim3(256), 0, s, a); break;
        default: hipLaunchKernelGGL((k_attend<BV, 8>), dim3(n_blocks), dim3(256), 0, s, a); break;
    }
}

hipError_t launch_attend(const DecArgs& a, int n_blocks, hipStream_t s) {
    if (n_blocks == 0) return hipSuccess;
    if (a.dtype == 1) launch_attend_g<2>(a, n_blocks, s);
    else launch_attend_g<4>(a, n_blocks, s);
    return hipGetLastError();
}

hipError_t launch_combine(const DecArgs& a, hipStream_t s) {
    const dim3 grid(a.B * a.Hkv), block(256);
    switch (a.G) {
        case 1: hipLaunchKernelGGL(k_combine<1>, grid, block, 0, s, a); break;
        case 2: hipLaunchKernelGGL(k_combine<2>, grid, block, 0, s, a); break;
        case 4: hipLaunchKernelGGL(k_combine<4>, grid, block, 0, s, a); break;
        default: hipLaunchKernelGGL(k_combine<8>, grid, block, 0, s, a); break;
    }
    return hipGetLastError();
}

}  // namespace mkv
