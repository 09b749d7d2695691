// Decode-step attention over the compressed store on gfx950 (arXiv 2607.00760, section 1: query-aware
// token selection at run time, kept together with channel compression through selection and attention;
// Observation & Approach 2: compact sparse attention on the packed cache, on the vector ALUs rather than the
// matrix cores, without unpacking it).
//
// Kernels, in stream order, for every (request r, KV head g):
//   prep     q'_h = q_h @ B_K (fp32), Qbar = sum of the group's q'_h; clears the selection state.
//   score    s_j = sum over token j's stored channels of Qbar_i * k_j,i for every stored key (c/8 lanes per
//            token, one coalesced 16-byte value load per lane and pass, eight passes in flight per wave, Qbar
//            gathered from LDS); writes an order-preserving 32-bit key per token and a 4096-bin histogram of the
//            key's top 12 bits.
//   collect  finds the histogram bin that holds the T-th largest key (coarse then fine histogram), and appends the
//            tokens above it and the candidates inside it to two per-stream lists.
//   emit     one workgroup per stream resolves the exact T-th key among the candidates (two more 10-bit radix
//            levels) and writes the selected tokens in ascending order through an LDS bitmap; ties go to the
//            lower token index.
//   attend   256, 128 or 64 selected tokens per workgroup (a quarter per wave; fewer when the selection is small):
//            exact logits of the group's query heads against the sparse keys, a softmax per wave and head,
//            weighted sum of the sparse values; emits (max, sum, partial output) per head.
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

// Keys and selection lists of stream (r, g) start at a 64-token aligned offset: requests are padded to a
// multiple of 64 tokens, so 16-byte vector loads of keys stay aligned.
__device__ __forceinline__ int64_t key_base(const DecArgs& a, int r, int g, int n) {
    return (int64_t)a.t_tokbase[r] * a.Hkv + (int64_t)g * ((n + 63) & ~63);
}

// =====================================================================================================
// prep
// =====================================================================================================
// Four workgroups per stream, one per quarter of the 128 output channels: q' = q @ B_K and Qbar for 32
// columns, a quarter of the stream's histogram cleared; the first workgroup also clears the selection state,
// and workgroup 0 of the grid writes the uploaded table words.
__global__ __launch_bounds__(256) void k_dec_prep(DecArgs a, Upload tab) {
    constexpr int QC = MKV_D / 4;                    // output columns per workgroup
    __shared__ __attribute__((aligned(16))) float bs[MKV_D][QC];
    __shared__ float qs[MKV_MAX_GROUP_DEV][MKV_D];
    __shared__ float qo[MKV_MAX_GROUP_DEV][QC];
    const int tid = threadIdx.x;
    if (blockIdx.x == 0)
        for (int i = tid; i < tab.n; i += 256) tab.dst[i] = tab.w[i];
    const int stream = blockIdx.x >> 2, qd = blockIdx.x & 3, r = stream / a.Hkv, g = stream - r * a.Hkv;
    const int G = a.G, Hq = a.G * a.Hkv;
    // the basis slot comes from the table words this launch carries when they include it (workgroup 0 writes
    // those words to memory during this kernel), else from memory, written by an earlier upload
    const int bi = (int)(a.t_bslot - tab.dst) + r;
    const int bslot = bi < tab.n ? tab.w[bi] : a.t_bslot[r];
    const float* Bk = a.basis ? a.basis + ((((size_t)bslot * a.Hkv + g) * 2) << 14) : nullptr;
    f32x4 v[4];
    if (Bk) {   // rows 0..127, columns [32 qd, 32 qd + 32): 1024 16-byte pieces, 4 per thread
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int idx = tid + 256 * j, row = idx >> 3, c4 = idx & 7;
            v[j] = *reinterpret_cast<const f32x4*>(Bk + row * MKV_D + QC * qd + 4 * c4);
        }
    }
    for (int i = tid; i < G * MKV_D; i += 256) {
        const int h = i >> 7, c = i & 127;
        const size_t qi = ((size_t)r * Hq + g * G + h) * MKV_D + c;
        qs[h][c] = a.dtype == 1 ? bf16_to_f32(reinterpret_cast<const uint16_t*>(a.q)[qi])
                                : reinterpret_cast<const float*>(a.q)[qi];
    }
    {   // a quarter of every histogram copy of the stream
        u32x4* hq = reinterpret_cast<u32x4*>(a.hist + (size_t)stream * a.hcopies * kHistBins);
        for (int j = tid; j < a.hcopies * (kHistBins / 16); j += 256) {
            const int c = j / (kHistBins / 16), i = j - c * (kHistBins / 16);
            hq[c * (kHistBins / 4) + qd * (kHistBins / 16) + i] = u32x4{0u, 0u, 0u, 0u};
        }
    }
    if (qd == 0)
        for (int i = tid; i < kCoarseOff + 64 * a.hcopies; i += 256) a.state[stream * kStateWords + i] = 0u;
    if (Bk) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int idx = tid + 256 * j, row = idx >> 3, c4 = idx & 7;
            *reinterpret_cast<f32x4*>(&bs[row][4 * c4]) = v[j];
        }
    }
    __syncthreads();
    for (int o = tid; o < G * QC; o += 256) {
        const int h = o / QC, col = o - h * QC;
        float acc;
        if (Bk) {
            acc = 0.f;
#pragma unroll 8
            for (int k = 0; k < MKV_D; ++k) acc = fmaf(qs[h][k], bs[k][col], acc);
        } else {
            acc = qs[h][QC * qd + col];
        }
        qo[h][col] = acc;
        a.qp[((size_t)r * Hq + g * G + h) * MKV_D + QC * qd + col] = acc;
    }
    __syncthreads();
    if (tid < QC) {
        float qb = 0.f;
        for (int h = 0; h < G; ++h) qb += qo[h][tid];
        a.qbar[(size_t)stream * MKV_D + QC * qd + tid] = qb;
    }
}

hipError_t launch_dec_prep(const DecArgs& a, const Upload& tab, hipStream_t s) {
    launch_kernel(k_dec_prep, dim3(4 * a.B * a.Hkv), dim3(256), 0, s, a, tab);
    return hipGetLastError();
}

// =====================================================================================================
// score
// =====================================================================================================
// Work split: the segments of one stream are dealt out to its workgroups in an interleaved order, so that the
// workgroups of a stream (which are dispatched together) sweep its payload front to back side by side rather
// than each streaming a distant chunk of its own.  With g workgroups for a stream of S segments, local slot k
// (k = 4*kk + w; wave w takes slots w, w+4, ...) of workgroup i holds segment 4*i + w + 4*g*kk.
//
// A wave reads its segments as a flat sequence of passes.  In every pass each lane loads one 16-byte chunk of
// stored values (8 bf16 or 4 fp32: VPL slots) and the matching VPL one-byte channel indices, so a token with c
// kept channels spans LPT = c / VPL consecutive lanes and a pass covers TPP = 64 / LPT tokens; the load shape is
// the same for every kept count.  A wave keeps kRing passes in flight (their loads issued before the oldest one
// is consumed).
constexpr int kRing = 8;
constexpr int kMaxSpw = 16;
constexpr uint32_t kOutOfRange = 0x80000000u;   // buffer offset past every segment: loads return 0
// Cache policy of the payload loads: non-temporal (the nt bit), since every byte is read once.  The stream then
// does not displace the lines the kernel writes (keys, histograms) or the step's small tables from the caches:
// measured at 8 x 131072 tokens, the kernel takes 263 us with it against 291 us without.
constexpr int kStreamLoad = 2;

__device__ __forceinline__ int uni(int x) { return __builtin_amdgcn_readfirstlane(x); }

// stream segment held by local slot k of workgroup i (stride = 4 * workgroups of the stream)
__device__ __forceinline__ int slot_segment(int i, int k, int stride) { return 4 * i + (k & 3) + stride * (k >> 2); }

struct PassMeta {
    int lc;      // log2 of the kept channels of the pass's segment
    int tbase;   // workgroup-local index (slot * 64 + token) of the pass's first token
    int tlim;    // workgroup-local end of the segment's tokens (-1: no pass)
};

// Walks a wave's segments (every fourth local slot) pass by pass.  All fields are wave-uniform and every count
// is a power of two, so lanes-per-token and tokens-per-pass are shifts.  Each segment gets a buffer resource of
// its own, sized to the segment, so that lanes past its last token read zeros.
template <int BV>
struct PassIter {
    static constexpr int LVPL = BV == 2 ? 3 : 2;    // log2 of values per lane per pass (16 bytes)
    const uint8_t* payload;
    const uint64_t* s_off;   // LDS: payload offset of each local slot's segment
    const int* s_m;          // LDS: log2(kept channels) | tokens << 8
    int k, kend, p, P, lc, ns;
    __amdgpu_buffer_rsrc_t rs;

    __device__ __forceinline__ void load_seg() {
        const int kk = min(k, kend - 1);
        const int w = uni(s_m[kk]);
        const uint64_t off = s_off[kk];
        const uint32_t lo = (uint32_t)uni((int)(uint32_t)off), hi = (uint32_t)uni((int)(uint32_t)(off >> 32));
        lc = w & 0xFF;
        ns = w >> 8;
        const int bytes = (ns << lc) * (BV + (lc < 7 ? 1 : 0));
        rs = __builtin_amdgcn_make_buffer_rsrc((void*)(payload + (((uint64_t)hi << 32) | lo)), (short)0, bytes,
                                               0x00020000);
        const int ltpp = 6 + LVPL - lc;              // log2 tokens per pass
        P = uni((ns + (1 << ltpp) - 1) >> ltpp);
    }
    __device__ __forceinline__ void next() {
        p = uni(p + 1);
        if (p == P) { p = 0; k = uni(k + 4); if (k < kend) load_seg(); }
    }
};

// Issues the buffer loads of the iterator's current pass (or, past the wave's last pass, loads that the range
// check turns into zeros without a memory access).  Lanes past the segment's last token get zeros the same way.
template <int BV>
__device__ __forceinline__ void issue_pass(PassIter<BV>& it, int lane, u32x4& v, u32x2& ix, PassMeta& m) {
    constexpr int LVPL = PassIter<BV>::LVPL, VPL = 1 << LVPL;
    const bool live = it.k < it.kend;
    const int llpt = it.lc - LVPL, ltpp = 6 - llpt;
    m.lc = it.lc;
    m.tbase = it.k * MKV_SEG + (it.p << ltpp);
    m.tlim = live ? it.k * MKV_SEG + it.ns : -1;
    const bool ok = live && (it.p << ltpp) + (lane >> llpt) < it.ns;
    const uint32_t voff = ok ? (uint32_t)((it.p << 10) + lane * 16) : kOutOfRange;
    const uint32_t ioff = (ok && it.lc < 7)
        ? (uint32_t)(((it.ns << it.lc) * BV) + (it.p << (6 + LVPL)) + lane * VPL) : kOutOfRange;
    v = __builtin_amdgcn_raw_buffer_load_b128(it.rs, voff, 0, kStreamLoad);
    if constexpr (VPL == 8) ix = __builtin_amdgcn_raw_buffer_load_b64(it.rs, ioff, 0, kStreamLoad);
    else ix.x = __builtin_amdgcn_raw_buffer_load_b32(it.rs, ioff, 0, kStreamLoad);
    if (live) it.next();
}

template <int BV>
__device__ __forceinline__ float bf_or_f(const uint32_t* w, int k) {
    if constexpr (BV == 2) return (k & 1) ? __uint_as_float(w[k >> 1] & 0xFFFF0000u) : __uint_as_float(w[k >> 1] << 16);
    else return __uint_as_float(w[k]);
}

template <int BV>
__device__ __forceinline__ void consume_pass(const u32x4& v, const u32x2& ix, const PassMeta& m, int lane,
                                             const float* sq, uint32_t* skeys) {
    constexpr int LVPL = PassIter<BV>::LVPL, VPL = 1 << LVPL;
    const int llpt = m.lc - LVPL;
    const int sub = lane & ((1 << llpt) - 1);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    float acc = 0.f;
    if (m.lc == 7) {
        // every channel stored: this lane holds channels [sub*VPL, sub*VPL + VPL)
        const f32x4* q4 = reinterpret_cast<const f32x4*>(sq + sub * VPL);
#pragma unroll
        for (int j = 0; j < VPL / 4; ++j) {
            const f32x4 qq = q4[j];
            acc = fmaf(qq.x, bf_or_f<BV>(w, 4 * j), acc);
            acc = fmaf(qq.y, bf_or_f<BV>(w, 4 * j + 1), acc);
            acc = fmaf(qq.z, bf_or_f<BV>(w, 4 * j + 2), acc);
            acc = fmaf(qq.w, bf_or_f<BV>(w, 4 * j + 3), acc);
        }
    } else {
#pragma unroll
        for (int k = 0; k < VPL; ++k) {
            const uint32_t iw = k < 4 ? ix.x : ix.y;
            const uint32_t ch = (iw >> (8 * (k & 3))) & 0xFFu;   // < 128 for stored data
            acc = fmaf(sq[ch], bf_or_f<BV>(w, k), acc);
        }
    }
    acc += dpp_f<0xB1>(acc);                    // pairs
    if (llpt >= 2) acc += dpp_f<0x4E>(acc);     // quads
    if (llpt >= 3) acc += dpp_f<0x141>(acc);    // groups of 8 (half-row mirror)
    if (llpt >= 4) acc += dpp_f<0x140>(acc);    // rows of 16 (row mirror)
    if (llpt >= 5) acc += __shfl_xor(acc, 16, MKV_WAVE);
    const int t = m.tbase + (lane >> llpt);
    if (sub == 0 && t < m.tlim) skeys[t] = score_key(acc);
}

// Grid: a.sgx workgroups per stream (the most any request needs), streams in order; workgroups past their
// stream's count exit at once.
template <int BV>
__global__ __launch_bounds__(256) void k_score(DecArgs a) {
    __shared__ float sq[2 * MKV_D];             // Qbar, then a zero pad that index bytes >= 128 can never reach
    __shared__ __attribute__((aligned(16))) uint32_t sh[kHistBins];
    __shared__ uint32_t shc[64];                    // coarse bins (top 6 key bits)
    __shared__ uint32_t skeys[kMaxSpw * MKV_SEG];   // this workgroup's keys, written out per segment at the end
    __shared__ uint64_t s_off[kMaxSpw];
    __shared__ int s_m[kMaxSpw];
    const int stream = uni((int)(blockIdx.x / (uint32_t)a.sgx)), i = uni((int)blockIdx.x - stream * a.sgx);
    const int r = uni(stream / a.Hkv), g = stream - r * a.Hkv;
    const int n = a.t_n[r], Sr = (n + MKV_SEG - 1) / MKV_SEG, gs = (Sr + a.spw - 1) / a.spw;
    if (i >= gs) return;                        // whole workgroup, before any barrier
    const int stride = 4 * gs;
    const int64_t seg0 = (int64_t)a.Hkv * a.t_segbase[r] + (int64_t)g * a.t_scap[r];
    const int64_t keybase = key_base(a, r, g, n);
    const int tid = threadIdx.x;
    int nloc = 0;                               // valid slots form a prefix of [0, spw)
    for (int kk = 0; kk < a.spw / 4; ++kk) nloc += max(0, min(4, Sr - (4 * i + stride * kk)));
    nloc = uni(nloc);
    if (tid < nloc) {
        const int sg = slot_segment(i, tid, stride);
        const int c = a.keep[a.codes[seg0 + sg]];
        s_off[tid] = a.seg_off[seg0 + sg];
        s_m[tid] = (31 - __clz(c)) | (min(MKV_SEG, n - sg * MKV_SEG) << 8);
    }
    for (int j = tid; j < kHistBins / 4; j += 256) reinterpret_cast<u32x4*>(sh)[j] = u32x4{0u, 0u, 0u, 0u};
    if (tid < 64) shc[tid] = 0u;
    if (tid < MKV_D) {
        sq[tid] = a.qbar[(size_t)stream * MKV_D + tid];
        sq[MKV_D + tid] = 0.f;
    }
    __syncthreads();

    const int wid = uni(tid >> 6), lane = tid & 63;   // the wave index is uniform across the wave
    if (wid < nloc) {
        PassIter<BV> it;
        it.payload = a.payload;
        it.s_off = s_off;
        it.s_m = s_m;
        it.k = wid;
        it.kend = nloc;
        it.p = 0;
        it.load_seg();
        int np = 0;   // passes of this wave
        for (int k = wid; k < nloc; k += 4) {
            const int w = s_m[k], ltpp = 6 + PassIter<BV>::LVPL - (w & 0xFF), ns = w >> 8;
            np += (ns + (1 << ltpp) - 1) >> ltpp;
        }
        np = uni(np);
        u32x4 v[kRing];
        u32x2 ix[kRing];
        PassMeta m[kRing];
#pragma unroll
        for (int k = 0; k < kRing; ++k) issue_pass<BV>(it, lane, v[k], ix[k], m[k]);
        for (int base = 0; base < np; base += kRing) {
#pragma unroll
            for (int k = 0; k < kRing; ++k) {
                consume_pass<BV>(v[k], ix[k], m[k], lane, sq, skeys);
                issue_pass<BV>(it, lane, v[k], ix[k], m[k]);
            }
        }
    }
    __syncthreads();
    // keys out (256 contiguous bytes per segment, streamed past the caches) and the workgroup histogram
    for (int j = tid; j < nloc * MKV_SEG; j += 256) {
        const int tok = slot_segment(i, j >> 6, stride) * MKV_SEG + (j & 63);
        if (tok < n) {
            const uint32_t key = skeys[j];
            __builtin_nontemporal_store(key, &a.keys[keybase + tok]);
            atomicAdd(&sh[key >> 20], 1u);
            atomicAdd(&shc[key >> 26], 1u);
        }
    }
    __syncthreads();
    // flush the non-empty fine and coarse bins into one of the stream's histogram copies
    // copy: by the XCD the workgroup runs on (hardware register XCC_ID), so that each XCD's workgroups update
    // their own copy
    const int copy = __builtin_amdgcn_s_getreg((3 << 11) | (0 << 6) | 20) & (a.hcopies - 1);
    uint32_t* gh = a.hist + ((size_t)stream * a.hcopies + copy) * kHistBins;
#pragma unroll 4
    for (int j = tid; j < kHistBins; j += 256) {
        const uint32_t c = sh[j];
        if (c) atomic_add_dev(&gh[j], c);
    }
    if (tid < 64) {
        const uint32_t c = shc[tid];
        if (c) atomic_add_dev(&a.state[stream * kStateWords + kCoarseOff + 64 * copy + tid], c);
    }
}

hipError_t launch_score(const DecArgs& a, int n_blocks, hipStream_t s) {
    if (n_blocks == 0) return hipSuccess;
    if (a.dtype == 1) launch_kernel(k_score<2>, dim3(n_blocks), dim3(256), 0, s, a);
    else launch_kernel(k_score<4>, dim3(n_blocks), dim3(256), 0, s, a);
    return hipGetLastError();
}

// =====================================================================================================
// selection: collect (grid-wide) and emit (one workgroup per stream)
// =====================================================================================================
struct KBlock { int r, g, kb, n, stream; int64_t keybase; };

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
    k.keybase = key_base(a, k.r, k.g, k.n);
    return k;
}


// Bin of the T-th largest key (first wave of the block): the 64-bin coarse histogram (top 6 key bits) gives the
// coarse bin, its 64 fine bins (top 12 bits) the bin p1.  res <- p1, keys above p1, keys in p1, keys to take in p1.
__device__ __forceinline__ void find_threshold(const DecArgs& a, int stream, uint32_t T, uint32_t* res) {
    const int lane = threadIdx.x & 63;
    const uint32_t* st = a.state + stream * kStateWords;
    // the copies are summed from loads issued together (copies past hcopies re-read the last one, unused)
    uint32_t cv = 0;
#pragma unroll
    for (int c = 0; c < kMaxHistCopies; ++c) {
        const uint32_t v = st[kCoarseOff + 64 * min(c, a.hcopies - 1) + 63 - lane];
        cv += c < a.hcopies ? v : 0u;
    }
    const uint32_t ci = wave_incl_u32(cv), ce = ci - cv;
    const uint64_t cb_bal = __ballot(ce < T && ci >= T);
    const int cl = max(__ffsll((unsigned long long)cb_bal) - 1, 0);
    const int cb = 63 - cl;
    const uint32_t above = (uint32_t)__builtin_amdgcn_readlane((int)ce, cl);   // cl is the same on every lane
    uint32_t fv = 0;
#pragma unroll
    for (int c = 0; c < kMaxHistCopies; ++c) {
        const uint32_t v = a.hist[((size_t)stream * a.hcopies + min(c, a.hcopies - 1)) * kHistBins + cb * 64 + 63 - lane];
        fv += c < a.hcopies ? v : 0u;
    }
    const uint32_t fi = wave_incl_u32(fv) + above, fe = fi - fv;
    if (fe < T && fi >= T) {
        res[0] = (uint32_t)(cb * 64 + 63 - lane);
        res[1] = fe;
        res[2] = fv;
        res[3] = T - fe;
    }
}

// For every block of 4096 keys of a stream: keys above the threshold bin go to the stream's list of taken tokens,
// keys inside it to the candidate list (both unordered; space reserved with one device atomic per list).
__global__ __launch_bounds__(256) void k_sel_collect(DecArgs a) {
    __shared__ uint32_t res[4];
    __shared__ uint32_t tmp[8];
    __shared__ uint32_t s_base[2];
    const KBlock k = kblock(a);
    const int tid = threadIdx.x;
    const uint32_t T = (uint32_t)a.t_T[k.r];
    // the block's keys do not depend on the threshold: their loads are issued first and overlap its search
    const int lo = k.kb * kKeysPerBlock + 16 * tid;
    const u32x4* keys4 = reinterpret_cast<const u32x4*>(a.keys + k.keybase);
    const int last4 = (((k.n + 63) & ~63) >> 2) - 1;
    u32x4 kv[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) kv[q] = keys4[min((lo >> 2) + q, last4)];
    if (tid < 4) res[tid] = 0u;
    __syncthreads();
    if (tid < 64) find_threshold(a, k.stream, T, res);
    __syncthreads();
    const uint32_t p1 = res[0], ngt = res[1];
    uint32_t* st = a.state + k.stream * kStateWords;
    if (k.kb == 0 && tid < 4) st[ST_P1 + tid] = res[tid];
    uint32_t kk[16];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        kk[4 * q] = kv[q].x; kk[4 * q + 1] = kv[q].y; kk[4 * q + 2] = kv[q].z; kk[4 * q + 3] = kv[q].w;
    }
    uint32_t gm = 0, cm = 0;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        const bool in = lo + j < k.n;
        gm |= ((in && (kk[j] >> 20) > p1) ? 1u : 0u) << j;
        cm |= ((in && (kk[j] >> 20) == p1) ? 1u : 0u) << j;
    }
    uint32_t tot;
    const uint32_t off = block_exscan((uint32_t)__popc(gm) | ((uint32_t)__popc(cm) << 16), tmp, &tot);
    if (tid == 0) {
        s_base[0] = (tot & 0xFFFFu) ? atomic_add_dev(&st[ST_GTFILL], tot & 0xFFFFu) : 0u;
        s_base[1] = (tot >> 16) ? atomic_add_dev(&st[ST_CFILL], tot >> 16) : 0u;
    }
    __syncthreads();
    uint2* L = a.L + k.keybase;
    uint32_t pg = s_base[0] + (off & 0xFFFFu), pc = ngt + s_base[1] + (off >> 16);
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        if ((gm >> j) & 1u) L[pg++] = make_uint2((uint32_t)(lo + j), kk[j]);
        if ((cm >> j) & 1u) L[pc++] = make_uint2((uint32_t)(lo + j), kk[j]);
    }
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

// Lists at least this long are read four entries per thread at a time (the loads' latencies overlap); shorter
// ones one entry at a time (the batching's extra loads and code cost more there: measured on a 32768-token layer
// and the ragged mix)
constexpr uint32_t kBatchedList = 8192;

// Entries i0, i0 + 1024, i0 + 2048, i0 + 3072 of a list of n >= 1 entries (indices past the end re-read the last
// entry, which the caller skips), loaded together so that their latencies overlap.
__device__ __forceinline__ void load4_entries(const uint2* list, uint32_t i0, uint32_t n, uint2 (&e)[4]) {
#pragma unroll
    for (int u = 0; u < 4; ++u) e[u] = list[min(i0 + u * 1024, n - 1)];
}
__device__ __forceinline__ void load4_keys(const uint2* list, uint32_t i0, uint32_t n, uint32_t (&k)[4]) {
#pragma unroll
    for (int u = 0; u < 4; ++u) k[u] = list[min(i0 + u * 1024, n - 1)].y;
}

// Tokens per bitmap tile of the emit kernel: one 32-bit word per thread of a 1024-thread workgroup.
constexpr int kTileWords = 1024;
constexpr int kTileBits = kTileWords * 32;
static_assert(kTileBits == kEmitTileTokens, "the host sizes the emit grid with kEmitTileTokens");

// Tokens of one bitmap tile in ascending order (thread t owns word t), written from position carry on; returns
// the tile's count.
__device__ __forceinline__ uint32_t emit_tile(const uint32_t* bm, int tile0, uint32_t carry, int32_t* srow,
                                              int32_t* urow, uint32_t* tmp) {
    const int tid = threadIdx.x;
    uint32_t x = bm[tid];
    uint32_t tot;
    uint32_t pos = carry + block_exscan((uint32_t)__popc(x), tmp, &tot);
    while (x) {
        const int bit = __ffs(x) - 1;
        x &= x - 1;
        const int32_t idx = tile0 + tid * 32 + bit;
        srow[pos] = idx;
        if (urow) urow[pos] = idx;
        ++pos;
    }
    return tot;
}

// One workgroup per (stream, tile of kTileBits tokens): the exact T-th key among the stream's candidates (two
// 10-bit radix levels, recomputed by every tile of the stream), the cut among keys equal to it (lowest token
// indices first), the count of selected tokens before the tile, then the tile's selected tokens in ascending
// order through an LDS bitmap.  Tile 0 also pads the caller's selection row with -1.
__global__ __launch_bounds__(1024) void k_sel_emit(DecArgs a) {
    __shared__ uint32_t bm[kTileWords];
    __shared__ uint32_t h[1024];
    __shared__ uint32_t tmp[20];
    __shared__ uint32_t res[4];
    const int stream = blockIdx.x / a.etiles, tile = blockIdx.x - stream * a.etiles;
    const int r = stream / a.Hkv, g = stream - r * a.Hkv;
    const int n = a.t_n[r], T = a.t_T[r];
    const int tid = threadIdx.x;
    const int t0 = tile * kTileBits;
    int32_t* urow = a.sel ? a.sel + (size_t)stream * a.sel_stride : nullptr;
    if (n > 0 && T > 0 && t0 < n) {
        const uint32_t* st = a.state + stream * kStateWords;
        const uint32_t p1 = st[ST_P1], ngt = st[ST_NGT], ncand = st[ST_NCAND], need = st[ST_NEED];
        const uint2* L = a.L + key_base(a, r, g, n);
        const uint2* cand = L + ngt;
        const bool all = (need == ncand);
        uint32_t kstar = 0, need_eq = 0;
        int cut = n;   // ties equal to K* are taken up to this token index
        if (!all) {
            h[tid] = 0u;
            __syncthreads();
            if (ncand >= kBatchedList) {
                for (uint32_t i0 = tid; i0 < ncand; i0 += 4 * 1024) {
                    uint32_t kv[4];
                    load4_keys(cand, i0, ncand, kv);
#pragma unroll
                    for (int u = 0; u < 4; ++u)
                        if (i0 + u * 1024 < ncand) atomicAdd(&h[(kv[u] >> 10) & 1023u], 1u);
                }
            } else {
                for (uint32_t i = tid; i < ncand; i += 1024) atomicAdd(&h[(cand[i].y >> 10) & 1023u], 1u);
            }
            __syncthreads();
            find_bin1024(h, need, tmp, res);
            const uint32_t b2 = res[0], need2 = res[1];
            const uint32_t pre22 = (p1 << 10) | b2;
            h[tid] = 0u;
            __syncthreads();
            if (ncand >= kBatchedList) {
                for (uint32_t i0 = tid; i0 < ncand; i0 += 4 * 1024) {
                    uint32_t kv[4];
                    load4_keys(cand, i0, ncand, kv);
#pragma unroll
                    for (int u = 0; u < 4; ++u)
                        if (i0 + u * 1024 < ncand && (kv[u] >> 10) == pre22) atomicAdd(&h[kv[u] & 1023u], 1u);
                }
            } else {
                for (uint32_t i = tid; i < ncand; i += 1024) {
                    const uint32_t key = cand[i].y;
                    if ((key >> 10) == pre22) atomicAdd(&h[key & 1023u], 1u);
                }
            }
            __syncthreads();
            find_bin1024(h, need2, tmp, res);
            kstar = (pre22 << 10) | res[0];
            need_eq = res[1];
            const uint32_t eq_total = h[res[0]];
            if (need_eq < eq_total) {
                // the need_eq-th smallest token index among the keys equal to K*: scan tie bitmaps tile by tile
                uint32_t seen = 0;
                cut = -1;
                for (int u0 = 0; u0 < n && cut < 0; u0 += kTileBits) {
                    bm[tid] = 0u;
                    __syncthreads();
                    for (uint32_t i = tid; i < ncand; i += 1024) {
                        const uint2 e = cand[i];
                        if (e.y == kstar && (int)e.x >= u0 && (int)e.x < u0 + kTileBits)
                            atomicOr(&bm[(e.x - u0) >> 5], 1u << ((e.x - u0) & 31));
                    }
                    __syncthreads();
                    uint32_t x = bm[tid];
                    uint32_t tot;
                    const uint32_t before = seen + block_exscan((uint32_t)__popc(x), tmp, &tot);
                    if (before < need_eq && before + (uint32_t)__popc(x) >= need_eq) {
                        uint32_t run = before;
                        while (x) {
                            const int bit = __ffs(x) - 1;
                            x &= x - 1;
                            if (++run == need_eq) { res[0] = (uint32_t)(u0 + tid * 32 + bit); break; }
                        }
                    }
                    seen += tot;
                    __syncthreads();
                    if (seen >= need_eq) cut = (int)res[0];
                    __syncthreads();
                }
            }
        }
        auto taken = [&](const uint2 e) { return all || e.y > kstar || (e.y == kstar && (int)e.x <= cut); };
        // one pass over both lists: count the selected tokens before this tile (they come first in the stream's
        // ascending row) and mark the tile's own in the LDS bitmap
        bm[tid] = 0u;
        __syncthreads();
        uint32_t c = 0;
        auto mark = [&](const uint2 e) {
            const int x = (int)e.x;
            if (x < t0) ++c;
            else if (x < t0 + kTileBits) atomicOr(&bm[(x - t0) >> 5], 1u << ((x - t0) & 31));
        };
        if (ngt + ncand >= kBatchedList) {
            for (uint32_t i0 = tid; i0 < ngt; i0 += 4 * 1024) {
                uint2 e[4];
                load4_entries(L, i0, ngt, e);
#pragma unroll
                for (int u = 0; u < 4; ++u)
                    if (i0 + u * 1024 < ngt) mark(e[u]);
            }
            for (uint32_t i0 = tid; i0 < ncand; i0 += 4 * 1024) {
                uint2 e[4];
                load4_entries(cand, i0, ncand, e);
#pragma unroll
                for (int u = 0; u < 4; ++u)
                    if (i0 + u * 1024 < ncand && taken(e[u])) mark(e[u]);
            }
        } else {
            for (uint32_t i = tid; i < ngt; i += 1024) mark(L[i]);
            for (uint32_t i = tid; i < ncand; i += 1024) {
                const uint2 e = cand[i];
                if (taken(e)) mark(e);
            }
        }
        uint32_t before = 0;
        block_exscan(c, tmp, &before);   // its barriers also order the bitmap writes before emit_tile's reads
        emit_tile(bm, t0, before, a.sel_int + (size_t)stream * a.sel_int_stride, urow, tmp);
    }
    if (urow && tile == 0) {
        const int start = (n > 0) ? min(T, n) : 0;
        for (int j = start + tid; j < a.sel_stride; j += 1024) urow[j] = -1;
    }
}

hipError_t launch_sel_collect(const DecArgs& a, int n_blocks, hipStream_t s) {
    if (n_blocks == 0) return hipSuccess;
    launch_kernel(k_sel_collect, dim3(n_blocks), dim3(256), 0, s, a);
    return hipGetLastError();
}
hipError_t launch_sel_emit(const DecArgs& a, int n_streams, hipStream_t s) {
    if (n_streams == 0) return hipSuccess;
    launch_kernel(k_sel_emit, dim3(n_streams * a.etiles), dim3(1024), 0, s, a);
    return hipGetLastError();
}

// =====================================================================================================
// sparse exact attention over the selected tokens
// =====================================================================================================
// One selected token's row, as seen by the 8 lanes of its group: each lane owns c/8 consecutive slots.  A wave
// loads one value shape for all its tokens, sized by the largest kept count among them (LW value words per lane,
// enough for that count), and each lane loads exactly its own index bytes.  Value bytes past a lane's own slots
// are ignored: they belong to the token's later rows or to the segment's index block, except in a segment of a
// few rows at c <= 32, where the last row's widest load ends at most 40 bytes past the segment; every store and
// pool buffer keeps 256 bytes after its last payload byte for that.
template <int LW>
struct RowBuf {
    uint32_t v[LW];
    uint32_t ix[2];
};

struct RowMeta {
    uint64_t vaddr;   // first value byte of the token's row in the segment
    uint64_t iaddr;   // first index byte of the token's row (unused when c == 128)
};

template <int BV, int LW>
__device__ __forceinline__ void load_row(RowBuf<LW>& rb, const uint8_t* payload, const RowMeta& rm, int lc, int sl,
                                         bool ok) {
    const int nsl_shift = lc - 3;                       // log2 of slots per lane
    const uint8_t* va = ok ? payload + rm.vaddr + (size_t)(sl << nsl_shift) * BV : payload;
    if constexpr (LW >= 4) {
#pragma unroll
        for (int j = 0; j < LW / 4; ++j) {
            const u32x4 x = reinterpret_cast<const u32x4*>(va)[j];
            rb.v[4 * j] = x.x; rb.v[4 * j + 1] = x.y; rb.v[4 * j + 2] = x.z; rb.v[4 * j + 3] = x.w;
        }
    } else {
        const u32x2 x = *reinterpret_cast<const u32x2*>(va);
        rb.v[0] = x.x; rb.v[1] = x.y;
    }
    // index bytes: exactly this lane's slots (8 at c = 64, 4 at c = 32, 2 at c = 16, naturally aligned), none
    // when every channel is stored
    rb.ix[0] = 0u;
    rb.ix[1] = 0u;
    if (ok && lc < 7) {
        const uint8_t* ia = payload + rm.iaddr + (uint64_t)(sl << nsl_shift);
        if (lc == 6) {
            const u32x2 y = *reinterpret_cast<const u32x2*>(ia);
            rb.ix[0] = y.x;
            rb.ix[1] = y.y;
        } else if (lc == 5) {
            rb.ix[0] = *reinterpret_cast<const uint32_t*>(ia);
        } else {
            rb.ix[0] = *reinterpret_cast<const uint16_t*>(ia);
        }
    }
}

template <int BV, int LW>
__device__ __forceinline__ float row_val(const RowBuf<LW>& rb, int k) {
    if constexpr (BV == 2) return (k & 1) ? __uint_as_float(rb.v[k >> 1] & 0xFFFF0000u) : __uint_as_float(rb.v[k >> 1] << 16);
    else return __uint_as_float(rb.v[k]);
}

// channel of slot k of this lane (k < 8 for stored indices; c == 128 uses the slot position)
__device__ __forceinline__ int row_ch(const uint32_t* ix, int lc, int sl, int k) {
    if (lc == 7) return sl * 16 + k;
    return (ix[k >> 2] >> (8 * (k & 3))) & 0xFF;
}

constexpr int kDenseRow = MKV_D + 4;   // dense value row: 128 channels, a dummy column, 16-byte aligned rows

// G consecutive floats of the channel-major query table (one LDS read for G = 2, 4; two for G = 8)
template <int G>
__device__ __forceinline__ void load_q(const float* qt, int ch, float (&q)[G]) {
    if constexpr (G == 1) {
        q[0] = qt[ch];
    } else if constexpr (G == 2) {
        const float2 x = *reinterpret_cast<const float2*>(qt + ch * 2);
        q[0] = x.x; q[1] = x.y;
    } else {
#pragma unroll
        for (int j = 0; j < G / 4; ++j) {
            const f32x4 x = *reinterpret_cast<const f32x4*>(qt + ch * G + 4 * j);
            q[4 * j] = x.x; q[4 * j + 1] = x.y; q[4 * j + 2] = x.z; q[4 * j + 3] = x.w;
        }
    }
}

// Zero the value words of this lane past its nk slots (narrow shapes, where every token's slots are indexed).
template <int BV, int LW>
__device__ __forceinline__ void mask_tail(RowBuf<LW>& rb, int nk) {
    constexpr int SPW = 4 / BV;   // slots per word
#pragma unroll
    for (int j = 1; j < LW; ++j) rb.v[j] = (j * SPW < nk) ? rb.v[j] : 0u;
}

// LDS of one attention workgroup (4 waves of 64 tokens)
template <int G>
struct AttnLds {
    float qt[MKV_D * G];          // rotated queries, channel-major
    float vb[4][8][kDenseRow];    // each wave's dense value rows of one pass (column 128: unused slots)
    float ps[4][64][G];           // logits, then softmax numerators, of each wave's 64 tokens
    float wm[4][G], wl[4][G];
    float wacc[4][G][MKV_D];
    RowMeta mk[4][64], mv[4][64];
    int mc[4][64];                // log2 c of K | log2 c of V << 8 | valid << 16
};

// One wave's 8 * NP tokens (NP passes of 8): logits, softmax and the weighted value sum.  LW value words per
// lane cover the wave's largest kept count; NF passes are in flight at a time, and the first value passes are
// issued before the softmax so that their latency overlaps it.
template <int BV, int G, int LW, int NP>
__device__ __forceinline__ void attend_wave(AttnLds<G>& L, const uint8_t* payload, int wid, int lane, float (&acc)[G][2],
                                            float (&mW)[G], float (&lW)[G]) {
    constexpr int SLOTS = LW * 4 / BV;                       // value slots a lane holds
    constexpr int NF = (LW <= 4 ? 4 : 2) < NP ? (LW <= 4 ? 4 : 2) : NP;   // passes in flight (128 VGPRs at G = 4)
    constexpr bool NARROW = LW == 2 * BV;                   // kept counts <= 64: every slot is indexed
    const int t8 = lane >> 3, sl = lane & 7;
    const float scale = 1.4426950408889634f * 0.08838834764831845f;   // log2(e) / sqrt(128)

#pragma unroll
    for (int grp = 0; grp < NP / NF; ++grp) {
        RowBuf<LW> kr[NF];
        int wd[NF];
#pragma unroll
        for (int q = 0; q < NF; ++q) {
            const int tk = (grp * NF + q) * 8 + t8;
            wd[q] = L.mc[wid][tk];
            load_row<BV, LW>(kr[q], payload, L.mk[wid][tk], wd[q] & 0xFF, sl, (wd[q] >> 16) & 1);
        }
#pragma unroll
        for (int q = 0; q < NF; ++q) {
            const int lck = wd[q] & 0xFF, nk = 1 << (lck - 3);
            float lg[G];
#pragma unroll
            for (int h = 0; h < G; ++h) lg[h] = 0.f;
            if constexpr (NARROW) {
                // slots past nk hold zeros; their index bytes may be anything, so take 7 bits (a valid channel)
                mask_tail<BV, LW>(kr[q], nk);
#pragma unroll
                for (int k = 0; k < SLOTS; ++k) {
                    const int ch = (int)__builtin_amdgcn_ubfe(kr[q].ix[k >> 2], 8 * (k & 3), 7);
                    const float x = row_val<BV, LW>(kr[q], k);
                    float qq[G];
                    load_q<G>(L.qt, ch, qq);
#pragma unroll
                    for (int h = 0; h < G; ++h) lg[h] = fmaf(qq[h], x, lg[h]);
                }
            } else {
#pragma unroll
                for (int k = 0; k < SLOTS; ++k) {
                    const bool on = k < nk;
                    const int ch = on ? row_ch(kr[q].ix, lck, sl, k) : 0;
                    const float x = on ? row_val<BV, LW>(kr[q], k) : 0.f;
                    float qq[G];
                    load_q<G>(L.qt, ch, qq);
#pragma unroll
                    for (int h = 0; h < G; ++h) lg[h] = fmaf(qq[h], x, lg[h]);
                }
            }
            const bool valid = (wd[q] >> 16) & 1;
#pragma unroll
            for (int h = 0; h < G; ++h) {
                const float v = sum8(lg[h]);
                if (sl == 0) L.ps[wid][(grp * NF + q) * 8 + t8][h] = valid ? v * scale : -INFINITY;
            }
        }
    }

    RowBuf<LW> vr[NF];
    int wv[NF];
    auto issue_v = [&](int grp) {
#pragma unroll
        for (int q = 0; q < NF; ++q) {
            const int tk = (grp * NF + q) * 8 + t8;
            wv[q] = L.mc[wid][tk];
            load_row<BV, LW>(vr[q], payload, L.mv[wid][tk], (wv[q] >> 8) & 0xFF, sl, (wv[q] >> 16) & 1);
        }
    };
    issue_v(0);
    wave_lds_sync();

    // ---- softmax over the wave's tokens, one lane per token ----
#pragma unroll
    for (int h = 0; h < G; ++h) {
        const float x = lane < 8 * NP ? L.ps[wid][lane][h] : -INFINITY;
        const float M = wave_max(x);
        const float e = (M == -INFINITY) ? 0.f : exp2f(x - M);
        mW[h] = M;
        lW[h] = wave_sum(e);
        if (lane < 8 * NP) L.ps[wid][lane][h] = e;
    }
    wave_lds_sync();

    // ---- weighted sum of the sparse value rows; lane owns channels 2*lane, 2*lane+1 ----
    float* dense = L.vb[wid][t8];
#pragma unroll
    for (int grp = 0; grp < NP / NF; ++grp) {
        if (grp > 0) issue_v(grp);
#pragma unroll
        for (int q = 0; q < NF; ++q) {
            const int pass = grp * NF + q;
#pragma unroll
            for (int j = 0; j < MKV_D / 8; j += 4)
                *reinterpret_cast<f32x4*>(&dense[sl * 16 + j]) = f32x4{0.f, 0.f, 0.f, 0.f};
            wave_lds_sync();
            {
                const bool valid = (wv[q] >> 16) & 1;
                const int lcv = (wv[q] >> 8) & 0xFF, nv = valid ? 1 << (lcv - 3) : 0;
                // every slot writes; unused ones (and invalid tokens) go to the dummy column
#pragma unroll
                for (int k = 0; k < SLOTS; ++k) {
                    const int ch = k < nv ? row_ch(vr[q].ix, lcv, sl, k) : MKV_D;
                    dense[ch] = row_val<BV, LW>(vr[q], k);
                }
            }
            wave_lds_sync();
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                const float2 v = *reinterpret_cast<const float2*>(&L.vb[wid][t][2 * lane]);
#pragma unroll
                for (int h = 0; h < G; ++h) {
                    const float pp = L.ps[wid][pass * 8 + t][h];
                    acc[h][0] = fmaf(pp, v.x, acc[h][0]);
                    acc[h][1] = fmaf(pp, v.y, acc[h][1]);
                }
            }
            wave_lds_sync();
        }
    }
}

// Grid: one workgroup per chunk of 32 * NP selected tokens of a stream (8 * NP per wave); fewer passes per wave
// give more, shorter workgroups when there are few selected tokens in all.
template <int BV, int G, int NP>
__global__ __launch_bounds__(256) void k_attend(DecArgs a) {
    constexpr int CHUNK = 32 * NP;
    __shared__ __attribute__((aligned(16))) AttnLds<G> L;
    const int b = blockIdx.x;
    const int r = find_slot(a.t_ablk, a.B, b);
    const int n = a.t_n[r], T = a.t_T[r];
    const int nach = (T + CHUNK - 1) / CHUNK;
    const int local = b - a.t_ablk[r];
    const int g = local / nach, chunk = local - g * nach;
    const int stream = r * a.Hkv + g, Hq = a.G * a.Hkv;
    const int tid = threadIdx.x, wid = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    for (int i = tid; i < MKV_D * G; i += 256) {
        const int h = i >> 7, ch = i & 127;
        L.qt[ch * G + h] = a.qp[((size_t)r * Hq + g * G + h) * MKV_D + ch];
    }
    int lcmax;
    {   // this lane's token: list entry, segments, row addresses
        const int32_t* list = a.sel_int + (size_t)stream * a.sel_int_stride;
        const int li = chunk * CHUNK + wid * (8 * NP) + lane;
        const int j = (lane < 8 * NP && li < T) ? list[li] : -1;
        int word;
        RowMeta k_{0, 0}, v_{0, 0};
        if (j >= 0) {
            const int s = j >> 6, tt = j & 63, ns = min(MKV_SEG, n - s * MKV_SEG);
            const int64_t gk = (int64_t)a.Hkv * a.t_segbase[r] + (int64_t)g * a.t_scap[r] + s, gv = a.S + gk;
            const int ck = a.keep[a.codes[gk]], cv = a.keep[a.codes[gv]];
            const uint64_t ok_ = a.seg_off[gk], ov = a.seg_off[gv];
            const int lck = 31 - __clz(ck), lcv = 31 - __clz(cv);
            k_.vaddr = ok_ + ((uint64_t)tt << lck) * BV;
            k_.iaddr = ok_ + ((uint64_t)ns << lck) * BV + ((uint64_t)tt << lck);
            v_.vaddr = ov + ((uint64_t)tt << lcv) * BV;
            v_.iaddr = ov + ((uint64_t)ns << lcv) * BV + ((uint64_t)tt << lcv);
            word = lck | (lcv << 8) | (1 << 16);
            lcmax = max(lck, lcv);
        } else {
            word = 3 | (3 << 8);
            lcmax = 3;
        }
        L.mk[wid][lane] = k_;
        L.mv[wid][lane] = v_;
        L.mc[wid][lane] = word;
    }
    const bool wide = __ballot(lcmax == 7) != 0;   // some token of the wave keeps all 128 channels
    __syncthreads();

    float acc[G][2], mW[G], lW[G];
#pragma unroll
    for (int h = 0; h < G; ++h) { acc[h][0] = 0.f; acc[h][1] = 0.f; }
    // value words per lane: c/8 slots of BV bytes for the wave's largest c (at least 8 bytes)
    if (!wide) attend_wave<BV, G, 2 * BV, NP>(L, a.payload, wid, lane, acc, mW, lW);
    else attend_wave<BV, G, 4 * BV, NP>(L, a.payload, wid, lane, acc, mW, lW);

    if (lane == 0) {
#pragma unroll
        for (int h = 0; h < G; ++h) { L.wm[wid][h] = mW[h]; L.wl[wid][h] = lW[h]; }
    }
#pragma unroll
    for (int h = 0; h < G; ++h) { L.wacc[wid][h][2 * lane] = acc[h][0]; L.wacc[wid][h][2 * lane + 1] = acc[h][1]; }
    __syncthreads();
    for (int i = tid; i < G * MKV_D; i += 256) {
        const int h = i >> 7, ch = i & 127;
        float M = -INFINITY;
#pragma unroll
        for (int w2 = 0; w2 < 4; ++w2) M = fmaxf(M, L.wm[w2][h]);
        float O = 0.f, Ls = 0.f;
        if (M != -INFINITY) {
#pragma unroll
            for (int w2 = 0; w2 < 4; ++w2) {
                if (L.wm[w2][h] != -INFINITY) {
                    const float f = exp2f(L.wm[w2][h] - M);
                    O = fmaf(L.wacc[w2][h][ch], f, O);
                    Ls = fmaf(L.wl[w2][h], f, Ls);
                }
            }
        }
        float* dst = a.part + ((size_t)b * G + h) * (MKV_D + 2);
        if (ch == 0) { dst[0] = M; dst[1] = Ls; }
        dst[2 + ch] = O;
    }
}

// Four workgroups per stream, one per quarter of the output channels: each merges the attention chunks'
// partials (log-sum-exp) for all 128 channels, then writes its quarter of out = o'·B_Vᵀ.  Wave w
// merges query heads w, w+4, ...; lane l owns channels 2l, 2l+1 and chunk weights are broadcast from the lane
// that computed them, so every chunk's loads are independent and issue together.
template <int G>
__global__ __launch_bounds__(256) void k_combine(DecArgs a) {
    constexpr int QR = MKV_D / 4;                  // output channels of this workgroup
    __shared__ float o[G][MKV_D];
    __shared__ float bsh[QR * (MKV_D + 1)];
    const int stream = blockIdx.x >> 2, qd = blockIdx.x & 3, r = stream / a.Hkv, g = stream - r * a.Hkv;
    const int n = a.t_n[r], T = (n > 0) ? a.t_T[r] : 0;
    const int nach = (T + a.achunk - 1) / a.achunk;
    const int first = a.t_ablk[r] + g * nach;
    const int tid = threadIdx.x, lane = tid & 63, wid = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int Hq = a.G * a.Hkv;
    const float* Bv = a.basis ? a.basis + ((((size_t)a.t_bslot[r] * a.Hkv + g) * 2 + 1) << 14) : nullptr;
    f32x4 bvr[4];
    if (Bv) {   // rows [QR qd, QR qd + QR) of B_V; issued first so that their latency overlaps the merge
        const f32x4* src = reinterpret_cast<const f32x4*>(Bv + (size_t)QR * qd * MKV_D);
#pragma unroll
        for (int j = 0; j < 4; ++j) bvr[j] = src[tid + 256 * j];
    }
    constexpr int PW = MKV_D + 2;
    for (int h = wid; h < G; h += 4) {
        float M = -INFINITY;
        for (int c = lane; c < nach; c += 64) M = fmaxf(M, a.part[((size_t)(first + c) * G + h) * PW]);
        M = wave_max(M);
        float O0 = 0.f, O1 = 0.f, Ls = 0.f;
        if (M != -INFINITY) {
            for (int c0 = 0; c0 < nach; c0 += 64) {
                const int c = c0 + lane;
                float f = 0.f, l = 0.f;
                if (c < nach) {
                    const float* pp = a.part + ((size_t)(first + c) * G + h) * PW;
                    const float m = pp[0];
                    f = (m == -INFINITY) ? 0.f : exp2f(m - M);
                    l = pp[1];
                }
                Ls += f * l;
                const int cnt = min(64, nach - c0);
                int k = 0;
                for (; k + 16 <= cnt; k += 16) {
                    float2 v[16];
#pragma unroll
                    for (int u = 0; u < 16; ++u)
                        v[u] = *reinterpret_cast<const float2*>(a.part + ((size_t)(first + c0 + k + u) * G + h) * PW + 2 + 2 * lane);
#pragma unroll
                    for (int u = 0; u < 16; ++u) {
                        const float fk = lane_f(f, k + u);
                        O0 = fmaf(fk, v[u].x, O0);
                        O1 = fmaf(fk, v[u].y, O1);
                    }
                }
                for (; k + 8 <= cnt; k += 8) {
                    float2 v[8];
#pragma unroll
                    for (int u = 0; u < 8; ++u)
                        v[u] = *reinterpret_cast<const float2*>(a.part + ((size_t)(first + c0 + k + u) * G + h) * PW + 2 + 2 * lane);
#pragma unroll
                    for (int u = 0; u < 8; ++u) {
                        const float fk = lane_f(f, k + u);
                        O0 = fmaf(fk, v[u].x, O0);
                        O1 = fmaf(fk, v[u].y, O1);
                    }
                }
                for (; k < cnt; ++k) {
                    const float2 v = *reinterpret_cast<const float2*>(a.part + ((size_t)(first + c0 + k) * G + h) * PW + 2 + 2 * lane);
                    const float fk = lane_f(f, k);
                    O0 = fmaf(fk, v.x, O0);
                    O1 = fmaf(fk, v.y, O1);
                }
            }
            Ls = wave_sum(Ls);
        }
        o[h][2 * lane] = (Ls > 0.f) ? O0 / Ls : 0.f;
        o[h][2 * lane + 1] = (Ls > 0.f) ? O1 / Ls : 0.f;
    }
    if (Bv) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int e = 4 * (tid + 256 * j), row = e >> 7, col = e & 127;
            float* d = &bsh[row * (MKV_D + 1) + col];
            d[0] = bvr[j].x; d[1] = bvr[j].y; d[2] = bvr[j].z; d[3] = bvr[j].w;
        }
    }
    __syncthreads();
    for (int i = tid; i < G * QR; i += 256) {
        const int h = i / QR, row = i - h * QR;
        float v;
        if (Bv) {
            v = 0.f;
#pragma unroll 8
            for (int k = 0; k < MKV_D; ++k) v = fmaf(o[h][k], bsh[row * (MKV_D + 1) + k], v);
        } else {
            v = o[h][QR * qd + row];
        }
        a.out[((size_t)r * Hq + g * G + h) * MKV_D + QR * qd + row] = v;
    }
}

template <int BV, int NP>
static void launch_attend_g(const DecArgs& a, int n_blocks, hipStream_t s) {
    switch (a.G) {
        case 1: launch_kernel((k_attend<BV, 1, NP>), dim3(n_blocks), dim3(256), 0, s, a); break;
        case 2: launch_kernel((k_attend<BV, 2, NP>), dim3(n_blocks), dim3(256), 0, s, a); break;
        case 4: launch_kernel((k_attend<BV, 4, NP>), dim3(n_blocks), dim3(256), 0, s, a); break;
        default: launch_kernel((k_attend<BV, 8, NP>), dim3(n_blocks), dim3(256), 0, s, a); break;
    }
}

template <int BV>
static void launch_attend_np(const DecArgs& a, int n_blocks, hipStream_t s) {
    switch (a.achunk) {
        case 64: launch_attend_g<BV, 2>(a, n_blocks, s); break;
        case 128: launch_attend_g<BV, 4>(a, n_blocks, s); break;
        default: launch_attend_g<BV, 8>(a, n_blocks, s); break;
    }
}

hipError_t launch_attend(const DecArgs& a, int n_blocks, hipStream_t s) {
    if (n_blocks == 0) return hipSuccess;
    if (a.achunk != 64 && a.achunk != 128 && a.achunk != 256) return hipErrorInvalidValue;
    if (a.dtype == 1) launch_attend_np<2>(a, n_blocks, s);
    else launch_attend_np<4>(a, n_blocks, s);
    return hipGetLastError();
}

hipError_t launch_combine(const DecArgs& a, int n_streams, hipStream_t s) {
    if (n_streams == 0) return hipSuccess;
    const dim3 grid(4 * n_streams), block(256);   // four workgroups per stream, one per quarter of the channels
    switch (a.G) {
        case 1: launch_kernel(k_combine<1>, grid, block, 0, s, a); break;
        case 2: launch_kernel(k_combine<2>, grid, block, 0, s, a); break;
        case 4: launch_kernel(k_combine<4>, grid, block, 0, s, a); break;
        default: launch_kernel(k_combine<8>, grid, block, 0, s, a); break;
    }
    return hipGetLastError();
}

}  // namespace mkv
