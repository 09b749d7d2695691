// Host entry points of the compressed KV cache library: argument checks, buffer layouts, the store handle,
// launch orchestration and optional kernel timing.  No device memory is allocated here.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <map>
#include <mutex>
#include <new>
#include <string>
#include <vector>

#include "../../include/mkv.h"
#include "kernels.h"

using namespace mkv;

namespace {

thread_local std::string g_err;

mkv_status fail(mkv_status st, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
    return st;
}

constexpr uint64_t kAlign = 256;
inline uint64_t align_up(uint64_t x) { return (x + kAlign - 1) / kAlign * kAlign; }
inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// ---- kernel timing --------------------------------------------------------------------------------------
enum KernelId {
    K_UPLOAD = 0, K_CMP_DECIDE, K_CMP_SCAN, K_CMP_PACK, K_DEC_PREP, K_SCORE, K_SEL_COLLECT, K_SEL_EMIT,
    K_ATTEND, K_COMBINE, K_DENSE_ATTEND, K_DENSE_COMBINE, K_GRAM, K_GRAM_REDUCE, K_APPEND, K_POOL_PLACE, K_POOL_FIX,
    K_CMP_FUSED, K_COUNT
};
static_assert(K_COUNT <= MKV_PROFILE_KERNELS, "kernel ids must fit the profiling arrays and mask");
const char* kKernelNames[K_COUNT] = {"upload", "compress_decide", "compress_scan", "compress_pack", "decode_prep",
                                     "score", "select_collect", "select_emit", "attend", "combine",
                                     "dense_attend", "dense_combine", "gram", "gram_reduce", "append", "pool_place",
                                     "pool_fix", "compress"};

struct Profiler {
    std::mutex mu;
    bool on = false;
    int max_launches = 0;
    uint32_t mask = 0;              // kernel ids to time
    struct Rec { int kid; hipEvent_t a, b; };
    std::vector<Rec> recs;
    std::vector<hipEvent_t> pool;   // created events, reused across sessions
    size_t used = 0;
} g_prof;

thread_local LaunchEvents t_launch_events;

// Times one launch: its events travel with the kernel's dispatch (see launch_kernel); a launch function that
// enqueues nothing leaves them unused, and they are then recorded back to back (zero duration).
struct Timed {
    int kid;
    hipStream_t s;
    hipEvent_t a = nullptr, b = nullptr;
    Timed(int k, hipStream_t st) : kid(k), s(st) {
        if (!g_prof.on || !((g_prof.mask >> k) & 1u)) return;
        std::lock_guard<std::mutex> lk(g_prof.mu);
        if ((int)g_prof.recs.size() >= g_prof.max_launches) return;
        while (g_prof.pool.size() < g_prof.used + 2) {
            hipEvent_t e;
            if (hipEventCreate(&e) != hipSuccess) return;
            g_prof.pool.push_back(e);
        }
        a = g_prof.pool[g_prof.used++];
        b = g_prof.pool[g_prof.used++];
        t_launch_events = LaunchEvents{a, b, false};
    }
    ~Timed() {
        if (!a) return;
        if (!t_launch_events.used) {
            (void)hipEventRecord(a, s);
            (void)hipEventRecord(b, s);
        }
        t_launch_events = LaunchEvents{};
        std::lock_guard<std::mutex> lk(g_prof.mu);
        g_prof.recs.push_back({kid, a, b});
    }
};

template <class F>
mkv_status run(int kid, hipStream_t s, F&& f) {
    hipError_t e;
    {
        Timed t(kid, s);
        e = f();
    }
    if (e != hipSuccess) return fail(MKV_E_DEVICE, "launch of %s failed: %s", kKernelNames[kid], hipGetErrorString(e));
    return MKV_OK;
}

// Uploads int32 words to device memory through kernel arguments (no host-to-device copy).
mkv_status upload_words(int32_t* dst, const std::vector<int32_t>& w, size_t from, hipStream_t s) {
    for (size_t i = from; i < w.size(); i += kUploadWords) {
        Upload u;
        u.dst = dst + i;
        u.n = (int32_t)std::min<size_t>(kUploadWords, w.size() - i);
        std::memcpy(u.w, w.data() + i, sizeof(int32_t) * u.n);
        mkv_status st = run(K_UPLOAD, s, [&] { return launch_upload(u, s); });
        if (st != MKV_OK) return st;
    }
    return MKV_OK;
}

// ---- argument checks ------------------------------------------------------------------------------------
int dtype_bytes(mkv_dtype d) { return d == MKV_BF16 ? 2 : 4; }

mkv_status check_policy(const mkv_seg_policy* p, mkv_dtype dt) {
    if (!p) return fail(MKV_E_ARG, "policy is NULL");
    if (p->seg_len != MKV_SEG_LEN) return fail(MKV_E_UNSUPPORTED, "seg_len must be %d (got %d)", MKV_SEG_LEN, p->seg_len);
    if (p->n_keep < 1 || p->n_keep > MKV_MAX_KEEP) return fail(MKV_E_ARG, "n_keep must be in [1, %d] (got %d)", MKV_MAX_KEEP, p->n_keep);
    if (p->keep[0] != MKV_HEAD_DIM) return fail(MKV_E_ARG, "keep[0] must be %d (got %d)", MKV_HEAD_DIM, p->keep[0]);
    for (int k = 0; k < p->n_keep; ++k) {
        const int c = p->keep[k];
        if (c != 128 && c != 64 && c != 32 && c != 16) return fail(MKV_E_UNSUPPORTED, "keep[%d] = %d: supported counts are 128, 64, 32, 16", k, c);
        if (k > 0 && c >= p->keep[k - 1]) return fail(MKV_E_ARG, "keep[] must be strictly decreasing");
    }
    if (dt == MKV_FP32 && p->n_keep > 3) return fail(MKV_E_UNSUPPORTED, "fp32 stores support at most 3 kept counts");
    if (!(p->energy_frac > 0.0 && p->energy_frac <= 1.0)) return fail(MKV_E_ARG, "energy_frac must be in (0, 1] (got %g)", p->energy_frac);
    return MKV_OK;
}

struct Shape {
    int32_t B = 0, Hkv = 0;
    mkv_dtype dtype = MKV_BF16;
    std::vector<int64_t> cu;       // current tokens: prefix sums
    int64_t total = 0;
    // Segment slots come from the capacities (the current contexts unless the store is growable), so that
    // appended tokens never move another stream's slots.
    std::vector<int64_t> cap;      // per request: token capacity (>= its context)
    std::vector<int32_t> scap;     // per request: segment slots per stream, ceil(cap / 64)
    std::vector<int32_t> segbase;  // per request: slots of the earlier requests (per KV head)
    int64_t total_cap = 0;
    int64_t S = 0;                 // segment slots per tensor
    bool growable = false;
    std::vector<int32_t> bslot;    // per request: basis slot (its index, unless the store is a pool view)
};

// Segment slots from capacities (cap NULL: the current contexts).
mkv_status set_capacity(Shape* sh, const int64_t* cap) {
    sh->cap.resize(sh->B);
    sh->scap.resize(sh->B);
    sh->segbase.resize(sh->B);
    int64_t segs = 0, tot = 0;
    for (int r = 0; r < sh->B; ++r) {
        const int64_t n = sh->cu[r + 1] - sh->cu[r];
        const int64_t c = cap ? cap[r] : n;
        if (c < n) return fail(MKV_E_ARG, "capacity[%d] = %lld is below its context %lld", r, (long long)c, (long long)n);
        sh->cap[r] = c;
        sh->scap[r] = (int32_t)cdiv(c, MKV_SEG_LEN);
        sh->segbase[r] = (int32_t)segs;
        segs += sh->scap[r];
        tot += c;
    }
    if (tot * (int64_t)sh->Hkv >= (int64_t)INT32_MAX)
        return fail(MKV_E_UNSUPPORTED, "capacity tokens x KV heads must stay below 2^31 (got %lld)", (long long)(tot * sh->Hkv));
    sh->total_cap = tot;
    sh->S = segs * sh->Hkv;
    sh->growable = cap != nullptr;
    sh->bslot.resize(sh->B);
    for (int r = 0; r < sh->B; ++r) sh->bslot[r] = r;
    return MKV_OK;
}

mkv_status check_kv(const mkv_kv_desc* kv, bool need_data, Shape* sh) {
    if (!kv) return fail(MKV_E_ARG, "kv descriptor is NULL");
    if (kv->batch < 1) return fail(MKV_E_ARG, "batch must be >= 1 (got %d)", kv->batch);
    if (kv->n_kv_heads < 1) return fail(MKV_E_ARG, "n_kv_heads must be >= 1 (got %d)", kv->n_kv_heads);
    if (kv->head_dim != MKV_HEAD_DIM) return fail(MKV_E_UNSUPPORTED, "head_dim must be %d (got %d)", MKV_HEAD_DIM, kv->head_dim);
    if (kv->dtype != MKV_BF16 && kv->dtype != MKV_FP32) return fail(MKV_E_ARG, "unknown dtype %d", (int)kv->dtype);
    if (!kv->cu_seqlens) return fail(MKV_E_ARG, "cu_seqlens is NULL");
    if (kv->cu_seqlens[0] != 0) return fail(MKV_E_ARG, "cu_seqlens[0] must be 0");
    sh->B = kv->batch;
    sh->Hkv = kv->n_kv_heads;
    sh->dtype = kv->dtype;
    sh->cu.assign(kv->cu_seqlens, kv->cu_seqlens + kv->batch + 1);
    for (int r = 0; r < kv->batch; ++r)
        if (sh->cu[r + 1] < sh->cu[r]) return fail(MKV_E_ARG, "cu_seqlens must be non-decreasing (request %d)", r);
    sh->total = sh->cu[kv->batch];
    if (sh->total * (int64_t)sh->Hkv >= (int64_t)INT32_MAX)
        return fail(MKV_E_UNSUPPORTED, "total tokens x KV heads must stay below 2^31 (got %lld)", (long long)(sh->total * sh->Hkv));
    if (need_data && sh->total > 0 && (!kv->K || !kv->V)) return fail(MKV_E_ARG, "K and V must be non-NULL");
    return set_capacity(sh, nullptr);
}

struct StoreLayout {
    uint64_t codes, seg_off, basis, payload, capacity;
    uint64_t open_pack, open_rows, open_bytes;   // growable stores: per-stream open-segment areas (0 otherwise)
    uint64_t bytes;
};

// Depends on the capacities only (never on the current contexts), so appends keep every offset.
StoreLayout store_layout(const Shape& sh) {
    StoreLayout L;
    L.codes = kAlign;   // first 256 bytes: header (payload bytes in use)
    L.seg_off = align_up(L.codes + 2 * (uint64_t)sh.S);
    L.basis = align_up(L.seg_off + 16 * (uint64_t)sh.S);
    L.payload = align_up(L.basis + (uint64_t)sh.B * sh.Hkv * 2 * MKV_HEAD_DIM * MKV_HEAD_DIM * sizeof(float));
    L.capacity = 2ull * sh.Hkv * (uint64_t)sh.total_cap * MKV_HEAD_DIM * dtype_bytes(sh.dtype);
    // one-pass bf16 compression starts each workgroup's run of segments at the run's first slot at full size
    // (64 tokens x 128 channels): room for every slot at full size
    if (!sh.growable && sh.dtype == MKV_BF16)
        L.capacity = std::max<uint64_t>(L.capacity, 2ull * (uint64_t)sh.S * MKV_SEG_LEN * MKV_HEAD_DIM * 2);
    // growable stores: the first compression packs each stream's unfinished last segment into the payload like
    // any other; the appends that extend it re-pack it into the stream's open area and seal it at the payload's
    // end, so that first copy stays behind unused.  Room for one such segment (at most 63 rows, all channels)
    // per stream keeps every seal inside the payload.
    if (sh.growable)
        L.capacity += 2ull * sh.B * sh.Hkv * (uint64_t)(MKV_SEG_LEN - 1) * MKV_HEAD_DIM * dtype_bytes(sh.dtype);
    // an open segment holds at most 64 rows, packed or raw: 64 * 128 values
    L.open_bytes = sh.growable ? (uint64_t)MKV_SEG_LEN * MKV_HEAD_DIM * dtype_bytes(sh.dtype) : 0;
    const uint64_t streams = 2ull * sh.B * sh.Hkv;
    L.open_pack = L.payload + L.capacity;          // packed open segments, addressed like payload (seg_off)
    L.open_rows = L.open_pack + streams * L.open_bytes;
    L.bytes = L.open_rows + streams * L.open_bytes + kAlign;   // slack: fixed-shape row loads may read past
    return L;
}

// Compression work split: segments per workgroup (about 4096 workgroups over both tensors) and workgroups per
// tensor.
struct CmpPlan {
    int64_t spw = 1, nblk = 0;
};
CmpPlan cmp_plan(const Shape& sh) {
    CmpPlan P;
    P.spw = std::max<int64_t>(1, std::min<int64_t>(16, (2 * sh.S) / 4096));
    for (int r = 0; r < sh.B; ++r)
        P.nblk += (int64_t)sh.Hkv * cdiv(cdiv(sh.cu[r + 1] - sh.cu[r], MKV_SEG_LEN), P.spw);
    return P;
}

struct ScratchLayout {
    uint64_t tab, thr, wg, bytes;
};
// bf16 stores of fixed size are compressed in one pass, which keeps no thresholds and no workgroup totals
bool one_pass(const Shape& sh) { return sh.dtype == MKV_BF16 && !sh.growable; }
// Scratch of a compression: request tables | per-vector thresholds | one payload total per decide workgroup
// (two passes only).  Paged pools always take the two-pass layout (one_pass_ok false).
ScratchLayout scratch_layout(const Shape& sh, bool one_pass_ok = false) {
    ScratchLayout L;
    L.tab = 0;
    L.thr = align_up(sizeof(int32_t) * (6ull * sh.B + 1));
    if (one_pass_ok && one_pass(sh)) {
        L.wg = L.thr;
        L.bytes = L.thr;
        return L;
    }
    L.wg = align_up(L.thr + 2ull * sh.total * sh.Hkv * 4 * sizeof(uint16_t));
    L.bytes = L.wg + 2ull * std::max<int64_t>(cmp_plan(sh).nblk, 1) * sizeof(uint64_t);
    return L;
}

bool aligned(const void* p) { return (reinterpret_cast<uintptr_t>(p) % kAlign) == 0; }

}  // namespace

namespace mkv {
LaunchEvents& launch_events() { return t_launch_events; }
}  // namespace mkv

struct mkv_store {
    Shape sh;
    mkv_seg_policy policy;
    int32_t has_basis = 0;
    StoreLayout lay;
    uint8_t* base = nullptr;
    std::vector<int64_t> cu_cap;   // prefix sums of the capacities (for mkv_store_view)
    bool pool_view = false;
    uint64_t view_payload = 0;     // pool views: payload bytes of the listed requests
};

// ======================================================================================================
extern "C" {

void mkv_default_policy(mkv_seg_policy* p) {
    if (!p) return;
    std::memset(p, 0, sizeof *p);
    p->seg_len = MKV_SEG_LEN;
    p->n_keep = 3;
    p->keep[0] = 128;
    p->keep[1] = 64;
    p->keep[2] = 32;
    p->energy_frac = 0.9;
}

const char* mkv_last_error(void) { return g_err.c_str(); }

static mkv_status shape_for(const mkv_kv_desc* kv, const mkv_seg_policy* policy, const int64_t* capacity,
                            bool need_data, Shape* sh) {
    mkv_status st = check_kv(kv, need_data, sh);
    if (st) return st;
    if ((st = check_policy(policy, sh->dtype))) return st;
    if (capacity) {
        if (sh->dtype != MKV_BF16) return fail(MKV_E_UNSUPPORTED, "growable stores take bf16 K/V only");
        if ((st = set_capacity(sh, capacity))) return st;
    }
    return MKV_OK;
}

static mkv_status compress_bytes(const mkv_kv_desc* kv, const mkv_seg_policy* policy, const int64_t* capacity,
                                 size_t* store_bytes, size_t* scratch_bytes) {
    Shape sh;
    mkv_status st = shape_for(kv, policy, capacity, false, &sh);
    if (st) return st;
    if (!store_bytes || !scratch_bytes) return fail(MKV_E_ARG, "output pointers are NULL");
    *store_bytes = store_layout(sh).bytes;
    *scratch_bytes = scratch_layout(sh, true).bytes;
    return MKV_OK;
}

mkv_status mkv_compress_bytes(const mkv_kv_desc* kv, const mkv_seg_policy* policy, size_t* store_bytes,
                              size_t* scratch_bytes) {
    return compress_bytes(kv, policy, nullptr, store_bytes, scratch_bytes);
}

mkv_status mkv_compress_bytes_growable(const mkv_kv_desc* kv, const mkv_seg_policy* policy, const int64_t* capacity,
                                       size_t* store_bytes, size_t* scratch_bytes) {
    if (!capacity) return fail(MKV_E_ARG, "capacity is NULL");
    return compress_bytes(kv, policy, capacity, store_bytes, scratch_bytes);
}

static mkv_status make_handle(const Shape& sh, const mkv_seg_policy* policy, int32_t has_basis, void* buf,
                              mkv_store** out) {
    mkv_store* h = new (std::nothrow) mkv_store;
    if (!h) return fail(MKV_E_ARG, "out of host memory");
    h->sh = sh;
    h->policy = *policy;
    h->has_basis = has_basis;
    h->lay = store_layout(sh);
    h->base = static_cast<uint8_t*>(buf);
    h->cu_cap.assign(1, 0);
    for (int r = 0; r < sh.B; ++r) h->cu_cap.push_back(h->cu_cap.back() + sh.cap[r]);
    *out = h;
    return MKV_OK;
}

static mkv_status compress(const mkv_kv_desc* kv, const float* basis, const mkv_seg_policy* policy,
                           const int64_t* capacity, void* store_buf, size_t store_bytes, void* scratch,
                           size_t scratch_bytes, mkv_stream_t stream_, mkv_store** out) {
    hipStream_t stream = reinterpret_cast<hipStream_t>(stream_);
    Shape sh;
    mkv_status st = shape_for(kv, policy, capacity, true, &sh);
    if (st) return st;
    if (!out) return fail(MKV_E_ARG, "out is NULL");
    if (!store_buf || !scratch) return fail(MKV_E_ARG, "store_buf and scratch must be non-NULL");
    if (!aligned(store_buf) || !aligned(scratch)) return fail(MKV_E_ARG, "store_buf and scratch must be 256-byte aligned");
    const StoreLayout L = store_layout(sh);
    const ScratchLayout SL = scratch_layout(sh, true);
    if (store_bytes < L.bytes) return fail(MKV_E_ARG, "store_bytes %zu < required %llu", store_bytes, (unsigned long long)L.bytes);
    if (scratch_bytes < SL.bytes) return fail(MKV_E_ARG, "scratch_bytes %zu < required %llu", scratch_bytes, (unsigned long long)SL.bytes);

    uint8_t* base = static_cast<uint8_t*>(store_buf);
    uint8_t* scr = static_cast<uint8_t*>(scratch);
    const int64_t spw = cmp_plan(sh).spw;
    std::vector<int32_t> tab(6 * sh.B + 1);
    int64_t nblk = 0;
    for (int r = 0; r < sh.B; ++r) {
        const int64_t n = sh.cu[r + 1] - sh.cu[r];
        tab[r] = (int32_t)sh.cu[r];
        tab[sh.B + r] = (int32_t)n;
        tab[2 * sh.B + r] = sh.segbase[r];
        tab[3 * sh.B + r] = sh.scap[r];
        tab[4 * sh.B + r] = (int32_t)nblk;
        tab[5 * sh.B + 1 + r] = r;   // open slot
        nblk += (int64_t)sh.Hkv * cdiv(cdiv(n, MKV_SEG_LEN), spw);
    }
    tab[5 * sh.B] = (int32_t)nblk;
    if (2 * nblk > INT32_MAX) return fail(MKV_E_UNSUPPORTED, "too many workgroups");

    if ((st = upload_words(reinterpret_cast<int32_t*>(scr + SL.tab), tab, 0, stream))) return st;
    const float* bcopy = nullptr;
    if (basis) {
        const size_t bb = (size_t)sh.B * sh.Hkv * 2 * MKV_HEAD_DIM * MKV_HEAD_DIM * sizeof(float);
        hipError_t e = hipMemcpyAsync(base + L.basis, basis, bb, hipMemcpyDeviceToDevice, stream);
        if (e != hipSuccess) return fail(MKV_E_DEVICE, "basis copy failed: %s", hipGetErrorString(e));
        bcopy = reinterpret_cast<const float*>(base + L.basis);
    }
    CmpArgs a;
    std::memset(&a, 0, sizeof a);
    a.K = kv->K;
    a.V = kv->V;
    a.basis = bcopy;
    a.tab = reinterpret_cast<const int32_t*>(scr + SL.tab);
    a.B = sh.B;
    a.Hkv = sh.Hkv;
    a.spw = (int32_t)spw;
    a.nblk = (int32_t)nblk;
    a.S = sh.S;
    a.total_tokens = sh.total;
    a.codes = base + L.codes;
    a.seg_off = reinterpret_cast<uint64_t*>(base + L.seg_off);
    a.payload = base + L.payload;
    a.thr = one_pass(sh) ? nullptr : reinterpret_cast<uint16_t*>(scr + SL.thr);
    a.wg_total = one_pass(sh) ? nullptr : reinterpret_cast<uint64_t*>(scr + SL.wg);
    for (int k = 0; k < 4; ++k) a.keep[k] = k < policy->n_keep ? policy->keep[k] : 0;
    a.n_keep = policy->n_keep;
    a.frac = policy->energy_frac;
    if (sh.growable) {
        a.open_rows = reinterpret_cast<uint16_t*>(base + L.open_rows);
        a.open_elems = (int64_t)(L.open_bytes / 2);
    }
    const int dt = sh.dtype == MKV_BF16 ? 1 : 0;
    uint64_t* total = reinterpret_cast<uint64_t*>(base);
    if (one_pass(sh)) {
        // one pass: the payload counter starts at zero (a kernel writes it, so that the call records no memset)
        if ((st = upload_words(reinterpret_cast<int32_t*>(base), std::vector<int32_t>(2, 0), 0, stream))) return st;
        a.total = total;
        if ((st = run(K_CMP_FUSED, stream, [&] { return launch_cmp_fused(a, stream); }))) return st;
        return make_handle(sh, policy, basis ? 1 : 0, store_buf, out);
    }
    if ((st = run(K_CMP_DECIDE, stream, [&] { return launch_cmp_decide(a, dt, stream); }))) return st;
    if ((st = run(K_CMP_SCAN, stream, [&] { return launch_cmp_scan(a.wg_total, 2 * nblk, total, stream); }))) return st;
    if ((st = run(K_CMP_PACK, stream, [&] { return launch_cmp_pack(a, dt, stream); }))) return st;
    return make_handle(sh, policy, basis ? 1 : 0, store_buf, out);
}

mkv_status mkv_compress(const mkv_kv_desc* kv, const float* basis, const mkv_seg_policy* policy, void* store_buf,
                        size_t store_bytes, void* scratch, size_t scratch_bytes, mkv_stream_t stream,
                        mkv_store** out) {
    return compress(kv, basis, policy, nullptr, store_buf, store_bytes, scratch, scratch_bytes, stream, out);
}

mkv_status mkv_compress_growable(const mkv_kv_desc* kv, const float* basis, const mkv_seg_policy* policy,
                                 const int64_t* capacity, void* store_buf, size_t store_bytes, void* scratch,
                                 size_t scratch_bytes, mkv_stream_t stream, mkv_store** out) {
    if (!capacity) return fail(MKV_E_ARG, "capacity is NULL");
    return compress(kv, basis, policy, capacity, store_buf, store_bytes, scratch, scratch_bytes, stream, out);
}

mkv_status mkv_append_workspace_bytes(const mkv_store* s, size_t* ws_bytes) {
    if (!s || !ws_bytes) return fail(MKV_E_ARG, "store and ws_bytes must be non-NULL");
    *ws_bytes = align_up(20ull * s->sh.B);
    return MKV_OK;
}

mkv_status mkv_append(mkv_store* s, const void* K_new, const void* V_new, const int32_t* active, void* ws,
                      size_t ws_bytes, mkv_stream_t stream_) {
    hipStream_t stream = reinterpret_cast<hipStream_t>(stream_);
    if (!s) return fail(MKV_E_ARG, "store is NULL");
    Shape& sh = s->sh;
    if (!sh.growable) return fail(MKV_E_ARG, "the store was not built growable (mkv_compress_growable)");
    if (!K_new || !V_new) return fail(MKV_E_ARG, "K_new and V_new must be non-NULL");
    if (!ws || !aligned(ws)) return fail(MKV_E_ARG, "ws must be non-NULL and 256-byte aligned");
    if (ws_bytes < align_up(20ull * sh.B)) return fail(MKV_E_ARG, "ws_bytes %zu too small", ws_bytes);
    std::vector<int32_t> tab;
    for (int r = 0; r < sh.B; ++r) {
        if (active && !active[r]) continue;
        const int64_t n = sh.cu[r + 1] - sh.cu[r];
        if (n + 1 > sh.cap[r]) return fail(MKV_E_ARG, "request %d is at its capacity (%lld tokens)", r, (long long)sh.cap[r]);
        tab.push_back(r);                     // row of K_new / V_new
        tab.push_back((int32_t)n);
        tab.push_back(sh.Hkv * sh.segbase[r]);
        tab.push_back(sh.scap[r]);
        tab.push_back(r);                     // open slot
    }
    const int n_req = (int)(tab.size() / 5);
    if (n_req == 0) return MKV_OK;
    int32_t* tdev = static_cast<int32_t*>(ws);
    mkv_status st;
    if ((st = upload_words(tdev, tab, 0, stream))) return st;
    const StoreLayout& L = s->lay;
    CmpArgs a;
    std::memset(&a, 0, sizeof a);
    for (int k = 0; k < 4; ++k) a.keep[k] = k < s->policy.n_keep ? s->policy.keep[k] : 0;
    a.n_keep = s->policy.n_keep;
    a.frac = s->policy.energy_frac;
    AppendArgs x;
    x.Kn = static_cast<const uint16_t*>(K_new);
    x.Vn = static_cast<const uint16_t*>(V_new);
    x.basis = s->has_basis ? reinterpret_cast<const float*>(s->base + L.basis) : nullptr;
    x.tab = tdev;
    x.Hkv = sh.Hkv;
    x.S = sh.S;
    x.codes = s->base + L.codes;
    x.seg_off = reinterpret_cast<uint64_t*>(s->base + L.seg_off);
    x.payload = s->base + L.payload;
    x.open_pack = L.open_pack - L.payload;
    x.open_bytes = L.open_bytes;
    x.open_rows = reinterpret_cast<uint16_t*>(s->base + L.open_rows);
    x.total = reinterpret_cast<unsigned long long*>(s->base);
    x.seal_off = nullptr;
    if ((st = run(K_APPEND, stream, [&] { return launch_cmp_append(a, x, n_req, stream); }))) return st;
    // the listed requests now hold one more token
    std::vector<int64_t> n(sh.B);
    for (int r = 0; r < sh.B; ++r) n[r] = sh.cu[r + 1] - sh.cu[r];
    for (int i = 0; i < n_req; ++i) n[tab[5 * i]] += 1;
    for (int r = 0; r < sh.B; ++r) sh.cu[r + 1] = sh.cu[r] + n[r];
    sh.total = sh.cu[sh.B];
    return MKV_OK;
}

mkv_status mkv_store_attach(const mkv_kv_desc* kv, const mkv_seg_policy* policy, int32_t has_basis, void* store_buf,
                            size_t store_bytes, mkv_store** out) {
    Shape sh;
    mkv_status st = check_kv(kv, false, &sh);
    if (st) return st;
    if ((st = check_policy(policy, sh.dtype))) return st;
    if (!out || !store_buf) return fail(MKV_E_ARG, "store_buf and out must be non-NULL");
    if (!aligned(store_buf)) return fail(MKV_E_ARG, "store_buf must be 256-byte aligned");
    const StoreLayout L = store_layout(sh);
    if (store_bytes < L.bytes) return fail(MKV_E_ARG, "store_bytes %zu < required %llu", store_bytes, (unsigned long long)L.bytes);
    return make_handle(sh, policy, has_basis ? 1 : 0, store_buf, out);
}

mkv_status mkv_store_view(const mkv_store* s, mkv_store_info* info) {
    if (!s || !info) return fail(MKV_E_ARG, "store and info must be non-NULL");
    std::memset(info, 0, sizeof *info);
    info->batch = s->sh.B;
    info->n_kv_heads = s->sh.Hkv;
    info->head_dim = MKV_HEAD_DIM;
    info->dtype = s->sh.dtype;
    info->policy = s->policy;
    info->has_basis = s->has_basis;
    info->total_tokens = s->sh.total;
    info->segments_per_tensor = s->sh.S;
    info->cu_seqlens = s->sh.cu.data();
    info->codes = s->base + s->lay.codes;
    info->seg_off = s->base + s->lay.seg_off;
    info->basis = s->has_basis ? s->base + s->lay.basis : nullptr;
    info->payload = s->base + s->lay.payload;
    info->payload_total = s->base;
    info->payload_capacity = s->lay.capacity;
    info->store_bytes = s->lay.bytes;
    info->cu_capacity = s->cu_cap.data();
    info->growable = s->sh.growable ? 1 : 0;
    info->seg_base = s->sh.segbase.data();
    info->seg_slots = s->sh.scap.data();
    info->basis_slot = s->sh.bslot.data();
    info->pool_view = s->pool_view ? 1 : 0;
    return MKV_OK;
}

mkv_status mkv_store_payload_bytes(const mkv_store* s, mkv_stream_t stream, uint64_t* bytes) {
    if (!s || !bytes) return fail(MKV_E_ARG, "store and bytes must be non-NULL");
    if (s->pool_view) {
        *bytes = s->view_payload;
        return MKV_OK;
    }
    hipError_t e = hipMemcpyAsync(bytes, s->base, sizeof(uint64_t), hipMemcpyDeviceToHost, reinterpret_cast<hipStream_t>(stream));
    if (e == hipSuccess) e = hipStreamSynchronize(reinterpret_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(MKV_E_DEVICE, "payload size read failed: %s", hipGetErrorString(e));
    return MKV_OK;
}

mkv_status mkv_store_destroy(mkv_store* s) {
    delete s;
    return MKV_OK;
}

// ---- paged pools -------------------------------------------------------------------------------------------
namespace {

struct PoolLayout {
    uint64_t codes, seg_off, basis, payload, open_pack, open_rows, open_bytes, bytes;
};

int64_t pool_max_segment_bytes(mkv_dtype dt) { return (int64_t)MKV_SEG_LEN * MKV_HEAD_DIM * dtype_bytes(dt); }

mkv_status check_pool_desc(const mkv_pool_desc* d) {
    if (!d) return fail(MKV_E_ARG, "pool descriptor is NULL");
    if (d->n_kv_heads < 1) return fail(MKV_E_ARG, "n_kv_heads must be >= 1 (got %d)", d->n_kv_heads);
    if (d->dtype != MKV_BF16 && d->dtype != MKV_FP32) return fail(MKV_E_ARG, "unknown dtype %d", (int)d->dtype);
    if (d->max_requests < 1) return fail(MKV_E_ARG, "max_requests must be >= 1 (got %d)", d->max_requests);
    if (d->segment_slots < 0) return fail(MKV_E_ARG, "segment_slots must be >= 0");
    if (d->segment_slots * (int64_t)d->n_kv_heads >= (int64_t)INT32_MAX)
        return fail(MKV_E_UNSUPPORTED, "segment_slots x n_kv_heads must stay below 2^31");
    if (d->n_pages < 1 || d->n_pages >= (int64_t)INT32_MAX) return fail(MKV_E_ARG, "n_pages must be in [1, 2^31)");
    if (d->page_bytes % kAlign != 0 || d->page_bytes < pool_max_segment_bytes(d->dtype) || d->page_bytes > (1ll << 31))
        return fail(MKV_E_ARG, "page_bytes (%lld) must be a multiple of 256 in [%lld, 2^31]", (long long)d->page_bytes,
                    (long long)pool_max_segment_bytes(d->dtype));
    if (d->appendable && d->dtype != MKV_BF16) return fail(MKV_E_UNSUPPORTED, "appendable pools take bf16 K/V only");
    return MKV_OK;
}

PoolLayout pool_layout(const mkv_pool_desc& d) {
    PoolLayout L;
    const uint64_t S = (uint64_t)d.segment_slots * d.n_kv_heads;
    L.codes = kAlign;
    L.seg_off = align_up(L.codes + 2 * S);
    L.basis = align_up(L.seg_off + 16 * S);
    L.payload = align_up(L.basis + (d.has_basis ? (uint64_t)d.max_requests * d.n_kv_heads * 2 * MKV_HEAD_DIM *
                                                     MKV_HEAD_DIM * sizeof(float) : 0));
    // appendable pools: per request id and stream, an open-segment area (packed, addressed like the payload)
    // and the open segment's original rows
    L.open_bytes = d.appendable ? (uint64_t)pool_max_segment_bytes(d.dtype) : 0;
    const uint64_t streams = 2ull * d.max_requests * d.n_kv_heads;
    L.open_pack = L.payload + (uint64_t)d.n_pages * d.page_bytes;
    L.open_rows = L.open_pack + streams * L.open_bytes;
    L.bytes = L.open_rows + streams * L.open_bytes + kAlign;   // slack: fixed-shape row loads may read past
    return L;
}

// Pages one stream of a request can take: every page holds at least floor(page_bytes / largest segment) whole
// segments.
int64_t pool_pages_bound(const mkv_pool_desc& d, int64_t segments) {
    return cdiv(segments, d.page_bytes / pool_max_segment_bytes(d.dtype));
}

struct PoolScratch {
    uint64_t cmp, pages, used, list_base, page_ids, bytes;
};

PoolScratch pool_scratch_layout(const mkv_pool_desc& d, const Shape& ash) {
    PoolScratch L;
    const uint64_t streams = 2ull * ash.B * ash.Hkv;
    int64_t ids = 0;
    for (int r = 0; r < ash.B; ++r) ids += 2ll * ash.Hkv * pool_pages_bound(d, cdiv(ash.cu[r + 1] - ash.cu[r], MKV_SEG_LEN));
    L.cmp = 0;
    L.pages = align_up(scratch_layout(ash).bytes);
    L.used = align_up(L.pages + 4 * streams);
    L.list_base = align_up(L.used + 8 * streams);
    L.page_ids = align_up(L.list_base + 4 * streams);
    L.bytes = align_up(L.page_ids + 4 * (uint64_t)std::max<int64_t>(ids, 1));
    return L;
}

}  // namespace

struct mkv_pool {
    mkv_pool_desc d;
    mkv_seg_policy policy;
    PoolLayout lay;
    uint8_t* base = nullptr;
    std::vector<int32_t> free_pages;           // stack: the next page handed out is at the back
    std::map<int64_t, int64_t> free_ranges;    // free segment-slot ranges (units of n_kv_heads slots): start -> length
    struct Req {
        int64_t n = -1;                        // tokens; -1: the id is free
        int64_t cap = 0;                       // token capacity (appendable pools; else n)
        int32_t ubase = 0, scap = 0;           // first slot unit and slots per stream (from the capacity)
        std::vector<int32_t> pages;
        uint64_t payload = 0;                  // packed bytes (appended segments: their reserved bytes)
        int32_t apage = -1;                    // page taking this request's appended segments
        uint64_t aused = 0;                    // bytes reserved in it
    };
    std::vector<Req> req;
    std::vector<int32_t> free_ids;             // stack
    int32_t live = 0;
};

namespace {

// First fit over the free slot ranges; -1 if no range is long enough.  Empty requests take no slots.
int64_t pool_take_range(mkv_pool* p, int64_t len) {
    if (len == 0) return 0;
    for (auto it = p->free_ranges.begin(); it != p->free_ranges.end(); ++it) {
        if (it->second < len) continue;
        const int64_t start = it->first, rest = it->second - len;
        p->free_ranges.erase(it);
        if (rest > 0) p->free_ranges[start + len] = rest;
        return start;
    }
    return -1;
}

void pool_give_range(mkv_pool* p, int64_t start, int64_t len) {
    if (len == 0) return;
    auto next = p->free_ranges.lower_bound(start);
    if (next != p->free_ranges.end() && start + len == next->first) {
        len += next->second;
        next = p->free_ranges.erase(next);
    }
    if (next != p->free_ranges.begin()) {
        auto prev = std::prev(next);
        if (prev->first + prev->second == start) {
            prev->second += len;
            return;
        }
    }
    p->free_ranges[start] = len;
}

// Returns an id (with its slots and pages) to the free lists.
void pool_release(mkv_pool* p, int32_t id) {
    mkv_pool::Req& q = p->req[id];
    pool_give_range(p, q.ubase, q.scap);
    for (auto it = q.pages.rbegin(); it != q.pages.rend(); ++it) p->free_pages.push_back(*it);
    q = mkv_pool::Req();
    p->free_ids.push_back(id);
    --p->live;
}

}  // namespace

mkv_status mkv_pool_bytes(const mkv_pool_desc* desc, size_t* pool_bytes) {
    mkv_status st = check_pool_desc(desc);
    if (st) return st;
    if (!pool_bytes) return fail(MKV_E_ARG, "pool_bytes is NULL");
    *pool_bytes = pool_layout(*desc).bytes;
    return MKV_OK;
}

mkv_status mkv_pool_create(const mkv_pool_desc* desc, const mkv_seg_policy* policy, void* pool_buf,
                           size_t pool_bytes, mkv_pool** out) {
    mkv_status st = check_pool_desc(desc);
    if (st) return st;
    if ((st = check_policy(policy, desc->dtype))) return st;
    if (!pool_buf || !out) return fail(MKV_E_ARG, "pool_buf and out must be non-NULL");
    if (!aligned(pool_buf)) return fail(MKV_E_ARG, "pool_buf must be 256-byte aligned");
    const PoolLayout L = pool_layout(*desc);
    if (pool_bytes < L.bytes) return fail(MKV_E_ARG, "pool_bytes %zu < required %llu", pool_bytes, (unsigned long long)L.bytes);
    mkv_pool* p = new (std::nothrow) mkv_pool;
    if (!p) return fail(MKV_E_ARG, "out of host memory");
    p->d = *desc;
    p->policy = *policy;
    p->lay = L;
    p->base = static_cast<uint8_t*>(pool_buf);
    p->free_pages.resize(desc->n_pages);
    for (int64_t i = 0; i < desc->n_pages; ++i) p->free_pages[i] = (int32_t)(desc->n_pages - 1 - i);   // page 0 first
    if (desc->segment_slots > 0) p->free_ranges[0] = desc->segment_slots;
    p->req.resize(desc->max_requests);
    for (int32_t i = desc->max_requests - 1; i >= 0; --i) p->free_ids.push_back(i);   // id 0 first
    *out = p;
    return MKV_OK;
}

mkv_status mkv_pool_destroy(mkv_pool* p) {
    delete p;
    return MKV_OK;
}

static mkv_status pool_add_shape(const mkv_pool* p, const mkv_kv_desc* kv, bool need_data, Shape* ash) {
    if (!p) return fail(MKV_E_ARG, "pool is NULL");
    mkv_status st = check_kv(kv, need_data, ash);
    if (st) return st;
    if (ash->Hkv != p->d.n_kv_heads) return fail(MKV_E_ARG, "n_kv_heads %d differs from the pool's %d", ash->Hkv, p->d.n_kv_heads);
    if (ash->dtype != p->d.dtype) return fail(MKV_E_ARG, "dtype differs from the pool's");
    return MKV_OK;
}

mkv_status mkv_pool_add_scratch_bytes(const mkv_pool* p, const mkv_kv_desc* kv, size_t* scratch_bytes) {
    Shape ash;
    mkv_status st = pool_add_shape(p, kv, false, &ash);
    if (st) return st;
    if (!scratch_bytes) return fail(MKV_E_ARG, "scratch_bytes is NULL");
    *scratch_bytes = pool_scratch_layout(p->d, ash).bytes;
    return MKV_OK;
}

mkv_status mkv_pool_add(mkv_pool* p, const mkv_kv_desc* kv, const float* basis, const int64_t* capacity,
                        void* scratch, size_t scratch_bytes, mkv_stream_t stream_, int32_t* ids) {
    hipStream_t stream = reinterpret_cast<hipStream_t>(stream_);
    Shape ash;
    mkv_status st = pool_add_shape(p, kv, true, &ash);
    if (st) return st;
    if (!ids) return fail(MKV_E_ARG, "ids is NULL");
    if (!scratch || !aligned(scratch)) return fail(MKV_E_ARG, "scratch must be non-NULL and 256-byte aligned");
    if ((basis != nullptr) != (p->d.has_basis != 0))
        return fail(MKV_E_ARG, p->d.has_basis ? "the pool keeps bases: basis must be non-NULL" : "the pool keeps no bases: basis must be NULL");
    const PoolScratch SL = pool_scratch_layout(p->d, ash);
    if (scratch_bytes < SL.bytes) return fail(MKV_E_ARG, "scratch_bytes %zu < required %llu", scratch_bytes, (unsigned long long)SL.bytes);
    const int B = ash.B, Hkv = ash.Hkv;
    if ((int)p->free_ids.size() < B) return fail(MKV_E_ARG, "the pool has %zu free request ids, %d requested", p->free_ids.size(), B);
    if (capacity && !p->d.appendable) return fail(MKV_E_ARG, "capacities need an appendable pool");
    for (int r = 0; capacity && r < B; ++r)
        if (capacity[r] < ash.cu[r + 1] - ash.cu[r] || capacity[r] > INT32_MAX)
            return fail(MKV_E_ARG, "capacity[%d] = %lld must lie in [its context %lld, 2^31)", r, (long long)capacity[r],
                        (long long)(ash.cu[r + 1] - ash.cu[r]));

    // request ids and segment-slot ranges (host bookkeeping; undone if anything below fails)
    std::vector<int32_t> got;
    auto undo = [&] { for (auto it = got.rbegin(); it != got.rend(); ++it) pool_release(p, *it); };
    for (int r = 0; r < B; ++r) {
        const int64_t n = ash.cu[r + 1] - ash.cu[r];
        const int64_t cap = capacity ? capacity[r] : n;
        const int32_t scap = (int32_t)cdiv(cap, MKV_SEG_LEN);
        const int64_t ub = pool_take_range(p, scap);
        if (ub < 0) {
            undo();
            return fail(MKV_E_ARG, "no free run of %d segment slots for request %d (pool segment_slots %lld)", scap, r,
                        (long long)p->d.segment_slots);
        }
        const int32_t id = p->free_ids.back();
        p->free_ids.pop_back();
        ++p->live;
        mkv_pool::Req& q = p->req[id];
        q.n = n;
        q.cap = cap;
        q.ubase = (int32_t)ub;
        q.scap = scap;
        got.push_back(id);
    }

    uint8_t* scr = static_cast<uint8_t*>(scratch);
    const ScratchLayout CL = scratch_layout(ash);
    const int64_t spw = cmp_plan(ash).spw;
    std::vector<int32_t> tab(6 * B + 1);
    int64_t nblk = 0;
    for (int r = 0; r < B; ++r) {
        const int64_t n = ash.cu[r + 1] - ash.cu[r];
        tab[r] = (int32_t)ash.cu[r];
        tab[B + r] = (int32_t)n;
        tab[2 * B + r] = p->req[got[r]].ubase;
        tab[3 * B + r] = p->req[got[r]].scap;
        tab[4 * B + r] = (int32_t)nblk;
        tab[5 * B + 1 + r] = got[r];   // open slot: the request's id
        nblk += (int64_t)Hkv * cdiv(cdiv(n, MKV_SEG_LEN), spw);
    }
    tab[5 * B] = (int32_t)nblk;
    if (2 * nblk > INT32_MAX) { undo(); return fail(MKV_E_UNSUPPORTED, "too many workgroups"); }
    const int64_t S = p->d.segment_slots * Hkv;
    const int streams = 2 * B * Hkv;

    CmpArgs a;
    std::memset(&a, 0, sizeof a);
    a.K = kv->K;
    a.V = kv->V;
    a.basis = basis;            // the caller's copy, indexed like the batch; the pool keeps its own below
    a.tab = reinterpret_cast<const int32_t*>(scr + CL.tab);
    a.B = B;
    a.Hkv = Hkv;
    a.spw = (int32_t)spw;
    a.nblk = (int32_t)nblk;
    a.S = S;
    a.total_tokens = ash.total;
    a.codes = p->base + p->lay.codes;
    a.seg_off = reinterpret_cast<uint64_t*>(p->base + p->lay.seg_off);
    a.payload = p->base + p->lay.payload;
    a.thr = reinterpret_cast<uint16_t*>(scr + CL.thr);
    a.wg_total = reinterpret_cast<uint64_t*>(scr + CL.wg);
    for (int k = 0; k < 4; ++k) a.keep[k] = k < p->policy.n_keep ? p->policy.keep[k] : 0;
    a.n_keep = p->policy.n_keep;
    a.frac = p->policy.energy_frac;
    a.preplaced = 1;
    if (p->d.appendable) {
        a.open_rows = reinterpret_cast<uint16_t*>(p->base + p->lay.open_rows);
        a.open_elems = (int64_t)(p->lay.open_bytes / 2);
    }
    PoolArgs pa;
    std::memset(&pa, 0, sizeof pa);
    pa.tab = a.tab;
    pa.B = B;
    pa.Hkv = Hkv;
    pa.bv = dtype_bytes(ash.dtype);
    pa.S = S;
    for (int k = 0; k < 4; ++k) pa.keep[k] = a.keep[k];
    pa.codes = a.codes;
    pa.seg_off = a.seg_off;
    pa.page_bytes = (uint64_t)p->d.page_bytes;
    pa.pages = reinterpret_cast<int32_t*>(scr + SL.pages);
    pa.used = reinterpret_cast<uint64_t*>(scr + SL.used);
    pa.list_base = reinterpret_cast<const int32_t*>(scr + SL.list_base);
    pa.page_ids = reinterpret_cast<const int32_t*>(scr + SL.page_ids);
    const int dt = ash.dtype == MKV_BF16 ? 1 : 0;

    // 1. decide every segment's kept count, 2. place the segments into pages (ordinals), then read the page
    // counts back: the pages a request needs depend on its data
    if ((st = upload_words(reinterpret_cast<int32_t*>(scr + CL.tab), tab, 0, stream))) { undo(); return st; }
    if ((st = run(K_CMP_DECIDE, stream, [&] { return launch_cmp_decide(a, dt, stream); }))) { undo(); return st; }
    if ((st = run(K_POOL_PLACE, stream, [&] { return launch_pool_place(pa, streams, stream); }))) { undo(); return st; }
    std::vector<int32_t> need(streams);
    std::vector<uint64_t> used(streams);
    hipError_t e = hipMemcpyAsync(need.data(), pa.pages, 4ull * streams, hipMemcpyDeviceToHost, stream);
    if (e == hipSuccess) e = hipMemcpyAsync(used.data(), pa.used, 8ull * streams, hipMemcpyDeviceToHost, stream);
    if (e == hipSuccess) e = hipStreamSynchronize(stream);
    if (e != hipSuccess) { undo(); return fail(MKV_E_DEVICE, "page count read-back failed: %s", hipGetErrorString(e)); }
    int64_t total = 0;
    for (int i = 0; i < streams; ++i) total += need[i];
    if (total > (int64_t)p->free_pages.size()) {
        undo();
        return fail(MKV_E_ARG, "the pool has %zu free pages, the new requests need %lld", p->free_pages.size(),
                    (long long)total);
    }
    // 3. hand out pages in stream order, 4. turn ordinals into payload offsets, 5. pack
    std::vector<int32_t> lists(streams + total);
    int64_t k = streams;
    for (int i = 0; i < streams; ++i) {
        lists[i] = (int32_t)(k - streams);
        mkv_pool::Req& q = p->req[got[i / (2 * Hkv)]];
        for (int j = 0; j < need[i]; ++j) {
            const int32_t pg = p->free_pages.back();
            p->free_pages.pop_back();
            q.pages.push_back(pg);
            lists[k++] = pg;
        }
        q.payload += used[i];
    }
    static_assert(sizeof(int32_t) == 4, "");
    e = hipMemcpyAsync(scr + SL.list_base, lists.data(), 4ull * streams, hipMemcpyHostToDevice, stream);
    if (e == hipSuccess && total > 0)
        e = hipMemcpyAsync(scr + SL.page_ids, lists.data() + streams, 4ull * total, hipMemcpyHostToDevice, stream);
    if (e == hipSuccess) e = hipStreamSynchronize(stream);   // the host lists go out of scope below
    if (e != hipSuccess) { undo(); return fail(MKV_E_DEVICE, "page list upload failed: %s", hipGetErrorString(e)); }
    if ((st = run(K_POOL_FIX, stream, [&] { return launch_pool_fix(pa, streams, stream); }))) { undo(); return st; }
    if ((st = run(K_CMP_PACK, stream, [&] { return launch_cmp_pack(a, dt, stream); }))) { undo(); return st; }
    if (basis) {
        const size_t per = (size_t)Hkv * 2 * MKV_HEAD_DIM * MKV_HEAD_DIM * sizeof(float);
        for (int r = 0; r < B; ++r) {
            e = hipMemcpyAsync(p->base + p->lay.basis + per * got[r], reinterpret_cast<const uint8_t*>(basis) + per * r,
                               per, hipMemcpyDeviceToDevice, stream);
            if (e != hipSuccess) { undo(); return fail(MKV_E_DEVICE, "basis copy failed: %s", hipGetErrorString(e)); }
        }
    }
    for (int r = 0; r < B; ++r) ids[r] = got[r];
    return MKV_OK;
}

mkv_status mkv_pool_append_workspace_bytes(const mkv_pool* p, int32_t n, size_t* ws_bytes) {
    if (!p || !ws_bytes || n < 0) return fail(MKV_E_ARG, "pool and ws_bytes must be non-NULL, n >= 0");
    *ws_bytes = align_up(20ull * n) + align_up(16ull * n * p->d.n_kv_heads);
    return MKV_OK;
}

mkv_status mkv_pool_append(mkv_pool* p, int32_t n, const int32_t* ids, const void* K_new, const void* V_new, void* ws,
                           size_t ws_bytes, mkv_stream_t stream_) {
    hipStream_t stream = reinterpret_cast<hipStream_t>(stream_);
    if (!p) return fail(MKV_E_ARG, "pool is NULL");
    if (!p->d.appendable) return fail(MKV_E_ARG, "the pool was not created appendable");
    if (n < 0 || (n > 0 && (!ids || !K_new || !V_new))) return fail(MKV_E_ARG, "ids, K_new and V_new must be non-NULL");
    if (n == 0) return MKV_OK;
    size_t need = 0;
    mkv_pool_append_workspace_bytes(p, n, &need);
    if (!ws || !aligned(ws) || ws_bytes < need) return fail(MKV_E_ARG, "ws must be 256-byte aligned with >= %zu bytes", need);
    const int Hkv = p->d.n_kv_heads;
    const uint64_t seal = (uint64_t)pool_max_segment_bytes(p->d.dtype);   // reserved per sealed segment
    int64_t new_pages = 0;
    for (int32_t i = 0; i < n; ++i) {
        if (ids[i] < 0 || ids[i] >= p->d.max_requests || p->req[ids[i]].n < 0)
            return fail(MKV_E_ARG, "request id %d is not in the pool", ids[i]);
        for (int32_t j = 0; j < i; ++j)
            if (ids[j] == ids[i]) return fail(MKV_E_ARG, "request id %d is listed twice", ids[i]);
        const mkv_pool::Req& q = p->req[ids[i]];
        if (q.n + 1 > q.cap) return fail(MKV_E_ARG, "request %d is at its capacity (%lld tokens)", ids[i], (long long)q.cap);
        if ((q.n + 1) % MKV_SEG_LEN == 0) {   // this append seals the request's 2 * n_kv_heads open segments
            uint64_t used = q.apage < 0 ? (uint64_t)p->d.page_bytes : q.aused;
            for (int k = 0; k < 2 * Hkv; ++k) {
                if (used + seal > (uint64_t)p->d.page_bytes) { ++new_pages; used = 0; }
                used += seal;
            }
        }
    }
    if (new_pages > (int64_t)p->free_pages.size())
        return fail(MKV_E_ARG, "the pool has %zu free pages, sealing the listed requests' segments needs %lld",
                    p->free_pages.size(), (long long)new_pages);
    // host-side placement of the sealed segments (worst-case size each), then one kernel
    std::vector<int32_t> words(5 * (size_t)n);
    std::vector<uint64_t> seals(2 * (size_t)Hkv * n, 0);
    for (int32_t i = 0; i < n; ++i) {
        mkv_pool::Req& q = p->req[ids[i]];
        words[5 * i] = i;
        words[5 * i + 1] = (int32_t)q.n;
        words[5 * i + 2] = Hkv * q.ubase;
        words[5 * i + 3] = q.scap;
        words[5 * i + 4] = ids[i];
        if ((q.n + 1) % MKV_SEG_LEN != 0) continue;
        for (int k = 0; k < 2 * Hkv; ++k) {
            if (q.apage < 0 || q.aused + seal > (uint64_t)p->d.page_bytes) {
                q.apage = p->free_pages.back();
                p->free_pages.pop_back();
                q.pages.push_back(q.apage);
                q.aused = 0;
            }
            seals[2 * (size_t)Hkv * i + k] = (uint64_t)q.apage * p->d.page_bytes + q.aused;
            q.aused += seal;
            q.payload += seal;
        }
    }
    std::vector<int32_t> up(words);
    const size_t o_seal = align_up(20ull * n) / 4;
    up.resize(o_seal + 4 * (size_t)Hkv * n, 0);
    std::memcpy(up.data() + o_seal, seals.data(), seals.size() * sizeof(uint64_t));
    int32_t* wdev = static_cast<int32_t*>(ws);
    mkv_status st;
    if ((st = upload_words(wdev, up, 0, stream))) return st;
    CmpArgs a;
    std::memset(&a, 0, sizeof a);
    for (int k = 0; k < 4; ++k) a.keep[k] = k < p->policy.n_keep ? p->policy.keep[k] : 0;
    a.n_keep = p->policy.n_keep;
    a.frac = p->policy.energy_frac;
    AppendArgs x;
    x.Kn = static_cast<const uint16_t*>(K_new);
    x.Vn = static_cast<const uint16_t*>(V_new);
    x.basis = p->d.has_basis ? reinterpret_cast<const float*>(p->base + p->lay.basis) : nullptr;
    x.tab = wdev;
    x.seal_off = reinterpret_cast<const uint64_t*>(wdev + o_seal);
    x.Hkv = Hkv;
    x.S = p->d.segment_slots * Hkv;
    x.codes = p->base + p->lay.codes;
    x.seg_off = reinterpret_cast<uint64_t*>(p->base + p->lay.seg_off);
    x.payload = p->base + p->lay.payload;
    x.open_pack = p->lay.open_pack - p->lay.payload;
    x.open_bytes = p->lay.open_bytes;
    x.open_rows = reinterpret_cast<uint16_t*>(p->base + p->lay.open_rows);
    x.total = nullptr;
    if ((st = run(K_APPEND, stream, [&] { return launch_cmp_append(a, x, n, stream); }))) return st;
    for (int32_t i = 0; i < n; ++i) p->req[ids[i]].n += 1;
    return MKV_OK;
}

mkv_status mkv_pool_remove(mkv_pool* p, int32_t n, const int32_t* ids) {
    if (!p) return fail(MKV_E_ARG, "pool is NULL");
    if (n < 0 || (n > 0 && !ids)) return fail(MKV_E_ARG, "ids must list n >= 0 request ids");
    for (int32_t i = 0; i < n; ++i) {
        if (ids[i] < 0 || ids[i] >= p->d.max_requests || p->req[ids[i]].n < 0)
            return fail(MKV_E_ARG, "request id %d is not in the pool", ids[i]);
        for (int32_t j = 0; j < i; ++j)
            if (ids[j] == ids[i]) return fail(MKV_E_ARG, "request id %d is listed twice", ids[i]);
    }
    for (int32_t i = 0; i < n; ++i) pool_release(p, ids[i]);
    return MKV_OK;
}

mkv_status mkv_pool_view(const mkv_pool* p, int32_t n, const int32_t* ids, mkv_store** out) {
    if (!p || !out) return fail(MKV_E_ARG, "pool and out must be non-NULL");
    if (n < 1 || !ids) return fail(MKV_E_ARG, "a view lists n >= 1 request ids");
    Shape sh;
    sh.B = n;
    sh.Hkv = p->d.n_kv_heads;
    sh.dtype = p->d.dtype;
    sh.cu.assign(1, 0);
    uint64_t payload = 0;
    for (int32_t i = 0; i < n; ++i) {
        if (ids[i] < 0 || ids[i] >= p->d.max_requests || p->req[ids[i]].n < 0)
            return fail(MKV_E_ARG, "request id %d is not in the pool", ids[i]);
        const mkv_pool::Req& q = p->req[ids[i]];
        sh.cu.push_back(sh.cu.back() + q.n);
        sh.cap.push_back(q.cap);
        sh.scap.push_back(q.scap);
        sh.segbase.push_back(q.ubase);
        sh.bslot.push_back(ids[i]);
        payload += q.payload;
    }
    sh.total = sh.cu.back();
    sh.total_cap = 0;
    for (int64_t c : sh.cap) sh.total_cap += c;
    if (sh.total * (int64_t)sh.Hkv >= (int64_t)INT32_MAX)
        return fail(MKV_E_UNSUPPORTED, "total tokens x KV heads must stay below 2^31 (got %lld)", (long long)(sh.total * sh.Hkv));
    sh.S = p->d.segment_slots * sh.Hkv;
    sh.growable = false;
    mkv_store* h = new (std::nothrow) mkv_store;
    if (!h) return fail(MKV_E_ARG, "out of host memory");
    h->sh = sh;
    h->policy = p->policy;
    h->has_basis = p->d.has_basis ? 1 : 0;
    h->lay.codes = p->lay.codes;
    h->lay.seg_off = p->lay.seg_off;
    h->lay.basis = p->lay.basis;
    h->lay.payload = p->lay.payload;
    h->lay.capacity = (uint64_t)p->d.n_pages * p->d.page_bytes;
    h->lay.open_pack = h->lay.open_rows = h->lay.open_bytes = 0;
    h->lay.bytes = p->lay.bytes;
    h->base = p->base;
    h->cu_cap.assign(1, 0);
    for (int32_t i = 0; i < n; ++i) h->cu_cap.push_back(h->cu_cap.back() + sh.cap[i]);
    h->pool_view = true;
    h->view_payload = payload;
    *out = h;
    return MKV_OK;
}

mkv_status mkv_pool_stats(const mkv_pool* p, mkv_pool_info* info) {
    if (!p || !info) return fail(MKV_E_ARG, "pool and info must be non-NULL");
    std::memset(info, 0, sizeof *info);
    info->desc = p->d;
    info->live_requests = p->live;
    info->free_pages = (int64_t)p->free_pages.size();
    for (const auto& fr : p->free_ranges) {
        info->free_segment_slots += fr.second;
        info->largest_free_run = std::max<int64_t>(info->largest_free_run, fr.second);
    }
    info->codes = p->base + p->lay.codes;
    info->seg_off = p->base + p->lay.seg_off;
    info->basis = p->d.has_basis ? p->base + p->lay.basis : nullptr;
    info->payload = p->base + p->lay.payload;
    info->pool_bytes = p->lay.bytes;
    return MKV_OK;
}

mkv_status mkv_pool_request(const mkv_pool* p, int32_t id, int64_t* n_tokens, int64_t* capacity, int64_t* pages,
                            uint64_t* payload_bytes) {
    if (!p) return fail(MKV_E_ARG, "pool is NULL");
    if (id < 0 || id >= p->d.max_requests || p->req[id].n < 0) return fail(MKV_E_ARG, "request id %d is not in the pool", id);
    const mkv_pool::Req& q = p->req[id];
    if (n_tokens) *n_tokens = q.n;
    if (capacity) *capacity = q.cap;
    if (pages) *pages = (int64_t)q.pages.size();
    if (payload_bytes) *payload_bytes = q.payload;
    return MKV_OK;
}

// ---- decode ------------------------------------------------------------------------------------------------
namespace {

struct DecPlan {
    int32_t G = 0, Hq = 0, spw = 0, sgx = 0, max_T = 0, hcopies = 1, etiles = 1, achunk = kAttnChunk;
    std::vector<int32_t> tab;    // n | segbase | scap | tokbase | T | kblk | ablk | basis slot
    int64_t n_sblk = 0, n_kblk = 0, n_ablk = 0;
    uint64_t o_tab, o_state, o_hist, o_qp, o_qbar, o_keys, o_L, o_sel, o_part, bytes;
};

mkv_status plan_decode(const mkv_store* s, int32_t n_q_heads, const int32_t* T, DecPlan* P) {
    if (!s) return fail(MKV_E_ARG, "store is NULL");
    if (!T) return fail(MKV_E_ARG, "T is NULL");
    const Shape& sh = s->sh;
    if (n_q_heads < 1 || n_q_heads % sh.Hkv != 0) return fail(MKV_E_ARG, "n_q_heads (%d) must be a positive multiple of n_kv_heads (%d)", n_q_heads, sh.Hkv);
    P->G = n_q_heads / sh.Hkv;
    if (P->G != 1 && P->G != 2 && P->G != 4 && P->G != 8) return fail(MKV_E_UNSUPPORTED, "query heads per KV head must be 1, 2, 4 or 8 (got %d)", P->G);
    P->Hq = n_q_heads;
    const int B = sh.B;
    // segments per score workgroup, a multiple of 4 (one segment per wave at a time): 8 once there are 64K
    // segments or more (measured best from 8 x 128K down to the 16-request ragged mix), else 4 for more
    // workgroups on small stores
    int64_t s_cur = 0;   // segments in use (the capacity may hold more)
    for (int r = 0; r < B; ++r) s_cur += (int64_t)sh.Hkv * cdiv(sh.cu[r + 1] - sh.cu[r], MKV_SEG_LEN);
    P->spw = s_cur >= 65536 ? 8 : 4;
    P->tab.assign(8 * B + 2, 0);
    int32_t* tn = P->tab.data();
    int32_t* tseg = tn + B;
    int32_t* tscap = tseg + B;
    int32_t* ttok = tscap + B;
    int32_t* tT = ttok + B;
    int32_t* tkb = tT + B;
    int32_t* tab_ = tkb + B + 1;
    int32_t* tbs = tab_ + B + 1;
    int64_t sgx = 0, kb = 0, ab = 0, kpad = 0;
    for (int r = 0; r < B; ++r) {
        if (T[r] < 1) return fail(MKV_E_ARG, "T[%d] = %d must be >= 1", r, T[r]);
        const int64_t n = sh.cu[r + 1] - sh.cu[r];
        const int64_t te = std::min<int64_t>(T[r], n);
        tn[r] = (int32_t)n;
        tseg[r] = sh.segbase[r];
        tscap[r] = sh.scap[r];
        ttok[r] = (int32_t)kpad;          // keys of request r start at Hkv * (earlier contexts padded to 64)
        kpad += cdiv(n, 64) * 64;
        tT[r] = (int32_t)te;
        tbs[r] = sh.bslot[r];
        tkb[r] = (int32_t)kb;
        sgx = std::max<int64_t>(sgx, cdiv(cdiv(n, MKV_SEG_LEN), P->spw));
        kb += (int64_t)sh.Hkv * cdiv(n, kKeysPerBlock);
        P->max_T = std::max<int32_t>(P->max_T, (int32_t)te);
        P->etiles = std::max<int32_t>(P->etiles, (int32_t)cdiv(n, kEmitTileTokens));
    }
    // selected tokens per attention workgroup: halved from 256 (down to 64) while the grid would not fill the
    // resident slots, so that small selections spread over more, shorter workgroups, as long as the combine
    // kernel merges at most 64 partials per head (its time grows with their number: at 1 x 1M tokens, 128
    // partials cost more there than the shorter attention workgroups save)
    auto attn_blocks = [&](int64_t chunk) {
        int64_t n_ab = 0;
        for (int r = 0; r < B; ++r) n_ab += (int64_t)sh.Hkv * cdiv(tT[r], chunk);
        return n_ab;
    };
    P->achunk = kAttnChunk;
    while (P->achunk > 64 && attn_blocks(P->achunk) < kAttnSlots && cdiv(P->max_T, P->achunk / 2) <= 64)
        P->achunk /= 2;
    for (int r = 0; r < B; ++r) {
        tab_[r] = (int32_t)ab;
        ab += (int64_t)sh.Hkv * cdiv(tT[r], P->achunk);
    }
    tkb[B] = (int32_t)kb;
    tab_[B] = (int32_t)ab;
    P->sgx = (int32_t)std::max<int64_t>(sgx, 1);
    P->n_sblk = (int64_t)P->sgx * B * sh.Hkv;
    P->n_kblk = kb;
    P->n_ablk = ab;
    if (P->n_sblk > INT32_MAX || kb > INT32_MAX || ab > INT32_MAX || (int64_t)B * sh.Hkv * P->etiles > INT32_MAX)
        return fail(MKV_E_UNSUPPORTED, "too many workgroups");
    const uint64_t streams = (uint64_t)B * sh.Hkv;
    const uint64_t th = (uint64_t)kpad * sh.Hkv;
    uint64_t o = 0;
    P->o_tab = o; o = align_up(o + 4 * P->tab.size());
    P->o_state = o; o = align_up(o + 4 * streams * kStateWords);
    // histogram copies: the score kernel's atomics on a stream's bins are spread over one copy per XCD up to 64
    // streams (8 x 131072 tokens: score -4.7 us, the larger clear in prep +1.3 us); above that one copy (the
    // 128-stream ragged mix: the clear would cost more than the spread saves)
    P->hcopies = streams <= 64 ? kMaxHistCopies : 1;
    P->o_hist = o; o = align_up(o + 4 * streams * (uint64_t)P->hcopies * kHistBins);
    P->o_qp = o; o = align_up(o + 4ull * B * n_q_heads * MKV_HEAD_DIM);
    P->o_qbar = o; o = align_up(o + 4 * streams * MKV_HEAD_DIM);
    P->o_keys = o; o = align_up(o + 4 * th);
    P->o_L = o; o = align_up(o + 8 * th);
    P->o_sel = o; o = align_up(o + 4 * streams * (uint64_t)std::max<int32_t>(P->max_T, 1));
    P->o_part = o; o = align_up(o + 4ull * std::max<int64_t>(ab, 1) * P->G * (MKV_HEAD_DIM + 2));
    P->bytes = o;
    return MKV_OK;
}

}  // namespace

mkv_status mkv_decode_workspace_bytes(const mkv_store* s, int32_t n_q_heads, const int32_t* T, size_t* ws_bytes) {
    DecPlan P;
    mkv_status st = plan_decode(s, n_q_heads, T, &P);
    if (st) return st;
    if (!ws_bytes) return fail(MKV_E_ARG, "ws_bytes is NULL");
    *ws_bytes = P.bytes;
    return MKV_OK;
}

namespace {

// The decode step over a planned workspace (every argument already checked).
mkv_status decode_run(const mkv_store* s, const void* q, const DecPlan& P, float* out, int32_t* sel,
                      int32_t sel_stride, void* ws, hipStream_t stream) {
    mkv_status st;
    const Shape& sh = s->sh;
    uint8_t* w = static_cast<uint8_t*>(ws);
    DecArgs a;
    std::memset(&a, 0, sizeof a);
    a.B = sh.B;
    a.Hkv = sh.Hkv;
    a.G = P.G;
    a.dtype = sh.dtype == MKV_BF16 ? 1 : 0;
    a.S = sh.S;
    a.codes = s->base + s->lay.codes;
    a.seg_off = reinterpret_cast<const uint64_t*>(s->base + s->lay.seg_off);
    a.payload = s->base + s->lay.payload;
    a.basis = s->has_basis ? reinterpret_cast<const float*>(s->base + s->lay.basis) : nullptr;
    for (int k = 0; k < 4; ++k) a.keep[k] = k < s->policy.n_keep ? s->policy.keep[k] : 0;
    a.q = q;
    a.out = out;
    a.sel = sel;
    a.sel_stride = sel_stride;
    a.sel_int = reinterpret_cast<int32_t*>(w + P.o_sel);
    a.sel_int_stride = std::max<int32_t>(P.max_T, 1);
    const int32_t* tb = reinterpret_cast<const int32_t*>(w + P.o_tab);
    a.t_n = tb;
    a.t_segbase = tb + sh.B;
    a.t_scap = tb + 2 * sh.B;
    a.t_tokbase = tb + 3 * sh.B;
    a.t_T = tb + 4 * sh.B;
    a.t_kblk = tb + 5 * sh.B;
    a.t_ablk = tb + 6 * sh.B + 1;
    a.t_bslot = tb + 7 * sh.B + 2;
    a.spw = P.spw;
    a.sgx = P.sgx;
    a.qp = reinterpret_cast<float*>(w + P.o_qp);
    a.qbar = reinterpret_cast<float*>(w + P.o_qbar);
    a.keys = reinterpret_cast<uint32_t*>(w + P.o_keys);
    a.hist = reinterpret_cast<uint32_t*>(w + P.o_hist);
    a.hcopies = P.hcopies;
    a.etiles = P.etiles;
    a.state = reinterpret_cast<uint32_t*>(w + P.o_state);
    a.L = reinterpret_cast<uint2*>(w + P.o_L);
    a.part = reinterpret_cast<float*>(w + P.o_part);
    a.achunk = P.achunk;

    // per-request tables: the first kUploadWords words ride on the prep kernel, the rest on upload launches
    int32_t* tdst = reinterpret_cast<int32_t*>(w + P.o_tab);
    if ((st = upload_words(tdst, P.tab, kUploadWords, stream))) return st;
    Upload first;
    first.dst = tdst;
    first.n = (int32_t)std::min<size_t>(kUploadWords, P.tab.size());
    std::memcpy(first.w, P.tab.data(), sizeof(int32_t) * first.n);
    if ((st = run(K_DEC_PREP, stream, [&] { return launch_dec_prep(a, first, stream); }))) return st;

    const int streams = sh.B * sh.Hkv;
    if ((st = run(K_SCORE, stream, [&] { return launch_score(a, (int)P.n_sblk, stream); }))) return st;
    if ((st = run(K_SEL_COLLECT, stream, [&] { return launch_sel_collect(a, (int)P.n_kblk, stream); }))) return st;
    if ((st = run(K_SEL_EMIT, stream, [&] { return launch_sel_emit(a, streams, stream); }))) return st;
    if ((st = run(K_ATTEND, stream, [&] { return launch_attend(a, (int)P.n_ablk, stream); }))) return st;
    if ((st = run(K_COMBINE, stream, [&] { return launch_combine(a, streams, stream); }))) return st;
    return MKV_OK;
}

mkv_status check_decode_args(const DecPlan& P, const void* q, float* out, int32_t* sel, int32_t sel_stride) {
    if (!q || !out) return fail(MKV_E_ARG, "q and out must be non-NULL");
    if (sel && sel_stride < P.max_T) return fail(MKV_E_ARG, "sel_stride %d < largest selection %d", sel_stride, P.max_T);
    return MKV_OK;
}

}  // namespace

mkv_status mkv_decode_attn(const mkv_store* s, const void* q, int32_t n_q_heads, const int32_t* T, float* out,
                           int32_t* sel, int32_t sel_stride, void* ws, size_t ws_bytes, mkv_stream_t stream_) {
    DecPlan P;
    mkv_status st = plan_decode(s, n_q_heads, T, &P);
    if (st) return st;
    if ((st = check_decode_args(P, q, out, sel, sel_stride))) return st;
    if (!ws) return fail(MKV_E_ARG, "ws is NULL");
    if (!aligned(ws)) return fail(MKV_E_ARG, "ws must be 256-byte aligned");
    if (ws_bytes < P.bytes) return fail(MKV_E_ARG, "ws_bytes %zu < required %llu", ws_bytes, (unsigned long long)P.bytes);
    return decode_run(s, q, P, out, sel, sel_stride, ws, reinterpret_cast<hipStream_t>(stream_));
}

size_t mkv_decode_noalloc_max_bytes(void) { return kStaticWorkspaceBytes; }

mkv_status mkv_decode_attn_noalloc(const mkv_store* s, const void* q, int32_t n_q_heads, const int32_t* T,
                                   float* out, int32_t* sel, int32_t sel_stride, mkv_stream_t stream_) {
    DecPlan P;
    mkv_status st = plan_decode(s, n_q_heads, T, &P);
    if (st) return st;
    if ((st = check_decode_args(P, q, out, sel, sel_stride))) return st;
    if (P.bytes > kStaticWorkspaceBytes)
        return fail(MKV_E_ARG, "this decode needs %llu bytes of workspace, above the %llu bytes the library keeps on "
                    "each device; call mkv_decode_attn with a caller workspace", (unsigned long long)P.bytes,
                    (unsigned long long)kStaticWorkspaceBytes);
    void* ws = nullptr;
    const hipError_t e = static_workspace(&ws);
    if (e != hipSuccess) return fail(MKV_E_DEVICE, "device-resident workspace unavailable: %s", hipGetErrorString(e));
    return decode_run(s, q, P, out, sel, sel_stride, ws, reinterpret_cast<hipStream_t>(stream_));
}

// ---- uncompressed baseline --------------------------------------------------------------------------------
namespace {

struct DensePlan {
    int32_t G = 0;
    std::vector<int32_t> tab;    // n | tok0 | T (= n) | first workgroup [B+1]
    int64_t n_blk = 0;
    int32_t cpw = 1;             // 512-token chunks per workgroup
    uint64_t o_tab = 0, o_part = 0, bytes = 0;
};

mkv_status plan_dense(const mkv_kv_desc* kv, int32_t n_q_heads, bool need_data, Shape* sh, DensePlan* P) {
    mkv_status st = check_kv(kv, need_data, sh);
    if (st) return st;
    if (sh->dtype != MKV_BF16) return fail(MKV_E_UNSUPPORTED, "the uncompressed baseline takes bf16 K/V only");
    if (n_q_heads < 1 || n_q_heads % sh->Hkv != 0)
        return fail(MKV_E_ARG, "n_q_heads (%d) must be a positive multiple of n_kv_heads (%d)", n_q_heads, sh->Hkv);
    P->G = n_q_heads / sh->Hkv;
    if (P->G != 1 && P->G != 2 && P->G != 4 && P->G != 8)
        return fail(MKV_E_UNSUPPORTED, "query heads per KV head must be 1, 2, 4 or 8 (got %d)", P->G);
    const int B = sh->B;
    P->tab.assign(4 * B + 1, 0);
    // chunks per workgroup: up to 8 while the grid keeps about 2048 workgroups (8 per CU), so that long
    // contexts leave few partials for the combine
    int64_t chunks = 0;
    for (int r = 0; r < B; ++r) chunks += (int64_t)sh->Hkv * cdiv(sh->cu[r + 1] - sh->cu[r], kDenseChunk);
    P->cpw = (int32_t)std::max<int64_t>(1, std::min<int64_t>(8, chunks / 2048));
    int64_t blk = 0;
    for (int r = 0; r < B; ++r) {
        const int64_t n = sh->cu[r + 1] - sh->cu[r];
        P->tab[r] = (int32_t)n;
        P->tab[B + r] = (int32_t)sh->cu[r];
        P->tab[2 * B + r] = (int32_t)n;
        P->tab[3 * B + r] = (int32_t)blk;
        blk += (int64_t)sh->Hkv * cdiv(n, (int64_t)kDenseChunk * P->cpw);
    }
    P->tab[4 * B] = (int32_t)blk;
    if (blk > INT32_MAX) return fail(MKV_E_UNSUPPORTED, "too many workgroups");
    P->n_blk = blk;
    P->o_tab = 0;
    P->o_part = align_up(4 * P->tab.size());
    P->bytes = align_up(P->o_part + 4ull * std::max<int64_t>(blk, 1) * P->G * (MKV_HEAD_DIM + 2));
    return MKV_OK;
}

}  // namespace

mkv_status mkv_dense_decode_workspace_bytes(const mkv_kv_desc* kv, int32_t n_q_heads, size_t* ws_bytes) {
    Shape sh;
    DensePlan P;
    mkv_status st = plan_dense(kv, n_q_heads, false, &sh, &P);
    if (st) return st;
    if (!ws_bytes) return fail(MKV_E_ARG, "ws_bytes is NULL");
    *ws_bytes = P.bytes;
    return MKV_OK;
}

mkv_status mkv_dense_decode_attn(const mkv_kv_desc* kv, const void* q, int32_t n_q_heads, float* out, void* ws,
                                 size_t ws_bytes, mkv_stream_t stream_) {
    hipStream_t stream = reinterpret_cast<hipStream_t>(stream_);
    Shape sh;
    DensePlan P;
    mkv_status st = plan_dense(kv, n_q_heads, true, &sh, &P);
    if (st) return st;
    if (!q || !out) return fail(MKV_E_ARG, "q and out must be non-NULL");
    if (!ws) return fail(MKV_E_ARG, "ws is NULL");
    if (!aligned(ws)) return fail(MKV_E_ARG, "ws must be 256-byte aligned");
    if (ws_bytes < P.bytes) return fail(MKV_E_ARG, "ws_bytes %zu < required %llu", ws_bytes, (unsigned long long)P.bytes);
    uint8_t* w = static_cast<uint8_t*>(ws);
    int32_t* tb = reinterpret_cast<int32_t*>(w + P.o_tab);
    if ((st = upload_words(tb, P.tab, 0, stream))) return st;
    const int B = sh.B;
    DenseArgs d;
    d.B = B;
    d.Hkv = sh.Hkv;
    d.G = P.G;
    d.cpw = P.cpw;
    d.K = static_cast<const uint16_t*>(kv->K);
    d.V = static_cast<const uint16_t*>(kv->V);
    d.q = static_cast<const uint16_t*>(q);
    d.t_n = tb;
    d.t_tok0 = tb + B;
    d.t_dblk = tb + 3 * B;
    d.part = reinterpret_cast<float*>(w + P.o_part);
    if ((st = run(K_DENSE_ATTEND, stream, [&] { return launch_dense_attend(d, (int)P.n_blk, stream); }))) return st;
    DecArgs a;
    std::memset(&a, 0, sizeof a);
    a.B = B;
    a.Hkv = sh.Hkv;
    a.G = P.G;
    a.out = out;
    a.t_n = tb;
    a.t_T = tb + 2 * B;
    a.t_ablk = tb + 3 * B;
    a.part = d.part;
    a.achunk = kDenseChunk * P.cpw;   // tokens per partial
    if ((st = run(K_DENSE_COMBINE, stream, [&] { return launch_combine(a, B * sh.Hkv, stream); }))) return st;
    return MKV_OK;
}

// ---- Gram matrices for basis refresh ----------------------------------------------------------------------
namespace {

struct GramPlan {
    std::vector<int32_t> tab;    // n | tok0 | first workgroup [B+1]
    int64_t n_blk = 0;
    uint64_t o_tab = 0, o_part = 0, bytes = 0;
};

mkv_status plan_gram(const mkv_kv_desc* kv, bool need_data, Shape* sh, GramPlan* P) {
    mkv_status st = check_kv(kv, need_data, sh);
    if (st) return st;
    if (sh->dtype != MKV_BF16) return fail(MKV_E_UNSUPPORTED, "the Gram matrices take bf16 K/V only");
    const int B = sh->B;
    P->tab.assign(3 * B + 1, 0);
    int64_t blk = 0;
    for (int r = 0; r < B; ++r) {
        const int64_t n = sh->cu[r + 1] - sh->cu[r];
        P->tab[r] = (int32_t)n;
        P->tab[B + r] = (int32_t)sh->cu[r];
        P->tab[2 * B + r] = (int32_t)blk;
        blk += 2ll * sh->Hkv * cdiv(n, kGramChunk);
    }
    P->tab[3 * B] = (int32_t)blk;
    if (blk > INT32_MAX || 32ll * B * sh->Hkv > INT32_MAX) return fail(MKV_E_UNSUPPORTED, "too many workgroups");
    P->n_blk = blk;
    P->o_part = align_up(4 * P->tab.size());
    P->bytes = align_up(P->o_part + 4ull * MKV_HEAD_DIM * MKV_HEAD_DIM * std::max<int64_t>(blk, 1));
    return MKV_OK;
}

}  // namespace

mkv_status mkv_gram_workspace_bytes(const mkv_kv_desc* kv, size_t* ws_bytes) {
    Shape sh;
    GramPlan P;
    mkv_status st = plan_gram(kv, false, &sh, &P);
    if (st) return st;
    if (!ws_bytes) return fail(MKV_E_ARG, "ws_bytes is NULL");
    *ws_bytes = P.bytes;
    return MKV_OK;
}

mkv_status mkv_gram(const mkv_kv_desc* kv, float* gram, void* ws, size_t ws_bytes, mkv_stream_t stream_) {
    hipStream_t stream = reinterpret_cast<hipStream_t>(stream_);
    Shape sh;
    GramPlan P;
    mkv_status st = plan_gram(kv, true, &sh, &P);
    if (st) return st;
    if (!gram) return fail(MKV_E_ARG, "gram is NULL");
    if (!ws) return fail(MKV_E_ARG, "ws is NULL");
    if (!aligned(ws) || !aligned(gram)) return fail(MKV_E_ARG, "ws and gram must be 256-byte aligned");
    if (ws_bytes < P.bytes) return fail(MKV_E_ARG, "ws_bytes %zu < required %llu", ws_bytes, (unsigned long long)P.bytes);
    uint8_t* w = static_cast<uint8_t*>(ws);
    int32_t* tb = reinterpret_cast<int32_t*>(w + P.o_tab);
    if ((st = upload_words(tb, P.tab, 0, stream))) return st;
    const int B = sh.B;
    GramArgs g;
    g.B = B;
    g.Hkv = sh.Hkv;
    g.K = static_cast<const uint16_t*>(kv->K);
    g.V = static_cast<const uint16_t*>(kv->V);
    g.t_n = tb;
    g.t_tok0 = tb + B;
    g.t_gblk = tb + 2 * B;
    g.part = reinterpret_cast<float*>(w + P.o_part);
    g.gram = gram;
    if ((st = run(K_GRAM, stream, [&] { return launch_gram(g, (int)P.n_blk, stream); }))) return st;
    if ((st = run(K_GRAM_REDUCE, stream, [&] { return launch_gram_reduce(g, stream); }))) return st;
    return MKV_OK;
}

// ---- profiling --------------------------------------------------------------------------------------------
mkv_status mkv_profile_start(int32_t max_launches, uint32_t kernel_mask) {
    if (max_launches < 0) return fail(MKV_E_ARG, "max_launches must be >= 0");
    std::lock_guard<std::mutex> lk(g_prof.mu);
    g_prof.recs.clear();
    g_prof.used = 0;
    g_prof.max_launches = max_launches;
    g_prof.mask = kernel_mask;
    g_prof.on = true;
    return MKV_OK;
}

mkv_status mkv_profile_stop(double* total_ms, int32_t* launches) {
    std::lock_guard<std::mutex> lk(g_prof.mu);
    g_prof.on = false;
    if (total_ms) for (int i = 0; i < MKV_PROFILE_KERNELS; ++i) total_ms[i] = 0.0;
    if (launches) for (int i = 0; i < MKV_PROFILE_KERNELS; ++i) launches[i] = 0;
    mkv_status st = MKV_OK;
    for (const auto& r : g_prof.recs) {
        float ms = 0.f;
        hipError_t e = hipEventSynchronize(r.b);
        if (e == hipSuccess) e = hipEventElapsedTime(&ms, r.a, r.b);
        if (e != hipSuccess) { st = fail(MKV_E_DEVICE, "event timing failed: %s", hipGetErrorString(e)); continue; }
        if (total_ms) total_ms[r.kid] += ms;
        if (launches) launches[r.kid] += 1;
    }
    g_prof.recs.clear();
    g_prof.used = 0;
    return st;
}

const char* mkv_kernel_name(int32_t id) {
    if (id < 0 || id >= K_COUNT) return nullptr;
    return kKernelNames[id];
}

}  // extern "C"
