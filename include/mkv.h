/*
 * mkv.h -- C ABI of a MosaicKV-style compressed KV cache for AMD MI355X (gfx950).
 *
 * Method: arXiv 2607.00760, "MosaicKV: Serving Long-Context LLM with Dynamic Two-D KV Cache Compression".
 *   - dynamic two-D compression (section 1, Observation & Approach 1): keys and values are rotated by an SVD
 *     basis, every KV vector keeps its own most important channels, and the cache is cut into segments that
 *     each get their own compression strategy;
 *   - compact sparse attention (section 1, Observation & Approach 2): the sparse cache is packed into a dense
 *     format in GPU memory and attention runs on it without unpacking;
 *   - query-aware token selection at run time (section 1, the paragraph on prior sequence compression), kept
 *     together with channel compression through selection and attention (section 1, Challenge 1).
 * The pages fix no numbers for segments, strategies or budgets; this library takes: 64-token segments, kept
 * channel counts {128, 64, 32} chosen per segment as the smallest count that keeps >= 90% of every vector's
 * squared L2 norm, equal magnitudes broken toward the lower channel index, and a per-request token budget T.
 *
 * Conventions for every call:
 *   - [host] pointers are CPU memory read during the call only; [dev] pointers are HIP device memory of the
 *     current device.
 *   - The caller allocates all device memory (store, scratch, workspace, outputs); the library never calls
 *     hipMalloc/hipFree.  Sizes come from the *_bytes calls.  (One exception for callers that cannot allocate:
 *     mkv_decode_attn_noalloc uses a workspace array held in the library's own code object.)
 *   - Device work is enqueued on the given stream and is asynchronous unless a call says it synchronises.
 *   - Every argument check runs on the host before anything is enqueued; on failure nothing is launched, the
 *     call returns MKV_E_ARG or MKV_E_UNSUPPORTED and mkv_last_error() says why.  A failed launch returns
 *     MKV_E_DEVICE.  No C++ exception crosses this boundary.
 *   - Preconditions not checked: finite inputs (NaN/Inf give unspecified results) and an orthonormal basis.
 *     The rotation and the decode arithmetic run in float32 (the segment energy rule in float64, exact for
 *     every bf16 value): rotated values, scores and logits must stay inside the float32 range.
 */
#ifndef MKV_H
#define MKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* mkv_stream_t; /* a hipStream_t; NULL is the legacy default stream */

typedef enum {
    MKV_OK = 0,
    MKV_E_ARG = 1,          /* invalid argument, shape, or undersized buffer */
    MKV_E_UNSUPPORTED = 2,  /* valid but not supported by this build (e.g. head_dim != 128) */
    MKV_E_DEVICE = 3        /* a HIP call or kernel launch failed */
} mkv_status;

typedef enum { MKV_FP32 = 0, MKV_BF16 = 1 } mkv_dtype;

#define MKV_HEAD_DIM 128
#define MKV_SEG_LEN 64
#define MKV_MAX_KEEP 4
#define MKV_MAX_GROUP 8        /* query heads per KV head */

/* Compression strategy set (the pages' "compression strategy" per KV-cache segment).
 * keep[0..n_keep) are kept-channel counts, strictly decreasing, keep[0] == 128, each in {128, 64, 32, 16}.
 * A vector admits count c when the sum of squares of its c largest-magnitude stored values is
 * >= energy_frac * (sum of squares of all its stored values), both sums in float64.  A segment takes the
 * smallest count every vector in it admits; its code is that count's index in keep[]. */
typedef struct {
    int32_t seg_len;      /* must be 64 */
    int32_t n_keep;       /* 1..4 */
    int32_t keep[MKV_MAX_KEEP];
    double energy_frac;   /* in (0, 1]; default 0.9 */
} mkv_seg_policy;

/* Shape of a batch of per-request KV caches for one layer. */
typedef struct {
    int32_t batch;               /* requests, >= 1 */
    int32_t n_kv_heads;          /* >= 1 */
    int32_t head_dim;            /* must be 128 */
    mkv_dtype dtype;             /* storage dtype of K, V, q and of the packed values */
    const int64_t* cu_seqlens;   /* [host] [batch+1], cu_seqlens[0] == 0, non-decreasing; request r owns tokens
                                    [cu_seqlens[r], cu_seqlens[r+1]) (a request may be empty) */
    const void* K;               /* [dev] [cu_seqlens[batch]][n_kv_heads][128] token-major, contiguous */
    const void* V;               /* [dev] same layout as K */
} mkv_kv_desc;

typedef struct mkv_store mkv_store;   /* opaque host handle */

/* Fills *policy with the default strategy set: seg_len 64, keep {128, 64, 32}, energy_frac 0.9. */
void mkv_default_policy(mkv_seg_policy* policy);

/* Worst-case store size (every segment at 128 channels; for bf16, every segment slot at 64 tokens) and the
 * scratch size mkv_compress needs.  Host-only; enqueues nothing. */
mkv_status mkv_compress_bytes(const mkv_kv_desc* kv, const mkv_seg_policy* policy,
                              size_t* store_bytes, size_t* scratch_bytes);

/* Dynamic two-D compression of K and V (section 1, Observation & Approach 1 of the pages).
 *   basis   [dev] float32 [batch][n_kv_heads][2][128][128] (index 2: 0 = K basis, 1 = V basis), row-major,
 *           columns are basis vectors: a stored vector is round_dtype(x @ B).  NULL: K and V are already rotated
 *           (they are stored as given) and decode applies no query/output rotation.  The store keeps a copy.
 *   store_buf [dev] >= store_bytes from mkv_compress_bytes, 256-byte aligned; the handle points into it, so it
 *           must outlive the handle.  scratch [dev] >= scratch_bytes, 256-byte aligned, free after the call.
 *   On success *out receives a new handle (release with mkv_store_destroy).  The packing runs asynchronously on
 *   `stream`; decode calls enqueued after it on the same stream see the finished store.
 * Store layout (all offsets from store_buf, see mkv_store_view): a segment is 64 consecutive tokens of one
 * (request r, KV head h, tensor X) stream from token 0 on, the last one shorter when n_r % 64 != 0.  Segments
 * are numbered X*S + n_kv_heads*seg_base[r] + h*S_r + s with S_r = ceil(cap_r/64), seg_base[r] = sum_{r'<r} S_r',
 * S = n_kv_heads * sum_r S_r, where cap_r is request r's token capacity (its context n_r, unless the store is
 * growable; slots past the context are unused).  Segment g has a uint8 code (index into policy.keep, c = keep[code]) and a uint64
 * byte offset into the payload; its payload is [n_s][c] values of the storage dtype, followed, when c < 128, by
 * [n_s][c] uint8 channel indices; each token's channels are in ascending order and values follow that order.
 * Segments never overlap and lie inside payload_capacity; the payload total counts their bytes.  Placement: a
 * bf16 store without capacities is compressed in one pass, each workgroup writing its run of consecutive
 * segments of one stream back to back from the run's first slot at full size (slot g at byte g * 64*128*2, so
 * unused bytes lie between runs); other stores hold all segments back to back in slot order. */
mkv_status mkv_compress(const mkv_kv_desc* kv, const float* basis, const mkv_seg_policy* policy,
                        void* store_buf, size_t store_bytes, void* scratch, size_t scratch_bytes,
                        mkv_stream_t stream, mkv_store** out);

/* ---- growing stores (incremental append) ---------------------------------------------------------------
 * A growable store keeps room for tokens appended while decoding: segment slots and packed-payload room for
 * capacity[r] >= n_r tokens of each request (host [batch]), and for every (request, KV head, tensor) stream an
 * open-segment area holding the original rows of its last, unfinished segment and that segment's packed form.
 * The pages keep newly generated KV vectors in a GPU-side buffer and fold them into the compressed cache off
 * the critical path (section 1, Observation & Approach 2).  Here each append re-compresses the stream's open
 * segment by the segment rule over its tokens so far (same rotation, selection and packing as mkv_compress),
 * and the append that completes a segment (64 tokens) seals it into the payload.  After any sequence of
 * appends, every segment holds exactly what mkv_compress would build from the extended contexts: the same
 * code, channels and values; only payload offsets differ.  The payload has room for the capacities at all 128
 * channels plus, per stream, the first compression's copy of its unfinished segment, which appends leave unused.
 * bf16 only (MKV_E_UNSUPPORTED otherwise).
 * mkv_compress_growable is mkv_compress with capacities; the sizes come from mkv_compress_bytes_growable. */
mkv_status mkv_compress_bytes_growable(const mkv_kv_desc* kv, const mkv_seg_policy* policy, const int64_t* capacity,
                                       size_t* store_bytes, size_t* scratch_bytes);
mkv_status mkv_compress_growable(const mkv_kv_desc* kv, const float* basis, const mkv_seg_policy* policy,
                                 const int64_t* capacity, void* store_buf, size_t store_bytes, void* scratch,
                                 size_t scratch_bytes, mkv_stream_t stream, mkv_store** out);

/* Appends one token to every request r with active[r] != 0 (active: [host] [batch], or NULL for every request):
 * K_new[r][h] and V_new[r][h] ([dev] [batch][n_kv_heads][128] bf16, unrotated like the K/V given to
 * mkv_compress) become token n_r of request r, and the handle's contexts advance.  Fails with MKV_E_ARG before
 * enqueueing anything if the store is not growable or a listed request is at its capacity.  Work is enqueued
 * on `stream`; decode calls enqueued after it on the same stream see the new tokens.  Calls that overlap on one
 * store race.  ws [dev] >= mkv_append_workspace_bytes, 256-byte aligned. */
mkv_status mkv_append_workspace_bytes(const mkv_store* store, size_t* ws_bytes);
mkv_status mkv_append(mkv_store* store, const void* K_new, const void* V_new, const int32_t* active, void* ws,
                      size_t ws_bytes, mkv_stream_t stream);

/* Wraps a handle around a store buffer that already holds a store of the documented layout for this shape
 * (e.g. one restored from a file or written by a test).  kv->K and kv->V are ignored.  has_basis says whether
 * the buffer's basis region is valid.  Enqueues nothing. */
mkv_status mkv_store_attach(const mkv_kv_desc* kv, const mkv_seg_policy* policy, int32_t has_basis,
                            void* store_buf, size_t store_bytes, mkv_store** out);

typedef struct {
    int32_t batch, n_kv_heads, head_dim;
    mkv_dtype dtype;
    mkv_seg_policy policy;
    int32_t has_basis;
    int64_t total_tokens;        /* cu_seqlens[batch] */
    int64_t segments_per_tensor; /* S above */
    const int64_t* cu_seqlens;   /* [host] owned by the handle */
    void* codes;                 /* [dev] uint8 [2][S] */
    void* seg_off;               /* [dev] uint64 [2][S], byte offsets into payload */
    void* basis;                 /* [dev] float32 [batch][n_kv_heads][2][128][128], or NULL */
    void* payload;               /* [dev] */
    void* payload_total;         /* [dev] uint64: payload bytes in use, written by mkv_compress */
    uint64_t payload_capacity;   /* bytes available at payload */
    uint64_t store_bytes;        /* bytes of the whole store buffer */
    const int64_t* cu_capacity;  /* [host] [batch+1] prefix sums of the token capacities; segment slots follow
                                    them (equal to cu_seqlens unless the store is growable) */
    int32_t growable;            /* built with mkv_compress_growable: accepts mkv_append */
    const int32_t* seg_base;     /* [host] [batch] seg_base[r] of the segment numbering above */
    const int32_t* seg_slots;    /* [host] [batch] S_r of the segment numbering above */
    const int32_t* basis_slot;   /* [host] [batch] request r's bases are basis[basis_slot[r]] (r, unless a pool view) */
    int32_t pool_view;           /* made by mkv_pool_view: the buffer regions above are the pool's */
} mkv_store_info;

/* Device addresses and host metadata of a store (for tests, export, and custom consumers). */
mkv_status mkv_store_view(const mkv_store* store, mkv_store_info* info);

/* Payload bytes in use (sum over all segments of both tensors).  SYNCHRONISES `stream`. */
mkv_status mkv_store_payload_bytes(const mkv_store* store, mkv_stream_t stream, uint64_t* bytes);

/* Frees the host handle only (the store buffer stays the caller's). NULL is accepted. */
mkv_status mkv_store_destroy(mkv_store* store);

/* Workspace bytes mkv_decode_attn needs for this store, query head count and budgets T [host] [batch]. */
mkv_status mkv_decode_workspace_bytes(const mkv_store* store, int32_t n_q_heads, const int32_t* T,
                                      size_t* ws_bytes);

/* One decode step of attention over the compressed store (section 1 of the pages: query-aware token
 * selection, then compact sparse attention without unpacking).  For request r and KV head g:
 *   q'_h = q_h @ B_K for the query heads h of group g (h / (n_q_heads/n_kv_heads) == g);
 *   Qbar = sum of the group's q'_h;  score_j = sum over token j's stored channels i of Qbar_i * k_j,i;
 *   Sel = the min(T[r], n_r) tokens of largest score (equal scores: lower token index first);
 *   out_h = (sum_{j in Sel} softmax_j(q'_h . k_j / sqrt(128)) * v_j) @ B_V^T  (dropped channels count as 0).
 *   q    [dev] [batch][n_q_heads][128] in the store's dtype; n_q_heads a multiple of n_kv_heads, group <= 8.
 *   T    [host] [batch], each >= 1 (values above n_r select every token).
 *   out  [dev] float32 [batch][n_q_heads][128]; an empty request (n_r == 0) gets zeros.
 *   sel  [dev] int32 [batch][n_kv_heads][sel_stride] or NULL: the selected token indices of each (r, g) in
 *        ascending order, -1 after the first min(T[r], n_r) entries; sel_stride >= max_r min(T[r], n_r).
 *   ws   [dev] >= mkv_decode_workspace_bytes, 256-byte aligned; contents are scratch.
 * Concurrent calls on different streams may share one store if each has its own workspace. */
mkv_status mkv_decode_attn(const mkv_store* store, const void* q, int32_t n_q_heads, const int32_t* T,
                           float* out, int32_t* sel, int32_t sel_stride, void* ws, size_t ws_bytes,
                           mkv_stream_t stream);

/* mkv_decode_attn without a caller workspace, for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc).  The workspace is a device-resident array
 * inside the library, mkv_decode_noalloc_max_bytes() = 128 MiB on each device the library is loaded on (held
 * until the process ends; that covers 8 x 131072 or 1 x 1048576 tokens at 8 KV heads); a call whose
 * mkv_decode_workspace_bytes exceeds it fails with MKV_E_ARG before anything is enqueued.  No device memory is
 * allocated or freed.  Every call on one device uses that device's one array, so calls that overlap on one GPU
 * (different streams or threads without ordering) race; calls ordered on one stream do not.  The array's
 * contents are scratch: each call clears what it needs.  Arguments and results as for mkv_decode_attn. */
size_t mkv_decode_noalloc_max_bytes(void);
mkv_status mkv_decode_attn_noalloc(const mkv_store* store, const void* q, int32_t n_q_heads, const int32_t* T,
                                   float* out, int32_t* sel, int32_t sel_stride, mkv_stream_t stream);

/* ---- paged pools -------------------------------------------------------------------------------------------
 * A pool holds the compressed caches of many requests of one layer in one buffer, for serving: requests are
 * added (compressed) and removed one by one, and any list of live requests decodes together through a store
 * view.  Each request's packed segments go into fixed-size pages taken from a free list, so removing a request
 * returns its pages and later requests reuse them without moving anyone's data; pages follow the compressed
 * size, so the pool holds as many requests as their compressed bytes allow.  Within a page, a stream's
 * segments are whole and in order (a segment never straddles two pages).  Every segment holds exactly what
 * mkv_compress would build for the same request (same code, channels and values); only payload offsets differ,
 * and decode over a view equals decode over a store of the same requests.
 * Pool buffer layout (offsets from pool_buf): header, codes uint8 [2][S], seg_off uint64 [2][S] (S =
 * n_kv_heads * segment_slots), bases float32 [max_requests][n_kv_heads][2][128][128] when has_basis, then
 * n_pages pages of page_bytes, then (appendable pools) per request id, KV head and tensor an open-segment area
 * holding the unfinished last segment packed (addressed like the pages, through seg_off) and the same area's
 * original rows.  A request with id i and segment-slot run starting at u numbers its segments
 * X*S + n_kv_heads*u + h*S_r + s with S_r = ceil(cap_r/64) (cap_r: its token capacity, n_r unless it was added
 * with one), and its bases sit at basis slot i.
 * Appends (appendable bf16 pools): mkv_pool_append adds one token to each listed request exactly as
 * mkv_append does for growable stores; a segment that an append completes is sealed into a page at a position
 * the host reserves for it with the uncompressed segment size (64*128*2 bytes), taken from the request's
 * current append page (all its streams' sealed segments share it) or from a new page.
 * Ordering: the pool's host bookkeeping is not thread-safe; pool calls and decode calls on its views must be
 * ordered by the caller (one stream, or synchronisation), since removing a request lets the next add overwrite
 * its pages. */
typedef struct {
    int32_t n_kv_heads;          /* >= 1 */
    mkv_dtype dtype;
    int32_t has_basis;           /* 1: every add passes bases (kept per request); 0: K/V are added pre-rotated */
    int32_t max_requests;        /* request ids are 0 .. max_requests-1 */
    int64_t segment_slots;       /* segment slots per (KV head, tensor), shared by the live requests: a request of
                                    n tokens takes a contiguous run of ceil(n/64) */
    int64_t n_pages;             /* >= 1 */
    int64_t page_bytes;          /* multiple of 256, >= 64*128*dtype bytes (one uncompressed segment), <= 2^31 */
    int32_t appendable;          /* 1: open-segment areas for mkv_pool_append (bf16 only) */
} mkv_pool_desc;

typedef struct mkv_pool mkv_pool;   /* opaque host handle */

typedef struct {
    mkv_pool_desc desc;
    int32_t live_requests;
    int64_t free_pages;
    int64_t free_segment_slots;  /* per (KV head, tensor), over all free runs */
    int64_t largest_free_run;    /* the longest run of free segment slots */
    void* codes;                 /* [dev] the pool's regions (layout above) */
    void* seg_off;
    void* basis;                 /* NULL without bases */
    void* payload;
    uint64_t pool_bytes;
} mkv_pool_info;

/* Bytes of a pool buffer for this descriptor.  Host-only. */
mkv_status mkv_pool_bytes(const mkv_pool_desc* desc, size_t* pool_bytes);
/* Creates an empty pool over pool_buf ([dev] >= mkv_pool_bytes, 256-byte aligned; it must outlive the pool
 * and every view).  Host-only: nothing is enqueued, the buffer's contents do not matter. */
mkv_status mkv_pool_create(const mkv_pool_desc* desc, const mkv_seg_policy* policy, void* pool_buf,
                           size_t pool_bytes, mkv_pool** out);
/* Scratch bytes mkv_pool_add needs for this batch of new requests. */
mkv_status mkv_pool_add_scratch_bytes(const mkv_pool* pool, const mkv_kv_desc* kv, size_t* scratch_bytes);
/* Compresses the requests of kv (shape checks as mkv_compress; n_kv_heads and dtype must match the pool) into
 * the pool and writes their ids to ids [host] [kv->batch].  basis: as for mkv_compress, required when the pool
 * has bases and NULL otherwise; the pool keeps a copy.  capacity: [host] [kv->batch] token capacities >= the
 * contexts for later appends (appendable pools only), or NULL.  SYNCHRONISES `stream` (twice): the pages a request
 * needs depend on its kept channel counts, so they are read back after the decide pass and handed out on the
 * host.  Fails with MKV_E_ARG, leaving the pool as it was, when ids, segment slots (a contiguous run per
 * request) or pages run short; the page check comes after the decide pass has run on the device, every other
 * check before anything is enqueued.  scratch [dev] >= mkv_pool_add_scratch_bytes, 256-byte aligned. */
mkv_status mkv_pool_add(mkv_pool* pool, const mkv_kv_desc* kv, const float* basis, const int64_t* capacity,
                        void* scratch, size_t scratch_bytes, mkv_stream_t stream, int32_t* ids);
/* Appends one token to each of the n listed live requests (ids [host] [n], distinct): K_new[i][h] and
 * V_new[i][h] ([dev] [n][n_kv_heads][128] bf16, unrotated like the K/V given to mkv_pool_add) become token n_r of
 * request ids[i].  Every check (appendable pool, live ids, capacity, free pages for the segments the append
 * seals) runs on the host before anything is enqueued; on failure nothing changes.  Views made earlier keep
 * the old token counts: make a new view to decode the extended requests.  ws [dev] >=
 * mkv_pool_append_workspace_bytes(pool, n), 256-byte aligned. */
mkv_status mkv_pool_append_workspace_bytes(const mkv_pool* pool, int32_t n, size_t* ws_bytes);
mkv_status mkv_pool_append(mkv_pool* pool, int32_t n, const int32_t* ids, const void* K_new, const void* V_new,
                           void* ws, size_t ws_bytes, mkv_stream_t stream);
/* Returns the listed requests' pages, slots and ids to the pool.  Host-only: the caller makes sure no enqueued
 * work still reads them (a later add on the same stream is ordered after earlier decodes on it).  Views that
 * list a removed request must not be used again.  Unknown or repeated ids: MKV_E_ARG, nothing removed. */
mkv_status mkv_pool_remove(mkv_pool* pool, int32_t n, const int32_t* ids);
/* A store handle over the listed live requests, in this order (request r of the view is ids[r]), for
 * mkv_decode_attn, mkv_decode_workspace_bytes and mkv_store_view; release with mkv_store_destroy.  Host-only.
 * mkv_store_payload_bytes of a view is the listed requests' packed bytes (no synchronisation). */
mkv_status mkv_pool_view(const mkv_pool* pool, int32_t n, const int32_t* ids, mkv_store** out);
/* Occupancy and device regions of the pool. */
mkv_status mkv_pool_stats(const mkv_pool* pool, mkv_pool_info* info);
/* Tokens, token capacity, pages and packed payload bytes of one live request (each output pointer may be NULL;
 * sealed appended segments count with their reserved size). */
mkv_status mkv_pool_request(const mkv_pool* pool, int32_t id, int64_t* n_tokens, int64_t* capacity, int64_t* pages,
                            uint64_t* payload_bytes);
/* Frees the host handle only. NULL is accepted. */
mkv_status mkv_pool_destroy(mkv_pool* pool);

/* ---- uncompressed baseline ---------------------------------------------------------------------------------
 * Decode attention over the uncompressed bf16 K/V of the descriptor (no rotation, no channel or token
 * selection): for request r and query head h of KV head g = h / (n_q_heads/n_kv_heads),
 *   out_h = sum over all n_r tokens j of softmax_j(q_h . k_j / sqrt(128)) * v_j.
 * The pages compare their compressed attention with such an uncompressed baseline (section 1, Observation &
 * Approach 2, where uncompressed decode attention is profiled as memory-bound).
 *   kv   bf16 only (MKV_E_UNSUPPORTED otherwise); K and V [dev] as in the descriptor.
 *   q    [dev] bf16 [batch][n_q_heads][128]; n_q_heads a multiple of n_kv_heads, group of 1, 2, 4 or 8.
 *   out  [dev] float32 [batch][n_q_heads][128]; an empty request gets zeros.
 *   ws   [dev] >= mkv_dense_decode_workspace_bytes, 256-byte aligned; contents are scratch. */
mkv_status mkv_dense_decode_workspace_bytes(const mkv_kv_desc* kv, int32_t n_q_heads, size_t* ws_bytes);
mkv_status mkv_dense_decode_attn(const mkv_kv_desc* kv, const void* q, int32_t n_q_heads, float* out, void* ws,
                                 size_t ws_bytes, mkv_stream_t stream);

/* ---- basis refresh -----------------------------------------------------------------------------------------
 * Gram matrices G = X^T X of every (request, KV head, tensor) stream X of bf16 K/V.  The pages rotate the KV
 * cache by an SVD basis computed off the decoding path (section 1, Observation & Approach 1 and 2); the right
 * singular vectors of X are the eigenvectors of G, so a caller refreshes a stream's basis by decomposing G
 * (a 128 x 128 symmetric matrix) and ordering the eigenvectors by decreasing eigenvalue.
 *   kv   bf16 only (MKV_E_UNSUPPORTED otherwise); K and V [dev] as in the descriptor.
 *   gram [dev] float32 [batch][n_kv_heads][2][128][128] (K's matrix, then V's), 256-byte aligned, fully written;
 *        an empty request gets zeros.  Products of bf16 values are exact; the sums are float32 (MFMA).
 *   ws   [dev] >= mkv_gram_workspace_bytes, 256-byte aligned; contents are scratch. */
mkv_status mkv_gram_workspace_bytes(const mkv_kv_desc* kv, size_t* ws_bytes);
mkv_status mkv_gram(const mkv_kv_desc* kv, float* gram, void* ws, size_t ws_bytes, mkv_stream_t stream);

/* Text of the last error on the calling thread; valid until the next call on that thread. */
const char* mkv_last_error(void);

/* ---- kernel timing (for benchmarks) --------------------------------------------------------------------
 * While profiling is on, every kernel the library launches whose id has its bit set in kernel_mask (bit i =
 * id i, see mkv_kernel_name) is bracketed by two HIP events recorded on the launch stream; other kernels run
 * untimed, so timing one kernel adds only its own two event records to the stream.  mkv_profile_stop
 * synchronises those events and returns, per kernel id, the summed duration in milliseconds and the launch
 * count (arrays of MKV_PROFILE_KERNELS entries), then clears them.  At most max_launches launches are timed
 * per session (later launches run untimed).  Not thread-safe with respect to concurrent library calls from
 * other threads. */
#define MKV_PROFILE_KERNELS 32
mkv_status mkv_profile_start(int32_t max_launches, uint32_t kernel_mask);
mkv_status mkv_profile_stop(double* total_ms, int32_t* launches);
const char* mkv_kernel_name(int32_t kernel_id);   /* NULL when the id is unused */

#ifdef __cplusplus
}
#endif
#endif /* MKV_H */
