// Internal interface between the host entry points (api.cpp) and the gfx950 kernels.
#pragma once
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mkv {

// Kernel timing: while the host times a launch it sets these events (thread-local, for exactly one launch), and the
// launch hands them to the dispatch itself (hipExtLaunchKernel), so timing adds no marker packets to the stream.
struct LaunchEvents {
    hipEvent_t start = nullptr, stop = nullptr;
    bool used = false;
};
LaunchEvents& launch_events();

template <typename... KArgs, typename... Args>
inline void launch_kernel(void (*kernel)(KArgs...), dim3 grid, dim3 block, uint32_t lds, hipStream_t s,
                          Args... args) {
    LaunchEvents& ev = launch_events();
    if (ev.start && !ev.used) {
        ev.used = true;
        hipExtLaunchKernelGGL(kernel, grid, block, lds, s, ev.start, ev.stop, 0u, args...);
    } else {
        hipLaunchKernelGGL(kernel, grid, block, lds, s, args...);
    }
}

constexpr int kUploadWords = 448;       // int32 words a table upload carries in its kernel arguments
constexpr int kHistBins = 4096;         // first radix level of the top-T select: key bits [31:20]
constexpr int kMaxHistCopies = 8;      // copies of each stream's histograms (spreads the score kernel's atomics)
constexpr int kCoarseOff = 64;          // coarse histograms (top 6 key bits, 64 bins per copy) inside the state words
constexpr int kStateWords = kCoarseOff + 64 * kMaxHistCopies;   // per (request, KV head) selection state
constexpr int kKeysPerBlock = 4096;     // keys per workgroup in the selection passes
constexpr int kAttnChunk = 256;         // selected tokens per attention workgroup (at most; 128 or 64 for small grids)
constexpr int kAttnSlots = 1024;        // attention workgroups resident at once (4 per CU)
constexpr int kEmitTileTokens = 32768;  // tokens per workgroup of the selection's emit kernel
constexpr int kDenseChunk = 512;        // tokens per workgroup of the uncompressed baseline
constexpr int kGramChunk = 16384;       // tokens per workgroup of the Gram matrices

// selection state words
enum { ST_P1 = 1, ST_NGT = 2, ST_NCAND = 3, ST_NEED = 4, ST_GTFILL = 5, ST_CFILL = 6 };

struct Upload {
    int32_t* dst;
    int32_t n;
    int32_t w[kUploadWords];
};

// ---- compression --------------------------------------------------------------------------------------
struct CmpArgs {
    const void* K;
    const void* V;
    const float* basis;         // [B][Hkv][2][128][128] or null (inputs already rotated)
    const int32_t* tab;         // tok_base[B] | n[B] | seg_base[B] | slots per stream[B] | cblk_base[B+1] | open slot[B]
    int32_t B, Hkv, spw, nblk;  // spw: segments per workgroup; nblk: workgroups per tensor
    int64_t S;                  // segments per tensor
    int64_t total_tokens;
    uint8_t* codes;             // [2][S]
    uint64_t* seg_off;          // [2][S]: byte offsets of the segments in the payload (written by the pack pass)
    uint8_t* payload;
    uint16_t* thr;              // [2][total_tokens][Hkv][4] per-vector magnitude thresholds (scratch)
    uint64_t* wg_total;         // [2*nblk] payload bytes of each workgroup's segments, then their offsets
    int32_t keep[4];
    int32_t n_keep;
    double frac;
    uint16_t* open_rows;        // growable stores: original rows of each stream's open segment (else null), by
                                // open slot (the request's index, or its id in a pool)
    int64_t open_elems;         // elements per stream in open_rows
    int32_t preplaced;          // pack: seg_off already holds every segment's payload offset (paged pools)
    uint64_t* total;            // one pass: payload bytes in use (zero before the launch; each workgroup adds)
};

// Paged pools: placement of the segments of the requests being added (tab as in CmpArgs).
struct PoolArgs {
    const int32_t* tab;
    int32_t B, Hkv, bv;
    int64_t S;
    int32_t keep[4];
    const uint8_t* codes;
    uint64_t* seg_off;
    uint64_t page_bytes;
    int32_t* pages;             // [2*B*Hkv] pages each stream needs (place)
    uint64_t* used;             // [2*B*Hkv] payload bytes of each stream (place)
    const int32_t* list_base;   // [2*B*Hkv] first entry of each stream in page_ids (fix)
    const int32_t* page_ids;    // page of each (stream, ordinal) (fix)
};

// One token appended to each listed request of a growable bf16 store or pool.
struct AppendArgs {
    const uint16_t* Kn;         // [rows][Hkv][128]
    const uint16_t* Vn;
    const float* basis;         // the store's copy, or null; indexed by open slot
    const int32_t* tab;         // per listed request: row of Kn/Vn | its tokens before the append | Hkv * seg_base |
                                // slots per stream | open slot (open areas and basis)
    const uint64_t* seal_off;   // [listed][2*Hkv] payload offset of a segment the append completes (pools), or null:
                                // taken from the payload counter
    int32_t Hkv;
    int64_t S;                  // segment slots per tensor
    uint8_t* codes;
    uint64_t* seg_off;
    uint8_t* payload;
    uint64_t open_pack;         // offset (from payload) of the per-stream packed open segments
    uint64_t open_bytes;        // bytes per stream of open_pack and of open_rows
    uint16_t* open_rows;
    unsigned long long* total;  // payload bytes in use (header)
};

hipError_t launch_upload(const Upload& u, hipStream_t s);
hipError_t launch_cmp_append(const CmpArgs& a, const AppendArgs& x, int n_requests, hipStream_t s);
hipError_t launch_cmp_decide(const CmpArgs& a, int dtype, hipStream_t s);
hipError_t launch_cmp_scan(uint64_t* wg_total, int64_t count, uint64_t* total, hipStream_t s);
hipError_t launch_cmp_pack(const CmpArgs& a, int dtype, hipStream_t s);
hipError_t launch_cmp_fused(const CmpArgs& a, hipStream_t s);
hipError_t launch_pool_place(const PoolArgs& p, int n_streams, hipStream_t s);
hipError_t launch_pool_fix(const PoolArgs& p, int n_streams, hipStream_t s);

// ---- decode -------------------------------------------------------------------------------------------
struct DecArgs {
    int32_t B, Hkv, G, dtype;
    int64_t S;
    const uint8_t* codes;
    const uint64_t* seg_off;
    const uint8_t* payload;
    const float* basis;         // store's copy or null
    int32_t keep[4];
    const void* q;
    float* out;
    int32_t* sel;               // user buffer or null
    int32_t sel_stride;
    int32_t* sel_int;           // internal selection lists [B*Hkv][sel_int_stride]
    int32_t sel_int_stride;
    // per-request tables (device): n | seg_base | segment slots per stream | key base (sum of earlier contexts
    // padded to 64 tokens) | T_eff | kblk_base | ablk_base
    const int32_t* t_n;
    const int32_t* t_segbase;
    const int32_t* t_scap;
    const int32_t* t_tokbase;
    const int32_t* t_T;
    const int32_t* t_kblk;
    const int32_t* t_ablk;
    const int32_t* t_bslot;     // basis slot of each request (its index unless the store is a pool view)
    int32_t spw;                // segments per score workgroup (a multiple of 4)
    int32_t sgx;                // score workgroups per stream in the grid (the most any request needs)
    float* qp;                  // [B][Hq][128]
    float* qbar;                // [B][Hkv][128]
    uint32_t* keys;             // [Hkv * sum of contexts padded to 64 tokens]
    uint32_t* hist;             // [B*Hkv][hcopies][4096]
    uint32_t* state;            // [B*Hkv][kStateWords]
    int32_t hcopies;            // histogram copies per stream (a power of two <= kMaxHistCopies)
    int32_t etiles;             // emit workgroups per stream: tiles of 32768 tokens of the longest context
    uint2* L;                   // same indexing as keys: taken tokens, then candidates, as (token index, key)
    float* part;                // [n_ablk][G][130]
    int32_t achunk;             // tokens per attention partial: 256, 128 or 64 (the combine kernel's chunk)
};

hipError_t launch_dec_prep(const DecArgs& a, const Upload& tab, hipStream_t s);
hipError_t launch_score(const DecArgs& a, int n_blocks, hipStream_t s);
hipError_t launch_sel_collect(const DecArgs& a, int n_blocks, hipStream_t s);
hipError_t launch_sel_emit(const DecArgs& a, int n_streams, hipStream_t s);
hipError_t launch_attend(const DecArgs& a, int n_blocks, hipStream_t s);
hipError_t launch_combine(const DecArgs& a, int n_streams, hipStream_t s);

// ---- uncompressed baseline ------------------------------------------------------------------------------
struct DenseArgs {
    int32_t B, Hkv, G;
    int32_t cpw;                // chunks of kDenseChunk tokens per workgroup (1..8)
    const uint16_t* K;          // bf16 [tokens][Hkv][128]
    const uint16_t* V;
    const uint16_t* q;          // bf16 [B][Hq][128]
    const int32_t* t_n;         // per request: context
    const int32_t* t_tok0;      // per request: first token
    const int32_t* t_dblk;      // [B+1] first workgroup of each request (Hkv * workgroups per request)
    float* part;                // [blocks][G][130]
};

hipError_t launch_dense_attend(const DenseArgs& a, int n_blocks, hipStream_t s);

// ---- Gram matrices for basis refresh --------------------------------------------------------------------
struct GramArgs {
    int32_t B, Hkv;
    const uint16_t* K;          // bf16 [tokens][Hkv][128]
    const uint16_t* V;
    const int32_t* t_n;         // per request: context
    const int32_t* t_tok0;      // per request: first token
    const int32_t* t_gblk;      // [B+1] first workgroup of each request (Hkv * 2 * chunks per request)
    float* part;                // [blocks][128][128] per-chunk partials
    float* gram;                // [B][Hkv][2][128][128]
};

hipError_t launch_gram(const GramArgs& a, int n_blocks, hipStream_t s);
hipError_t launch_gram_reduce(const GramArgs& a, hipStream_t s);

// ---- device-resident decode workspace (noalloc.hip) ------------------------------------------------------
constexpr uint64_t kStaticWorkspaceBytes = 128ull << 20;   // 128 MiB per device
// Device address of the current device's copy (looked up on the first call per device, then kept).
hipError_t static_workspace(void** ptr);

}  // namespace mkv
