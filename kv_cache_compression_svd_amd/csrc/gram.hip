// Gram matrices G = X^T X of bf16 K/V streams, for refreshing the rotation bases on the device.
//
// MosaicKV rotates every KV vector by an SVD basis (§1, Observation & Approach 1) and computes the bases off
// the decoding path (Observation & Approach 2).  The right singular vectors of X are the eigenvectors of X^T X;
// this file computes X^T X with MFMA (the contraction over tokens is a dense GEMM), leaving the 128 x 128
// eigendecomposition to the host.  Workgroups take 16384-token chunks of one (request, KV head, tensor) stream
// and write a float32 partial; a second kernel sums the partials of each stream.
#include "common.cuh"
#include "kernels.h"

namespace mkv {

constexpr int kGramTile = 64;          // tokens per LDS tile
constexpr int kGramRow = 80;           // LDS row (one channel, token-contiguous) in bf16 elements: 160 bytes

// LDS position of token t of channel row: the 16-byte chunk of 8 tokens is swizzled by the row's group of 8
// channels, which spreads the transposed stores over the banks (at most 2-way) and keeps the 16-byte
// fragment reads conflict-free.
__device__ __forceinline__ int gram_pos(int row, int t) {
    return row * kGramRow + 8 * ((t >> 3) ^ ((row >> 3) & 7)) + (t & 7);
}

// Thread t loads tokens 4*(t/16) .. +3 of the tile, channels 8*(t%16) .. +7 (four 16-byte pieces, each token's
// 256-byte row read by 16 consecutive lanes), and writes them transposed: 8 channels x 4 tokens, one 8-byte
// LDS store per channel (4 tokens stay inside one 8-token chunk, so the swizzle keeps them contiguous).  Rows past the chunk's end read the last valid row and are stored as zeros.
struct GramLoad {
    u32x4 w[4];
};

__device__ __forceinline__ void gram_load(GramLoad& L, const uint16_t* X, size_t rs, int tile0, int cnt, int tid) {
    const int c8 = tid & 15, t4 = tid >> 4;
#pragma unroll
    for (int a = 0; a < 4; ++a) {
        const int t = min(tile0 + 4 * t4 + a, cnt - 1);
        L.w[a] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(X + (size_t)t * rs + 8 * c8));   // read once
    }
}

__device__ __forceinline__ void gram_store(const GramLoad& L, uint16_t* Xt, int tile0, int cnt, int tid) {
    const int c8 = tid & 15, t4 = tid >> 4;
    uint32_t w[4][4];
#pragma unroll
    for (int a = 0; a < 4; ++a) {
        const bool ok = tile0 + 4 * t4 + a < cnt;
        w[a][0] = ok ? L.w[a].x : 0u; w[a][1] = ok ? L.w[a].y : 0u;
        w[a][2] = ok ? L.w[a].z : 0u; w[a][3] = ok ? L.w[a].w : 0u;
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        // word k of token a holds channels 2k (low half) and 2k+1 (high half)
        const uint32_t lo01 = __builtin_amdgcn_perm(w[1][k], w[0][k], 0x05040100u);   // ch 2k: tokens 0, 1
        const uint32_t lo23 = __builtin_amdgcn_perm(w[3][k], w[2][k], 0x05040100u);   // ch 2k: tokens 2, 3
        const uint32_t hi01 = __builtin_amdgcn_perm(w[1][k], w[0][k], 0x07060302u);   // ch 2k+1: tokens 0, 1
        const uint32_t hi23 = __builtin_amdgcn_perm(w[3][k], w[2][k], 0x07060302u);
        *reinterpret_cast<u32x2*>(&Xt[gram_pos(8 * c8 + 2 * k, 4 * t4)]) = u32x2{lo01, lo23};
        *reinterpret_cast<u32x2*>(&Xt[gram_pos(8 * c8 + 2 * k + 1, 4 * t4)]) = u32x2{hi01, hi23};
    }
}

// Wave w accumulates a 4 x 4 block of the 16 x 16 output tiles (row blocks 4*(w/2) .., column blocks
// 4*(w%2) ..): 8 fragment reads feed 16 MFMAs per 32-token step.  A block fragment (lane l: channel
// 16*blk + l%16, tokens 8*(l/16) .. +7 of the step) has the layout of both the A operand of its row block
// and the B operand of its column block.
__global__ __launch_bounds__(256) void k_gram(GramArgs a) {
    __shared__ __attribute__((aligned(16))) uint16_t xt[MKV_D * kGramRow];
    const int b = blockIdx.x;
    const int r = find_slot(a.t_gblk, a.B, b);
    const int n = a.t_n[r], nch = (n + kGramChunk - 1) / kGramChunk;
    const int local = b - a.t_gblk[r];
    const int s = local / nch, chunk = local - s * nch;     // s = 2 * head + tensor
    const int h = s >> 1, X = s & 1;
    const int t0 = chunk * kGramChunk, cnt = min(kGramChunk, n - t0);
    const int tid = threadIdx.x, lane = tid & 63, wid = __builtin_amdgcn_readfirstlane(tid >> 6);
    const size_t rs = (size_t)a.Hkv * MKV_D;
    const uint16_t* src = (X ? a.V : a.K) + ((size_t)(a.t_tok0[r] + t0) * a.Hkv + h) * MKV_D;
    const int ntile = (cnt + kGramTile - 1) / kGramTile;

    const int rb0 = 4 * (wid >> 1), cb0 = 4 * (wid & 1);   // the wave's 4 x 4 block of 16 x 16 output tiles
    f32x4 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    GramLoad ld;
    gram_load(ld, src, rs, 0, cnt, tid);
    for (int tl = 0; tl < ntile; ++tl) {
        __syncthreads();   // the previous tile's fragments have been read
        gram_store(ld, xt, tl * kGramTile, cnt, tid);
        if (tl + 1 < ntile) gram_load(ld, src, rs, (tl + 1) * kGramTile, cnt, tid);
        __syncthreads();
#pragma unroll 1
        for (int ks = 0; ks < kGramTile / 32; ++ks) {
            const int col = 32 * ks + 8 * (lane >> 4);
            bf16x8 fa[4], fb[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                fa[i] = *reinterpret_cast<const bf16x8*>(&xt[gram_pos(16 * (rb0 + i) + (lane & 15), col)]);
                fb[i] = *reinterpret_cast<const bf16x8*>(&xt[gram_pos(16 * (cb0 + i) + (lane & 15), col)]);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
        }
    }
    // partial of this chunk: row 16*(rb0 + i) + 4*(lane/16) + e, column 16*(cb0 + j) + lane%16
    float* dst = a.part + (size_t)b * (MKV_D * MKV_D);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                dst[(16 * (rb0 + i) + 4 * (lane >> 4) + e) * MKV_D + 16 * (cb0 + j) + (lane & 15)] = acc[i][j][e];
}

// One workgroup per (stream, 1024-element slice of its 128 x 128 matrix): the sum of the stream's partials.
__global__ __launch_bounds__(256) void k_gram_reduce(GramArgs a) {
    const int slice = blockIdx.x & 15, stream = blockIdx.x >> 4;   // stream = (r * Hkv + h) * 2 + X
    const int r = stream / (2 * a.Hkv), s = stream - r * 2 * a.Hkv;
    const int n = a.t_n[r], nch = (n + kGramChunk - 1) / kGramChunk;
    const int first = a.t_gblk[r] + s * nch;
    const int e = slice * 1024 + 4 * threadIdx.x;
    f32x4 sum = {0.f, 0.f, 0.f, 0.f};
    for (int c = 0; c < nch; ++c) sum += *reinterpret_cast<const f32x4*>(a.part + (size_t)(first + c) * (MKV_D * MKV_D) + e);
    *reinterpret_cast<f32x4*>(a.gram + (size_t)stream * (MKV_D * MKV_D) + e) = sum;
}

hipError_t launch_gram(const GramArgs& a, int n_blocks, hipStream_t s) {
    if (n_blocks == 0) return hipSuccess;
    launch_kernel(k_gram, dim3(n_blocks), dim3(256), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_gram_reduce(const GramArgs& a, hipStream_t s) {
    launch_kernel(k_gram_reduce, dim3(16 * 2 * a.B * a.Hkv), dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace mkv
