// Internal definitions shared by the libvsa kernels and the host entry points.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "attn_layout.hpp"
#include "vsa.h"

namespace vsa {

constexpr int kBlock = 64;

// Kernel-side view of a problem (passed by value to every kernel).
// Token rows of q/out and k/v are addressed through element strides (d is
// contiguous): [B,H,S,D] and [B,S,H,D] are both "dense" (one sequence per
// batch item), the packed layout is [H,slots,D].  The attention kernels work
// on 64-token blocks; the coarse branch and the routing on VSA blocks of
// 64 * ratio tokens (ratio 1, 2 or 4).  Packed metadata (cu_*, bs_*,
// total_*, max_*) counts VSA blocks, each occupying 64 * ratio slots.
struct DevProblem {
    int packed;  // 0 dense ([B,H,S,D] or [B,S,H,D]), 1 block-padded packed [H,slots,D]
    int bshd;    // dense tensors are [B,S,H,D]
    int H, D;
    int nseq;  // B (dense) or num_seqs (packed)
    // dense
    int Sq, Skv, nQ, nKV;  // lengths and 64-token block counts
    int ratio;             // VSA block = 64 * ratio tokens (1 in the coarse view)
    int nQB, nKVB;         // VSA blocks per sequence (= nQ, nKV when ratio is 1)
    int kk;                // min(topk, nKVB): row length of q2k_idx (dense)
    // packed
    const int* cu_q;
    const int* cu_kv;
    const int* bs_q;  // valid tokens per VSA block
    const int* bs_kv;
    const int* topk_s;
    int total_q, total_kv, max_q, max_kv, max_topk;
    int idx_row;  // row length of q2k_idx: kk (dense) or max_topk (packed)
    // element strides of token rows: sequence (batch item), head, token
    int64_t q_sb, q_sh, q_st;
    int64_t kv_sb, kv_sh, kv_st;
};

// One sequence on one head: where its blocks live.  "Blocks" are 64-token
// blocks (the attention kernels' tiles); in the coarse view (ratio 1) they
// are the VSA blocks.
struct SeqView {
    int nq, nkv, k;       // query blocks, KV blocks, top-k (clamped, in VSA blocks)
    int qblk0, kvblk0;    // first global VSA block (packed: index into bs_q / bs_kv) or 0 (dense)
    int64_t qblk_base;    // index of block 0 in 64-token-block arrays (row statistics)
    int64_t kvblk_base;   // the same for k/v
    int64_t qvsa_base;    // index of VSA block 0 in VSA-block arrays (out_c, q2k_idx, q2k_num)
    int64_t kvvsa_base;   // the same for k/v
    int64_t qrow_base;    // row (token slot) of block 0 in [.., S] row-indexed arrays (lse)
    int64_t kvrow_base;   // the same for k/v
    int64_t q_off, kv_off;  // element offset of token row 0 in q/out and in k/v
    int64_t q_st, kv_st;    // element stride between consecutive token rows
    int idx_rebase;       // added to local VSA block numbers when stored in q2k_idx
};

__device__ __forceinline__ int clampi(int x, int lo, int hi) { return x < lo ? lo : (x > hi ? hi : x); }

__device__ __forceinline__ SeqView seq_view(const DevProblem& P, int s, int h) {
    SeqView v;
    if (!P.packed) {
        v.nq = P.nQ;
        v.nkv = P.nKV;
        v.k = P.kk;
        v.qblk0 = 0;
        v.kvblk0 = 0;
        const int64_t sh = (int64_t)s * P.H + h;
        v.qblk_base = sh * P.nQ;
        v.kvblk_base = sh * P.nKV;
        v.qvsa_base = sh * P.nQB;
        v.kvvsa_base = sh * P.nKVB;
        v.qrow_base = sh * P.Sq;
        v.kvrow_base = sh * P.Skv;
        v.q_off = (int64_t)s * P.q_sb + (int64_t)h * P.q_sh;
        v.kv_off = (int64_t)s * P.kv_sb + (int64_t)h * P.kv_sh;
        v.q_st = P.q_st;
        v.kv_st = P.kv_st;
        v.idx_rebase = 0;
    } else {
        int q0 = clampi(P.cu_q[s], 0, P.total_q);
        int q1 = clampi(P.cu_q[s + 1], q0, P.total_q);
        int k0 = clampi(P.cu_kv[s], 0, P.total_kv);
        int k1 = clampi(P.cu_kv[s + 1], k0, P.total_kv);
        const int lr = P.ratio >> 1;  // log2(ratio): 64-token blocks per VSA block
        const int nkvb = min(k1 - k0, P.max_kv);
        v.nq = min(q1 - q0, P.max_q) << lr;
        v.nkv = nkvb << lr;
        v.k = clampi(P.topk_s[s], 1, min(P.max_topk, max(nkvb, 1)));
        v.qblk0 = q0;
        v.kvblk0 = k0;
        v.qvsa_base = (int64_t)h * P.total_q + q0;
        v.kvvsa_base = (int64_t)h * P.total_kv + k0;
        v.qblk_base = v.qvsa_base << lr;
        v.kvblk_base = v.kvvsa_base << lr;
        v.qrow_base = v.qblk_base * kBlock;
        v.kvrow_base = v.kvblk_base * kBlock;
        v.q_off = v.qrow_base * P.D;
        v.kv_off = v.kvrow_base * P.D;
        v.q_st = P.D;
        v.kv_st = P.D;
        v.idx_rebase = k0;
    }
    return v;
}

// Valid tokens of 64-token block r of a packed VSA block holding `size`
// tokens: the first block keeps at least one token (sizes are clamped to
// [1, 64 ratio]), later ones may be empty.
__device__ __forceinline__ int packed_sub_size(int size, int r) {
    return clampi(size - kBlock * r, r == 0 ? 1 : 0, kBlock);
}
// Valid tokens of local query / KV block i of sequence view v.
__device__ __forceinline__ int q_block_size(const DevProblem& P, const SeqView& v, int i) {
    if (!P.packed) return min(kBlock, P.Sq - kBlock * i);
    const int lr = P.ratio >> 1;
    return packed_sub_size(P.bs_q[v.qblk0 + (i >> lr)], i & ((1 << lr) - 1));
}
__device__ __forceinline__ int kv_block_size(const DevProblem& P, const SeqView& v, int j) {
    if (!P.packed) return min(kBlock, P.Skv - kBlock * j);
    const int lr = P.ratio >> 1;
    return packed_sub_size(P.bs_kv[v.kvblk0 + (j >> lr)], j & ((1 << lr) - 1));
}

// Sequence owning global query VSA block g (packed): largest s with cu_q[s] <= g.
__device__ __forceinline__ int seq_of_qblock(const DevProblem& P, int g) {
    int lo = 0, hi = P.nseq - 1;
    while (lo < hi) {
        int mid = (lo + hi + 1) >> 1;
        if (P.cu_q[mid] <= g) lo = mid; else hi = mid - 1;
    }
    return lo;
}

// ---------------------------------------------------------------------------
// 3-D tile partition of a T x H x W token grid (raster order, w fastest) into
// tiles of tt x th x tw tokens (at most 256): tiles in raster order of their
// tile coordinates (edge tiles shorter), tokens in raster order inside a
// tile; each tile is one VSA block of blk slots, the smallest of 64, 128 and
// 256 that holds it.  ("[kernel] Extract VSA utility functions into
// fastvideo_kernel", Summary; the 128/256-token variants of "[chore] release
// fastvideo-kernel 0.3.0".)
// ---------------------------------------------------------------------------
struct TileGrid {
    int T, H, W;     // token grid
    int tt, th, tw;  // tile extents
    int nt, nh, nw;  // tiles along each axis
    int ntiles;
    int blk;         // slots per tile (VSA block size)
};

__host__ __device__ inline TileGrid make_tile_grid(int T, int H, int W, int tt, int th, int tw) {
    TileGrid g;
    g.T = T; g.H = H; g.W = W;
    g.tt = tt; g.th = th; g.tw = tw;
    g.nt = (T + tt - 1) / tt;
    g.nh = (H + th - 1) / th;
    g.nw = (W + tw - 1) / tw;
    g.ntiles = g.nt * g.nh * g.nw;
    const int vol = tt * th * tw;
    g.blk = vol <= kBlock ? kBlock : (vol <= 2 * kBlock ? 2 * kBlock : 4 * kBlock);
    return g;
}

// Extents of tile b along t, h, w; returns its token count.
__host__ __device__ inline int tile_extents(const TileGrid& g, int b, int& et, int& eh, int& ew) {
    const int bt = b / (g.nh * g.nw), bh = (b / g.nw) % g.nh, bw = b % g.nw;
    et = g.T - bt * g.tt < g.tt ? g.T - bt * g.tt : g.tt;
    eh = g.H - bh * g.th < g.th ? g.H - bh * g.th : g.th;
    ew = g.W - bw * g.tw < g.tw ? g.W - bw * g.tw : g.tw;
    return et * eh * ew;
}

// Raster index of the u-th token (u < tile size) of tile b.
__host__ __device__ inline int64_t tile_token_raster(const TileGrid& g, int b, int u, int eh, int ew) {
    const int bt = b / (g.nh * g.nw), bh = (b / g.nw) % g.nh, bw = b % g.nw;
    const int lt = u / (eh * ew), lh = (u / ew) % eh, lw = u % ew;
    return ((int64_t)(bt * g.tt + lt) * g.H + (bh * g.th + lh)) * g.W + (bw * g.tw + lw);
}

// ---------------------------------------------------------------------------
// launchers (one per kernel family; each returns hipError_t of the launch)
// ---------------------------------------------------------------------------
// Block means over VSA blocks of 64 * P.ratio tokens.
hipError_t launch_pool(const DevProblem& P, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                       double* qc, double* kc, double* vc, hipStream_t st);
// The same for Q and K only (V is then pooled by launch_coarse_topk).
hipError_t launch_pool_qk(const DevProblem& P, const uint16_t* q, const uint16_t* k, double* qc, double* kc,
                          hipStream_t st);
// The problem as the coarse branch sees it: VSA blocks as its blocks.
inline DevProblem coarse_view(const DevProblem& P) {
    DevProblem C = P;
    C.nQ = P.nQB;
    C.nKV = P.nKVB;
    C.ratio = 1;
    return C;
}
// scratch: coarse_scratch_doubles(P) doubles (block-level scores and row sums).
// With pool_p and v set, V has not been pooled yet: the first score launch
// also pools it (pool_p = the full problem, v its bf16 tensor) into vc, in
// workgroups of its own that run beside the score tiles.
hipError_t launch_coarse_topk(const DevProblem& P, const double* qc, const double* kc,
                              double* vc, float* out_c, int* idx, int* num, double* scratch,
                              hipStream_t st, const DevProblem* pool_p = nullptr, const uint16_t* v = nullptr);
size_t coarse_scratch_doubles(const DevProblem& P);
// out[r][j] = a[query block i] . b[KV block j] (float64, raw dot products) for
// every sequence s and head h, r = (s * H + h) * max_q + i, row length max_kv
// (max_q / max_kv: nQ / nKV for DENSE); rows and columns past a sequence's
// blocks are not written.
hipError_t launch_coarse_scores(const DevProblem& P, const double* a, const double* b, double* out,
                                hipStream_t st);
hipError_t launch_sparse_attn(const DevProblem& P, const uint16_t* q, const uint16_t* k,
                              const uint16_t* v, const int* idx, const int* num, uint16_t* out,
                              hipStream_t st);
hipError_t launch_sparse_attn_combine(const DevProblem& P, const uint16_t* q, const uint16_t* k,
                                      const uint16_t* v, const int* idx, const int* num, const float* out_c,
                                      const uint16_t* gate, int mode, int64_t gs0, int64_t gs1, int64_t gs2,
                                      uint16_t* out, uint16_t* out_s, float* lse, hipStream_t st);
// gather (scatter = false): x [B, Hh, T*H*W, elems] raster -> y [Hh, B * blk *
// ntiles, elems] tile order with zero padding; scatter: the inverse.
hipError_t launch_tile_copy(const TileGrid& g, const uint16_t* src, uint16_t* dst, int B, int Hh, int elems,
                            bool scatter, hipStream_t st);
hipError_t launch_combine(const DevProblem& P, const float* out_c, const uint16_t* gate, int mode,
                          int64_t gs0, int64_t gs1, int64_t gs2, uint16_t* out, hipStream_t st);

constexpr int kMaxKvBlocks = 4096;

// Backward pass.  Row statistics: per query block 64 log-sum-exp values
// (+inf on padding rows) then 64 softmax-backward row terms (0 on padding).
constexpr int kStatRow = 2 * kBlock;

struct BwdArgs {
    // inputs
    const uint16_t *q, *k, *v, *dout, *out_s, *gate;
    const float *out_c, *lse;
    const int *idx, *num;
    int gate_mode;
    int64_t gs0, gs1, gs2;
    // outputs
    uint16_t *dq, *dk, *dv, *dgate;
    // workspace: float64 block-resolution data ([query blocks][D] for qc, doc,
    // dqc; [KV blocks][D] for kc, vc, dkc, dvc; [sequences * H * max query
    // blocks][max KV blocks] for pbuf, dsbuf, rows as launch_coarse_scores),
    // row statistics [query blocks][kStatRow], inverse routing [KV blocks][max
    // query blocks]
    double *qc, *kc, *vc, *doc, *dqc, *dkc, *dvc, *pbuf, *dsbuf;
    float* rs;
    int *k2q, *k2q_num;
    // qc, kc and vc already hold the block means of q, k and v (those the
    // forward computed): the pool launch is skipped
    bool pooled;
};
hipError_t launch_backward(const DevProblem& P, const BwdArgs& A, hipStream_t st);

}  // namespace vsa
