// Backward pass of the VSA forward: gradients of q, k, v and the gate for a
// given output gradient, with the routing (q2k_idx) held fixed - the top-k
// choice is piecewise constant in the inputs and carries no gradient.
// ("[kernel] Add varlen support for block-sparse attention", Test plan:
// backward of the block-sparse attention; "[chore] release fastvideo-kernel
// 0.3.0", Block-sparse / VSA attention improvements: forward and backward.)
//
// With out = out_c[block] * g + O (O the block-sparse attention output, out_c
// the coarse attention of the block means, g the gate or 1) the launches are:
//   1. combine backward, per query block: the softmax-backward row term
//      delta[t] = dout[t] . O[t], dOc[block] = sum_t dout[t] * g[t],
//      dg[t] = dout[t] * out_c[block] (summed over d for a per-token gate), and
//      the row statistics (log-sum-exp, delta) of the block in one 512-byte row;
//   2. the block means again (the forward's pool kernel);
//   3. coarse backward in float64 at block level: S = Qc Kc^T and dP = dOc
//      Vc^T, the coarse softmax P and dS = P (dP - rowsum(P dP)), then
//      dQc = dS Kc / sqrt(D), dKc = dS^T Qc / sqrt(D), dVc = P^T dOc;
//   4. the inverse routing: for every KV block, the query blocks whose list
//      holds it, ascending;
//   5. dQ per query block over its listed KV blocks: S and P = exp(S - lse)
//      again, dP = dO V^T, dS = P (dP - delta), dQ = dS K / sqrt(D), plus
//      dQc / (block size) - the gradient through the block mean;
//   6. dK, dV per KV block over the query blocks that listed it: dV = P^T dO,
//      dK = dS^T Q / sqrt(D), plus dKc, dVc / (block size).
// Steps 5 and 6 run bf16 MFMA with float32 accumulation on the operand
// layouts of the forward kernel (32x32x16 tiles, products computed
// transposed so that every lane owns one column), recompute P from the saved
// log-sum-exp instead of storing it, and each write every output row once
// (no atomics, deterministic).
#include <math.h>

#include "attn_common.hpp"

namespace vsa {
namespace {

using namespace attn;

constexpr int kThreads = 256;      // block-level kernels
constexpr int kAttnThreads = 128;  // MFMA kernels: 2 waves, 32 columns each
// The block lists are walked from a rotated start: work item i begins at
// entry (i mod kSweep) n / kSweep of its n entries and wraps around, kSweep
// being about the number of workgroups resident on one XCD (32 CUs times the
// workgroups per CU).  The lists are ascending, so workgroups running
// together read nearby entries at the same time and share them in L2,
// instead of all starting at the front while earlier ones are deep into
// theirs.  Only the order of the (float32) accumulations changes.
constexpr int kSweepDq = 128;
constexpr int kSweepDkdv = 96;

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ double wave_sum(double x) {
    for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
    return x;
}
// Sequence owning global KV block g (packed): largest s with cu_kv[s] <= g.
__device__ __forceinline__ int seq_of_kvblock(const DevProblem& P, int g) {
    int lo = 0, hi = P.nseq - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (P.cu_kv[mid] <= g) lo = mid; else hi = mid - 1;
    }
    return lo;
}

// ---------------------------------------------------------------------------
// 1. combine backward: grid (VSA blocks: nQB or total_q, H, B or 1); the
// workgroup walks the VSA block's 64-token query blocks in order
// ---------------------------------------------------------------------------
template <int D, int MODE>
__global__ __launch_bounds__(kThreads) void bwd_combine_kernel(
    DevProblem P, const uint16_t* __restrict__ dout, const uint16_t* __restrict__ out_s,
    const float* __restrict__ out_c, const uint16_t* __restrict__ gate, int64_t gs0, int64_t gs1, int64_t gs2,
    const float* __restrict__ lse, float* __restrict__ rs, double* __restrict__ doc, uint16_t* __restrict__ dgate) {
    constexpr int QD = D / 4;  // d values per thread, 4 threads per token
    __shared__ float red[kBlock][D + 1];
    int s, I;
    const int h = blockIdx.y;
    if (!P.packed) {
        I = blockIdx.x;
        s = blockIdx.z;
    } else {
        s = seq_of_qblock(P, blockIdx.x);
        I = (int)blockIdx.x - clampi(P.cu_q[s], 0, P.total_q);
    }
    const SeqView sv = seq_view(P, s, h);
    const int R = P.ratio;  // 64-token query blocks per VSA block
    if (I < 0 || R * I >= sv.nq) return;
    // row of the VSA block in the block-resolution arrays (out_c, dOc)
    const int64_t cb = sv.qvsa_base + I;
    const int64_t g0 = (P.packed ? 0 : (int64_t)s * gs0) + (int64_t)h * gs1;
    const int t = threadIdx.x / 4, d0 = (threadIdx.x % 4) * QD;
    const float* ocr = out_c + cb * D;
    double dsum = 0.0;  // thread d < D: dOc[d] summed over the VSA block's tokens
    for (int r = 0; r < R; ++r) {
        const int i = R * I + r;
        if (i >= sv.nq) break;  // the same for every thread
        const int size = q_block_size(P, sv, i);
        const int64_t row0 = sv.qrow_base + (int64_t)kBlock * i;  // row of token 0 in [.., S] arrays (lse)
        const int64_t qb = sv.qblk_base + i;                       // 64-token block (statistics)
        // token index of the block's first row along the gate's token axis
        const int64_t tok0 = (int64_t)kBlock * (P.packed ? sv.qblk0 * R + i : i);
        // element offset of token t of this block in dout / out_s / a full dgate
        const int64_t qo = sv.q_off + ((int64_t)kBlock * i + t) * sv.q_st;
        float dpart = 0.f, gpart = 0.f;
        float contrib[QD];
#pragma unroll
        for (int e = 0; e < QD; ++e) contrib[e] = 0.f;
        if (t < size) {
            const int64_t goff = g0 + (tok0 + t) * gs2;
            const float g = MODE == VSA_GATE_TOKEN ? bf16_lo(gate[goff]) : 1.f;
#pragma unroll
            for (int c = 0; c < QD / 8; ++c) {
                const uint4 a = *reinterpret_cast<const uint4*>(dout + qo + d0 + 8 * c);
                const uint4 o = *reinterpret_cast<const uint4*>(out_s + qo + d0 + 8 * c);
                uint4 gg = make_uint4(0, 0, 0, 0);
                if (MODE == VSA_GATE_FULL) gg = *reinterpret_cast<const uint4*>(gate + goff + d0 + 8 * c);
                const uint32_t aw[4] = {a.x, a.y, a.z, a.w}, ow[4] = {o.x, o.y, o.z, o.w};
                const uint32_t gw[4] = {gg.x, gg.y, gg.z, gg.w};
                uint32_t dg[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int dd = 8 * c + 2 * e;
                    const float a0 = bf16_lo(aw[e]), a1 = bf16_hi(aw[e]);
                    dpart = fmaf(a0, bf16_lo(ow[e]), dpart);
                    dpart = fmaf(a1, bf16_hi(ow[e]), dpart);
                    const float c0 = ocr[d0 + dd], c1 = ocr[d0 + dd + 1];
                    if (MODE == VSA_GATE_FULL) {
                        contrib[dd] = a0 * bf16_lo(gw[e]);
                        contrib[dd + 1] = a1 * bf16_hi(gw[e]);
                        dg[e] = bf16pair(a0 * c0, a1 * c1);
                    } else {
                        contrib[dd] = a0 * g;
                        contrib[dd + 1] = a1 * g;
                        if (MODE == VSA_GATE_TOKEN) gpart = fmaf(a1, c1, fmaf(a0, c0, gpart));
                    }
                }
                if (MODE == VSA_GATE_FULL)
                    *reinterpret_cast<uint4*>(dgate + qo + d0 + 8 * c) = make_uint4(dg[0], dg[1], dg[2], dg[3]);
            }
        } else if (MODE == VSA_GATE_FULL && P.packed) {
#pragma unroll
            for (int c = 0; c < QD / 8; ++c)
                *reinterpret_cast<uint4*>(dgate + qo + d0 + 8 * c) = make_uint4(0, 0, 0, 0);
        }
        // the 4 threads of a token are consecutive lanes
        dpart += __shfl_xor(dpart, 1);
        dpart += __shfl_xor(dpart, 2);
        gpart += __shfl_xor(gpart, 1);
        gpart += __shfl_xor(gpart, 2);
        if (threadIdx.x % 4 == 0) {
            const bool valid = t < size;
            // padding rows: lse = +inf makes every recomputed probability 0
            rs[qb * kStatRow + t] = valid ? lse[row0 + t] : INFINITY;
            rs[qb * kStatRow + kBlock + t] = valid ? dpart : 0.f;
            // a token gate's gradient in the query layout: element offset / D
            if (MODE == VSA_GATE_TOKEN && (valid || P.packed))
                dgate[qo / D] = (uint16_t)(bf16pair(valid ? gpart : 0.f, 0.f) & 0xffffu);
        }
#pragma unroll
        for (int e = 0; e < QD; ++e) red[t][d0 + e] = contrib[e];
        __syncthreads();
        for (int d = threadIdx.x; d < D; d += kThreads)
            for (int tt = 0; tt < size; ++tt) dsum += (double)red[tt][d];
        __syncthreads();  // red is rewritten by the next 64-token block
    }
    for (int d = threadIdx.x; d < D; d += kThreads) doc[cb * D + d] = dsum;
}

// ---------------------------------------------------------------------------
// 3. coarse backward (float64).  The block-level matrices S = Qc Kc^T and
// dP = dOc Vc^T come from the forward's tiled score kernel (rows r = (s H +
// h) max_q + i, row length ld = max_kv); then, per row, P = softmax(S /
// sqrt(D)) and dS = P (dP - sum_j P_j dP_j) in place; then three tiled
// products: dQc = dS Kc / sqrt(D), dKc = dS^T Qc / sqrt(D), dVc = P^T dOc.
// ---------------------------------------------------------------------------
// One wave per row; grid ceil(rows / 4), rows = sequences * H * max_q.
__global__ __launch_bounds__(kThreads) void bwd_coarse_softmax_kernel(DevProblem P, double* __restrict__ sbuf,
                                                                      double* __restrict__ dbuf, int ld, int maxq,
                                                                      double scale) {
    const int wave = threadIdx.x / 64, lane = threadIdx.x % 64;
    const int64_t r = (int64_t)blockIdx.x * (kThreads / 64) + wave;
    if (r >= (int64_t)P.nseq * P.H * maxq) return;
    const int i = (int)(r % maxq);
    const int sh = (int)(r / maxq);
    const SeqView sv = seq_view(P, sh / P.H, sh % P.H);
    if (i >= sv.nq) return;
    double* srow = sbuf + r * ld;  // S, then P
    double* drow = dbuf + r * ld;  // dP, then dS
    const int n = sv.nkv;
    double mx = -INFINITY;
    for (int j = lane; j < n; j += 64) mx = fmax(mx, srow[j]);
    for (int o = 32; o > 0; o >>= 1) mx = fmax(mx, __shfl_xor(mx, o));
    double sum = 0.0;
    for (int j = lane; j < n; j += 64) {
        const double w = exp((srow[j] - mx) * scale);
        srow[j] = w;
        sum += w;
    }
    sum = wave_sum(sum);
    const double inv = 1.0 / sum;
    double dot = 0.0;
    for (int j = lane; j < n; j += 64) {
        const double p = srow[j] * inv;
        srow[j] = p;
        dot = fma(p, drow[j], dot);
    }
    dot = wave_sum(dot);
    for (int j = lane; j < n; j += 64) drow[j] = srow[j] * (drow[j] - dot);
}

// out[o][d] = alpha sum_k M(o, k) X[k][d] over one sequence and head:
//   TRANS = false: o = query block, k = KV block, M(o, k) = m[row(o)][k],
//                  X = a KV-block array, out a query-block array;
//   TRANS = true:  o = KV block, k = query block, M(o, k) = m[row(k)][o],
//                  X = a query-block array, out a KV-block array.
// 64 output rows x D / 2 columns per workgroup (the two column halves of a
// row tile in consecutive workgroups, so that a head's few row tiles spread
// over twice as many CUs), 16-wide k slices of M and X staged in LDS (the
// next slice prefetched into registers), products by float64 MFMA
// (v_mfma_f64_16x16x4): each wave computes 16 or 32 output rows by 32
// columns.  Grid (2 ceil(max rows / 64), H, sequences).
constexpr int kMmSplit = 2;
typedef double f64x4 __attribute__((ext_vector_type(4)));

template <int D, bool TRANS>
__global__ __launch_bounds__(kThreads) void bwd_coarse_mm_kernel(DevProblem P, const double* __restrict__ m,
                                                                 const double* __restrict__ x,
                                                                 double* __restrict__ out, int ld, int maxq,
                                                                 double alpha) {
    // LDS rows 16 doubles longer than their 64 or 32 values (32 banks modulo
    // 64): the four 16-lane groups of an operand read fall on disjoint banks
    constexpr int kTile = 64, kSlice = 16, kPad = 16;
    constexpr int DC = D / kMmSplit;     // columns per workgroup
    constexpr int NT = 2;                // 16-column products per wave
    constexpr int MT = DC == 64 ? 2 : 1; // 16-row products per wave
    static_assert(DC == 32 || DC == 64, "64 or 32 columns per workgroup");
    __shared__ __attribute__((aligned(16))) double mt[kSlice][kTile + kPad];  // [k][o]
    __shared__ __attribute__((aligned(16))) double xs[kSlice][DC + kPad];     // [k][d - cbase]
    const int s = blockIdx.z, h = blockIdx.y;
    const SeqView sv = seq_view(P, s, h);
    const int nout = TRANS ? sv.nkv : sv.nq, nk = TRANS ? sv.nq : sv.nkv;
    const int cbase = (blockIdx.x % kMmSplit) * DC;
    const int o0 = (blockIdx.x / kMmSplit) * kTile;
    if (o0 >= nout) return;
    const int64_t row0 = ((int64_t)s * P.H + h) * maxq;  // m row of query block 0
    const int64_t xbase = TRANS ? sv.qblk_base : sv.kvblk_base;
    const int64_t obase = TRANS ? sv.kvblk_base : sv.qblk_base;
    const int tid = threadIdx.x;
    // wave w computes outputs wr .. wr + 16 MT - 1, columns wc .. wc + 31 of
    // the tile: lane (i = lane % 16, g = lane / 16) supplies M(row i, k g) and
    // X[k g][col i] of each 4-wide k step
    const int wave = tid / 64, lane = tid % 64, lm = lane & 15, lg = lane >> 4;
    const int wr = MT == 2 ? 32 * (wave >> 1) : 16 * wave;
    const int wc = MT == 2 ? 32 * (wave & 1) : 0;
    f64x4 acc[MT][NT];
#pragma unroll
    for (int a = 0; a < MT; ++a)
#pragma unroll
        for (int b = 0; b < NT; ++b) acc[a][b] = f64x4{0.0, 0.0, 0.0, 0.0};
    // staging of M: TRANS = false, thread t holds k = 4 (t % 4) .. + 3 of output
    // row t / 4; TRANS = true, thread t holds outputs 4 (t % 16) .. + 3 of k row t / 16
    const int ma = TRANS ? tid / 16 : tid / 4;
    const int mb = TRANS ? 4 * (tid % 16) : 4 * (tid % 4);
    double mv[4];
    double2 xv[DC / 32];
    auto fetch = [&](int k0) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            int o, k;
            if (TRANS) { k = k0 + ma; o = o0 + mb + e; } else { o = o0 + ma; k = k0 + mb + e; }
            const bool ok = o < nout && k < nk;
            mv[e] = ok ? (TRANS ? m[(row0 + k) * ld + o] : m[(row0 + o) * ld + k]) : 0.0;
        }
#pragma unroll
        for (int p = 0; p < DC / 32; ++p) {
            const int e = tid + kThreads * p;  // double2 index in the [16][DC] slice
            const int kr = e / (DC / 2), dc = 2 * (e % (DC / 2));
            xv[p] = k0 + kr < nk ? *reinterpret_cast<const double2*>(x + (xbase + k0 + kr) * D + cbase + dc)
                                 : make_double2(0.0, 0.0);
        }
    };
    fetch(0);
    for (int k0 = 0; k0 < nk; k0 += kSlice) {
        __syncthreads();  // previous slice fully consumed
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            if (TRANS) mt[ma][mb + e] = mv[e]; else mt[mb + e][ma] = mv[e];
        }
#pragma unroll
        for (int p = 0; p < DC / 32; ++p) {
            const int e = tid + kThreads * p;
            *reinterpret_cast<double2*>(&xs[e / (DC / 2)][2 * (e % (DC / 2))]) = xv[p];
        }
        __syncthreads();
        if (k0 + kSlice < nk) fetch(k0 + kSlice);
#pragma unroll
        for (int k4 = 0; k4 < kSlice; k4 += 4) {
            const int kk = k4 + lg;
            double a[MT], b[NT];
#pragma unroll
            for (int i = 0; i < MT; ++i) a[i] = mt[kk][wr + 16 * i + lm];
#pragma unroll
            for (int j = 0; j < NT; ++j) b[j] = xs[kk][wc + 16 * j + lm];
#pragma unroll
            for (int i = 0; i < MT; ++i)
#pragma unroll
                for (int j = 0; j < NT; ++j) acc[i][j] = __builtin_amdgcn_mfma_f64_16x16x4f64(a[i], b[j], acc[i][j], 0, 0, 0);
        }
    }
    // accumulator e of product (i, j): output wr + 16 i + 4 e + g, column wc + 16 j + m
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int o = o0 + wr + 16 * i + 4 * e + lg;
            if (o >= nout) continue;
            double* dst = out + (obase + o) * D + cbase + wc + lm;
#pragma unroll
            for (int j = 0; j < NT; ++j) dst[16 * j] = acc[i][j][e] * alpha;
        }
}

// ---------------------------------------------------------------------------
// 4. inverse routing: one wave per KV block, grid (ceil(max KV blocks / 4),
// H, sequences)
// ---------------------------------------------------------------------------
// Whether x is in the ascending list row[0..n).
__device__ __forceinline__ bool list_has(const int* row, int n, int x) {
    int lo = 0, hi = n;  // first position with row[pos] >= x
    while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (row[mid] < x) lo = mid + 1; else hi = mid;
    }
    return lo < n && row[lo] == x;
}

__global__ __launch_bounds__(kThreads) void bwd_k2q_kernel(DevProblem P, const int* __restrict__ idx,
                                                           const int* __restrict__ num, int* __restrict__ k2q,
                                                           int* __restrict__ k2q_num, int ldq) {
    const int wave = threadIdx.x / 64, lane = threadIdx.x % 64;
    const int s = blockIdx.z, h = blockIdx.y;
    const int j = blockIdx.x * (kThreads / 64) + wave;
    const SeqView sv = seq_view(P, s, h);
    if (j >= sv.nkv) return;
    // lists hold VSA blocks of 64 * ratio tokens
    const int lr = P.ratio >> 1;
    const int key = (j >> lr) + sv.idx_rebase;  // as stored in q2k_idx
    const int64_t kb = sv.kvblk_base + j;
    // an empty 64-token block of a packed VSA block (KV or query side) takes
    // part in no product
    const bool kv_empty = P.packed && lr > 0 && kv_block_size(P, sv, j) == 0;
    int count = 0;
    for (int i0 = 0; i0 < sv.nq && !kv_empty; i0 += 64) {
        const int i = i0 + lane;
        bool member = false;
        if (i < sv.nq && (!P.packed || lr == 0 || q_block_size(P, sv, i) > 0)) {
            const int64_t qb = sv.qvsa_base + (i >> lr);  // the list of i's VSA block
            member = list_has(idx + qb * P.idx_row, clampi(num[qb], 0, P.idx_row), key);
        }
        const uint64_t mask = __ballot(member);
        const uint64_t below = mask & ((1ull << lane) - 1ull);
        if (member) k2q[kb * ldq + count + __popcll(below)] = i;
        count += __popcll(mask);
    }
    if (lane == 0) k2q_num[kb] = count;
}

// ---------------------------------------------------------------------------
// shared pieces of the two MFMA kernels
// ---------------------------------------------------------------------------
// LDS operand reads of a [64][D] tile, from per-lane byte offsets computed
// once per kernel.  Every swizzle depends on the row through its low 4 bits
// only, so moving by 32 rows (mt) or 16 rows (s4) is a constant that the
// compiler folds into the instruction's offset field; only the k-step (row
// operands) or the d tile and 8-row group (transposed operands) need a
// register each.
//
// Row operand: lane (l32, hh) gets T[32 mt + l32][16 ks + 8 hh .. + 7] (A
// operand of a 32x32x16 product whose rows are the tile's rows).
template <int CH, int SW>
__device__ __forceinline__ uint32_t row_offset(int l32, int hh, int ks) {
    return 2u * (uint32_t)tile_off<CH>(l32, 2 * ks + hh, tile_swz<CH, SW>(l32));
}
template <int CH>
__device__ __forceinline__ bf16x8 row_read(const uint16_t* tile, uint32_t off, int mt) {
    return as_bf16x8(*reinterpret_cast<const uint4*>((const char*)tile + off + mt * 32 * CH * 16));
}
// Transposed operand for k-step s4 (16 rows) and 32-row d tile dt: lane
// (l32, hh) gets T[16 s4 + 4 hh + {0..3, 8..11}][32 dt + l32], the k-slot
// order of a B operand taken from an accumulator (see pack_half).  Two
// transpose reads, rows 16 s4 + 8 jj + 4 hh + tr_r.
template <int CH, int SW>
__device__ __forceinline__ uint32_t tr_offset(int dt, int jj, int hh, int tr_r, int tr_d) {
    const int tok = 8 * jj + 4 * hh + tr_r;
    const int d = 32 * dt + tr_d;
    return 2u * (uint32_t)(tile_off<CH>(tok, d >> 3, tile_swz<CH, SW>(tok)) + (d & 7));
}
template <int CH>
__device__ __forceinline__ bf16x8 tr_read(const uint16_t* tile, uint32_t off0, uint32_t off1, int s4) {
    typedef __attribute__((address_space(3))) const char lds_char;
    lds_char* base = (lds_char*)tile + s4 * 16 * CH * 16;
    const s16x4 h0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(base + off0));
    const s16x4 h1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(base + off1));
    const uint2 a = __builtin_bit_cast(uint2, h0), b = __builtin_bit_cast(uint2, h1);
    return as_bf16x8(make_uint4(a.x, a.y, b.x, b.y));
}
// One row of D bf16 values as the B operand of products over d: lane (l32,
// hh) gets src[16 ks + 8 hh .. + 7] for every k-step (zeros if !valid).
template <int KS>
__device__ __forceinline__ void load_b_row(const uint16_t* src, bool valid, int hh, bf16x8 (&f)[KS]) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        uint4 u = make_uint4(0, 0, 0, 0);
        if (valid) u = *reinterpret_cast<const uint4*>(src + 16 * ks + 8 * hh);
        f[ks] = as_bf16x8(u);
    }
}

// ---------------------------------------------------------------------------
// 5. dQ: one workgroup (2 waves) per query block; wave w owns query rows
// 32 w .. 32 w + 31, one per lane column, with its Q and dO rows in registers
// as B operands.  One K tile (read by rows for S^T = K Q^T and transposed for
// dQ^T = K^T dS^T) and one V tile (read by rows for dP^T = V dO^T) in LDS, both
// in the dual layout, 32 KiB for D = 128, so that four workgroups share a
// CU.  Per listed KV block t: wait for V_t and K_t; per 32-token half, dP^T
// (accumulated onto -delta, so it holds dP^T - delta) and S^T, then dS^T =
// exp2(S^T c - lse) (dP^T - delta) packed to bf16; release V_t and start
// V_{t+1}; dQ^T += K^T dS^T; release K_t and start K_{t+1}.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(kAttnThreads, 2) void bwd_dq_kernel(
    DevProblem P, const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const uint16_t* __restrict__ dout, const float* __restrict__ rs, const int* __restrict__ idx,
    const int* __restrict__ num, const double* __restrict__ dqc, uint16_t* __restrict__ dq, float c_log2,
    float scale) {
    constexpr int KS = D / 16, DT = D / 32, CH = D / 8;
    __shared__ __attribute__((aligned(1024))) uint16_t k_tile[kBlock * D];
    __shared__ __attribute__((aligned(1024))) uint16_t v_tile[kBlock * D];

    int s, h, i;
    SeqView sv;
    if (!P.packed) {
        const int N = P.nQ * P.H * P.nseq;
        const int lin = xcd_remap(blockIdx.x, N);
        i = lin % P.nQ;
        const int rest = lin / P.nQ;
        h = rest % P.H;
        s = rest / P.H;
        sv = seq_view(P, s, h);
    } else {
        const int lr = P.ratio >> 1;
        const int N = (P.total_q << lr) * P.H;
        const int lin = xcd_remap(blockIdx.x, N);
        const int g = lin % (P.total_q << lr);
        h = lin / (P.total_q << lr);
        s = seq_of_qblock(P, g >> lr);
        sv = seq_view(P, s, h);
        i = g - (sv.qblk0 << lr);
        if (i < 0 || i >= sv.nq) return;
    }
    const int qsize = q_block_size(P, sv, i);  // 0: an empty block of a packed VSA block
    const int64_t qoff0 = sv.q_off + (int64_t)kBlock * i * sv.q_st;  // element offset of the block's row 0
    const int64_t qb = sv.qblk_base + i;                              // 64-token block (statistics)
    // VSA blocks of 64 * ratio tokens: the list, out_c and dQc are per VSA
    // block; a listed VSA block J stands for 64-token KV blocks
    // J ratio .. J ratio + ratio - 1
    const int lr = P.ratio >> 1;
    const int64_t qbv = sv.qvsa_base + (i >> lr);
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, l32 = lane & 31, hh = lane >> 5;
    const int qr = 32 * wave + l32;
    const bool qvalid = qr < qsize;

    bf16x8 qf[KS], df[KS];
    load_b_row<KS>(q + qoff0 + qr * sv.q_st, qvalid, hh, qf);
    load_b_row<KS>(dout + qoff0 + qr * sv.q_st, qvalid, hh, df);
    const float lse = rs[qb * kStatRow + qr];  // +inf for padding rows
    const float delta = rs[qb * kStatRow + kBlock + qr];

    f32x16 acc[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[dt][e] = 0.f;

    const int nsel = __builtin_amdgcn_readfirstlane(qsize > 0 ? clampi(num[qbv], 0, P.idx_row) : 0);
    const int n = nsel << lr;  // 64-token KV blocks to visit
    const_int* list = (const_int*)uniform_ptr(idx + qbv * P.idx_row);
    const_int* bs_kv = (const_int*)(P.packed ? uniform_ptr(P.bs_kv + sv.kvblk0) : nullptr);
    const int rebase = __builtin_amdgcn_readfirstlane(sv.idx_rebase);
    const int nkv = __builtin_amdgcn_readfirstlane(sv.nkv);
    const int t0 = n > 0 ? ((i % kSweepDq) * n) / kSweepDq : 0;
    // valid tokens of local KV block j (packed: 0 for an empty 64-token block
    // of a VSA block)
    auto kv_size = [&](int j) -> int {
        return P.packed ? packed_sub_size(bs_kv[j >> lr], j & ((1 << lr) - 1)) : min(kBlock, P.Skv - kBlock * j);
    };
    auto next_valid = [&](int& t) -> int {
        for (; t < n; ++t) {
            int pos = t0 + t;
            if (pos >= n) pos -= n;
            const int J = list[pos >> lr] - rebase;
            // no sequence has 2^28 VSA blocks: such an entry (or a negative
            // one) is out of range, and is kept from wrapping by the shift
            if ((unsigned)J >= (1u << 28)) continue;
            const int j = (J << lr) + (pos & ((1 << lr) - 1));
            if (j < nkv && (lr == 0 || !P.packed || kv_size(j) > 0)) return j;
        }
        return -1;
    };
    // both tiles in the dual layout (V is only read by rows, which that layout
    // serves without conflicts too), so they share every lane offset
    const uint32_t off0 = (uint32_t)lane_src_offset<CH, kSwzDual>(wave, lane, 0);
    const uint32_t off1 = (uint32_t)lane_src_offset<CH, kSwzDual>(wave, lane, 1) - 2048u;
    const uint32_t k_lds = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)k_tile + 1024u * wave);
    const uint32_t v_lds = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)v_tile + 1024u * wave);
    const int L16 = lane & 15, g16 = lane >> 4;
    const int tr_r = tr_token(L16), tr_d = 16 * (g16 & 1) + 4 * tr_dquad(L16);
    uint32_t t_row[KS], k_tr[DT][2];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) t_row[ks] = row_offset<CH, kSwzDual>(l32, hh, ks);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) k_tr[dt][jj] = tr_offset<CH, kSwzDual>(dt, jj, hh, tr_r, tr_d);
    const uint32_t pitch = __builtin_amdgcn_readfirstlane((uint32_t)(2 * sv.kv_st));  // bytes between KV rows
    auto issue_v = [&](int jj, int vs) {
        load_tile<D, kSwzDual>(v_lds, v + sv.kv_off + (int64_t)kBlock * jj * sv.kv_st, vs, wave, lane, off0, off1,
                               pitch);
    };
    auto issue_k = [&](int jj, int vs) {
        load_tile<D, kSwzDual>(k_lds, k + sv.kv_off + (int64_t)kBlock * jj * sv.kv_st, vs, wave, lane, off0, off1,
                               pitch);
    };

    // the operands above are in registers before the first direct copy, so
    // the copies are the only vector-memory operations the waits count
    __builtin_amdgcn_s_waitcnt(0);

    int t = 0;
    int j = next_valid(t);
    int kvsize = j >= 0 ? kv_size(j) : 0;
    if (j >= 0) {
        issue_v(j, kvsize);
        issue_k(j, kvsize);
    }
    while (j >= 0) {
        ++t;
        const int jn = next_valid(t);
        const bool more = jn >= 0;
        const int kvsize_n = more ? kv_size(jn) : 0;
        wait_vmcnt<0>();  // V_t and K_t landed
        wg_barrier();
        // One 32-token half (mt) of the block at a time: dP^T - delta = V dO^T -
        // delta and S^T = K Q^T (rows = KV tokens 32 mt + 8 (e / 4) + 4 hh +
        // e % 4, lane column = query), then dS^T = exp2(S^T c - lse) (dP^T -
        // delta), kept as the bf16 B operands of k-steps 2 mt and 2 mt + 1.
        bf16x8 dsb[4];
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
            f32x16 pacc, sacc;
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                pacc[e] = -delta;
                sacc[e] = 0.f;
            }
            // operands are read one k-step ahead of their MFMAs; the scheduling
            // barriers keep the compiler from hoisting every read (registers)
            bf16x8 va = row_read<CH>(v_tile, t_row[0], mt);
            bf16x8 ka = row_read<CH>(k_tile, t_row[0], mt);
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                bf16x8 vn = va, kn = ka;
                if (ks + 1 < KS) {
                    vn = row_read<CH>(v_tile, t_row[ks + 1], mt);
                    kn = row_read<CH>(k_tile, t_row[ks + 1], mt);
                }
                __builtin_amdgcn_sched_barrier(0);
                pacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, df[ks], pacc, 0, 0, 0);
                sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[ks], sacc, 0, 0, 0);
                __builtin_amdgcn_sched_barrier(0);
                va = vn;
                ka = kn;
            }
            if (kvsize < kBlock) {  // tokens past a partial block: S = -inf, P = 0
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const int tok = 32 * mt + 8 * (e >> 2) + 4 * hh + (e & 3);
                    if (tok >= kvsize) sacc[e] = -INFINITY;
                }
            }
#pragma unroll
            for (int e = 0; e < 16; ++e) sacc[e] = __builtin_amdgcn_exp2f(fmaf(sacc[e], c_log2, -lse)) * pacc[e];
#pragma unroll
            for (int hf = 0; hf < 2; ++hf)
                dsb[2 * mt + hf] = as_bf16x8(make_uint4(
                    bf16pair(sacc[8 * hf + 0], sacc[8 * hf + 1]), bf16pair(sacc[8 * hf + 2], sacc[8 * hf + 3]),
                    bf16pair(sacc[8 * hf + 4], sacc[8 * hf + 5]), bf16pair(sacc[8 * hf + 6], sacc[8 * hf + 7])));
        }
        wg_barrier();  // both waves are done with the V tile
        if (more) issue_v(jn, kvsize_n);
        // dQ^T += K^T dS^T over 4 k-steps of 16 KV tokens
        {
            bf16x8 ta = tr_read<CH>(k_tile, k_tr[0][0], k_tr[0][1], 0);
#pragma unroll
            for (int x = 0; x < 4 * DT; ++x) {
                const int s4 = x / DT, dt = x % DT;
                bf16x8 tn = ta;
                if (x + 1 < 4 * DT) {
                    const int dn = (x + 1) % DT;
                    tn = tr_read<CH>(k_tile, k_tr[dn][0], k_tr[dn][1], (x + 1) / DT);
                }
                __builtin_amdgcn_sched_barrier(0);
                acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ta, dsb[s4], acc[dt], 0, 0, 0);
                __builtin_amdgcn_sched_barrier(0);
                ta = tn;
            }
        }
        wg_barrier();  // both waves are done with the K tile
        if (more) issue_k(jn, kvsize_n);
        j = jn;
        kvsize = kvsize_n;
    }

    // lane holds dQ[qr][32 dt + 8 (e / 4) + 4 hh + e % 4]
    uint16_t* orow = dq + qoff0 + qr * sv.q_st;
    if (qvalid) {
        // the gradient through the block mean: dQc over the VSA block's valid tokens
        const double* cr = dqc + qbv * D;
        const int vsize = P.packed ? clampi(P.bs_q[sv.qblk0 + (i >> lr)], 1, kBlock << lr)
                                   : min(kBlock << lr, P.Sq - (kBlock << lr) * (i >> lr));
        const float inv_size = 1.f / (float)vsize;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const int d0 = 32 * dt + 8 * jj + 4 * hh;
                float r[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) r[e] = fmaf(acc[dt][4 * jj + e], scale, (float)cr[d0 + e] * inv_size);
                *reinterpret_cast<uint2*>(orow + d0) = make_uint2(bf16pair(r[0], r[1]), bf16pair(r[2], r[3]));
            }
    } else if (P.packed) {
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj)
                *reinterpret_cast<uint2*>(orow + 32 * dt + 8 * jj + 4 * hh) = make_uint2(0, 0);
    }
}

// ---------------------------------------------------------------------------
// 6. dK, dV: one workgroup (4 waves) per KV block.  Wave w serves KV tokens
// 32 g .. 32 g + 31 (g = w / 2, one token per lane column) in role r = w % 2:
// role 0 holds the K rows, computes S = Q K^T and P = exp2(S c - lse) and
// accumulates dV^T = dO^T P; role 1 holds the V rows, computes dP - delta =
// dO V^T - delta, takes P from role 0 (float32, through LDS) to form dS =
// P (dP - delta) and accumulates dK^T = Q^T dS.  So no product is computed
// twice, P is the only value exchanged and it flows one way, and a wave
// holds one 32 x D operand and one 32 x D accumulator, which lets three
// waves share a SIMD.
// The query blocks that listed this KV block are walked in stages of 32
// query rows (a block's second half only if it has valid rows there); the Q
// and dO rows of a stage (dual layout: read by rows for S and dP, transposed
// for dV^T and dK^T) and its 32 log-sum-exp and delta values are
// double-buffered in LDS, the copy of stage u + 1 running during stage u:
// 40.5 KiB for D = 128.
// ---------------------------------------------------------------------------
// bf16 B operand of k-step hf (16 rows) of one 32x32 accumulator whose rows
// are the k dimension: k-slots 8 hh .. 8 hh + 7 hold rows 16 hf + 4 hh +
// {0..3, 8..11}, matching tr_read.
__device__ __forceinline__ bf16x8 pack_half(const f32x16& x, int hf) {
    const int b = 8 * hf;
    return as_bf16x8(make_uint4(bf16pair(x[b + 0], x[b + 1]), bf16pair(x[b + 2], x[b + 3]),
                                bf16pair(x[b + 4], x[b + 5]), bf16pair(x[b + 6], x[b + 7])));
}

constexpr int kDkdvThreads = 256;
constexpr int kHalf = kBlock / 2;  // query rows per stage

template <int D>
__global__ __launch_bounds__(kDkdvThreads, 3) void bwd_dkdv_kernel(
    DevProblem P, const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const uint16_t* __restrict__ dout, const float* __restrict__ rs, const int* __restrict__ k2q,
    const int* __restrict__ k2q_num, int ldq, const double* __restrict__ dkc, const double* __restrict__ dvc,
    uint16_t* __restrict__ dk, uint16_t* __restrict__ dv, float c_log2, float scale) {
    constexpr int KS = D / 16, DT = D / 32, CH = D / 8;
    __shared__ __attribute__((aligned(1024))) uint16_t q_tile[2][kHalf * D];
    __shared__ __attribute__((aligned(1024))) uint16_t o_tile[2][kHalf * D];
    __shared__ __attribute__((aligned(16))) float stats[2][2 * kHalf];  // [buffer][lse 0..31, delta 32..63]
    // P of the stage from role 0: [token group][accumulator element / 4][lane]
    __shared__ __attribute__((aligned(16))) float4 xch[2][4][64];

    int s, h, j;
    SeqView sv;
    if (!P.packed) {
        const int N = P.nKV * P.H * P.nseq;
        const int lin = xcd_remap(blockIdx.x, N);
        j = lin % P.nKV;
        const int rest = lin / P.nKV;
        h = rest % P.H;
        s = rest / P.H;
        sv = seq_view(P, s, h);
    } else {
        const int lr = P.ratio >> 1;
        const int N = (P.total_kv << lr) * P.H;
        const int lin = xcd_remap(blockIdx.x, N);
        const int g = lin % (P.total_kv << lr);
        h = lin / (P.total_kv << lr);
        s = seq_of_kvblock(P, g >> lr);
        sv = seq_view(P, s, h);
        j = g - (sv.kvblk0 << lr);
        if (j < 0 || j >= sv.nkv) return;
    }
    const int kvsize = kv_block_size(P, sv, j);  // 0: an empty block of a packed VSA block (no list)
    const int64_t kvoff0 = sv.kv_off + (int64_t)kBlock * j * sv.kv_st;  // element offset of the block's row 0
    const int64_t kb = sv.kvblk_base + j;                               // 64-token block (inverse lists)
    // dKc / dVc are per VSA block of 64 * ratio tokens
    const int lr = P.ratio >> 1;
    const int64_t kbv = sv.kvvsa_base + (j >> lr);
    // wave, token group and role are wave-uniform: readfirstlane puts them in
    // scalar registers, so role-dependent code is branched over, not selected
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63, l32 = lane & 31, hh = lane >> 5;
    const int grp = wave >> 1, role = wave & 1;
    const int kr = 32 * grp + l32;
    const bool kvalid = kr < kvsize;

    // role 0: K^T operand of S = Q K^T; role 1: V^T operand of dP = dO V^T
    bf16x8 bfrag[KS];
    load_b_row<KS>((role ? v : k) + kvoff0 + kr * sv.kv_st, kvalid, hh, bfrag);

    // role 0: dV^T, role 1: dK^T (unscaled), 32 x D each
    f32x16 acc[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[dt][e] = 0.f;

    const int m = __builtin_amdgcn_readfirstlane(clampi(k2q_num[kb], 0, ldq));
    const_int* list = (const_int*)uniform_ptr(k2q + kb * ldq);
    const_int* bs_q = (const_int*)(P.packed ? uniform_ptr(P.bs_q + sv.qblk0) : nullptr);
    const int nq = __builtin_amdgcn_readfirstlane(sv.nq);
    // valid rows of local query block i (the lists hold no empty block)
    auto q_size = [&](int i) -> int {
        return P.packed ? packed_sub_size(bs_q[i >> lr], i & ((1 << lr) - 1)) : min(kBlock, P.Sq - kBlock * i);
    };
    const int x0 = m > 0 ? ((j % kSweepDkdv) * m) / kSweepDkdv : 0;
    auto entry = [&](int x) -> int {
        int pos = x0 + x;
        if (pos >= m) pos -= m;
        return clampi(list[pos], 0, nq - 1);
    };
    constexpr uint32_t kTileBytes = 2u * kHalf * D;
    constexpr uint32_t kStatBytes = 4u * 2 * kHalf;
    const uint32_t off = (uint32_t)lane_src_offset4<CH, kSwzDual>(wave, lane);
    const uint32_t q_lds = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)&q_tile[0][0] + 1024u * wave);
    const uint32_t o_lds = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)&o_tile[0][0] + 1024u * wave);
    const uint32_t st_lds = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)&stats[0][0]);
    // statistics copy: lanes 0..7 fetch the stage's 32 lse values, lanes 8..15
    // its 32 delta values (rows 64 .. 127 of the block's statistics row)
    const uint32_t st_off = lane < 8 ? 16u * lane : 256u + 16u * (lane - 8);
    const int L16 = lane & 15, g16 = lane >> 4;
    const int tr_r = tr_token(L16), tr_d = 16 * (g16 & 1) + 4 * tr_dquad(L16);
    uint32_t t_row[KS], t_tr[DT][2];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) t_row[ks] = row_offset<CH, kSwzDual>(l32, hh, ks);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) t_tr[dt][jj] = tr_offset<CH, kSwzDual>(dt, jj, hh, tr_r, tr_d);
    float4* p_xch = &xch[grp][0][lane];

    // copies of stage (query block i, half hf) into buffer b
    const uint32_t qpitch = __builtin_amdgcn_readfirstlane((uint32_t)(2 * sv.q_st));  // bytes between query rows
    auto issue = [&](int i, int hf, int b) {
        const int64_t o0 = sv.q_off + ((int64_t)kBlock * i + kHalf * hf) * sv.q_st;
        const int valid = min(q_size(i) - kHalf * hf, kHalf);
        load_tile_n<D, kSwzDual, kHalf, 4>(q_lds + kTileBytes * b, q + o0, valid, wave, lane, off, qpitch);
        load_tile_n<D, kSwzDual, kHalf, 4>(o_lds + kTileBytes * b, dout + o0, valid, wave, lane, off, qpitch);
        if (wave == 0 && lane < 16)
            dma_16B(uniform_ptr(rs + (sv.qblk_base + i) * kStatRow + kHalf * hf), st_off, st_lds + kStatBytes * b);
    };

    __builtin_amdgcn_s_waitcnt(0);
    int x = 0, hf = 0;
    int ci = m > 0 ? entry(0) : 0;  // query block of the current stage
    if (m > 0) issue(ci, 0, 0);
    int buf = 0;
    while (x < m) {
        // the stage after (x, hf): the block's second half if it has valid rows
        int nx = x, nhf = 1, ni = ci;
        if (hf == 1 || q_size(ci) <= kHalf) {
            nx = x + 1;
            nhf = 0;
            ni = nx < m ? entry(nx) : 0;
        }
        wait_vmcnt<0>();
        wg_barrier();  // this stage is in LDS; every wave is done with the other buffer
        if (nx < m) issue(ni, nhf, buf ^ 1);
        const uint16_t* qt = q_tile[buf];
        const uint16_t* ot = o_tile[buf];
        const float* st = stats[buf];
        // role 0: S = Q K^T; role 1: dP = dO V^T; rows = the stage's 32 queries
        // 8 (e / 4) + 4 hh + e % 4, lane column = KV token
        f32x16 a;
#pragma unroll
        for (int e = 0; e < 16; ++e) a[e] = 0.f;
        {
            const uint16_t* my_tile = role ? ot : qt;
            bf16x8 ta = row_read<CH>(my_tile, t_row[0], 0);
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                bf16x8 tn = ta;
                if (ks + 1 < KS) tn = row_read<CH>(my_tile, t_row[ks + 1], 0);
                __builtin_amdgcn_sched_barrier(0);
                a = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ta, bfrag[ks], a, 0, 0, 0);
                __builtin_amdgcn_sched_barrier(0);
                ta = tn;
            }
        }
        // role 0: P = exp2(S c - lse[row]) (padding rows have lse = +inf: P = 0;
        // columns past a partial KV block: P = 0); role 1: dP - delta[row]
        if (role == 0) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const float4 st4 = *reinterpret_cast<const float4*>(st + 8 * g + 4 * hh);
                const float sv4[4] = {st4.x, st4.y, st4.z, st4.w};
#pragma unroll
                for (int e = 0; e < 4; ++e) a[4 * g + e] = __builtin_amdgcn_exp2f(fmaf(a[4 * g + e], c_log2, -sv4[e]));
            }
            if (kvsize < kBlock && !kvalid) {
#pragma unroll
                for (int e = 0; e < 16; ++e) a[e] = 0.f;
            }
        } else {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const float4 st4 = *reinterpret_cast<const float4*>(st + kHalf + 8 * g + 4 * hh);
                const float sv4[4] = {st4.x, st4.y, st4.z, st4.w};
#pragma unroll
                for (int e = 0; e < 4; ++e) a[4 * g + e] -= sv4[e];
            }
        }
        if (role == 0) {
#pragma unroll
            for (int e4 = 0; e4 < 4; ++e4)
                p_xch[64 * e4] = make_float4(a[4 * e4], a[4 * e4 + 1], a[4 * e4 + 2], a[4 * e4 + 3]);
        }
        wg_barrier();  // P of this stage is in LDS
        // the bf16 B operands of the stage's two k-steps: P (role 0) or
        // dS = P (dP - delta) (role 1)
        bf16x8 opb[2];
        if (role == 0) {
#pragma unroll
            for (int k2 = 0; k2 < 2; ++k2) opb[k2] = pack_half(a, k2);
        } else {
            f32x16 dm;
#pragma unroll
            for (int e4 = 0; e4 < 4; ++e4) {
                const float4 p4 = p_xch[64 * e4];
                dm[4 * e4 + 0] = p4.x * a[4 * e4 + 0];
                dm[4 * e4 + 1] = p4.y * a[4 * e4 + 1];
                dm[4 * e4 + 2] = p4.z * a[4 * e4 + 2];
                dm[4 * e4 + 3] = p4.w * a[4 * e4 + 3];
            }
#pragma unroll
            for (int k2 = 0; k2 < 2; ++k2) opb[k2] = pack_half(dm, k2);
        }
        // role 0: dV^T += dO^T P; role 1: dK^T += Q^T dS, over all of d; the
        // transposed operand read one product ahead
        {
            const uint16_t* tt = role ? qt : ot;
            bf16x8 ta = tr_read<CH>(tt, t_tr[0][0], t_tr[0][1], 0);
#pragma unroll
            for (int y = 0; y < 2 * DT; ++y) {
                const int k2 = y / DT, dt = y % DT;
                bf16x8 na = ta;
                if (y + 1 < 2 * DT) {
                    const int k2n = (y + 1) / DT, dtn = (y + 1) % DT;
                    na = tr_read<CH>(tt, t_tr[dtn][0], t_tr[dtn][1], k2n);
                }
                __builtin_amdgcn_sched_barrier(0);
                acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ta, opb[k2], acc[dt], 0, 0, 0);
                __builtin_amdgcn_sched_barrier(0);
                ta = na;
            }
        }
        x = nx;
        hf = nhf;
        ci = ni;
        buf ^= 1;
    }

    // lane holds dV (role 0) / dK (role 1) [kr][32 dt + 8 (e / 4) + 4 hh + e % 4]
    uint16_t* row = (role ? dk : dv) + kvoff0 + kr * sv.kv_st;
    if (kvalid) {
        // the gradient through the block means, over the VSA block's valid tokens
        const double* cr = (role ? dkc : dvc) + kbv * D;
        const int vsize = P.packed ? clampi(P.bs_kv[sv.kvblk0 + (j >> lr)], 1, kBlock << lr)
                                   : min(kBlock << lr, P.Skv - (kBlock << lr) * (j >> lr));
        const float inv_size = 1.f / (float)vsize;
        const float mul = role ? scale : 1.f;  // dK = Q^T dS / sqrt(D)
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const int d0 = 32 * dt + 8 * jj + 4 * hh;
                float r[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) r[e] = fmaf(acc[dt][4 * jj + e], mul, (float)cr[d0 + e] * inv_size);
                *reinterpret_cast<uint2*>(row + d0) = make_uint2(bf16pair(r[0], r[1]), bf16pair(r[2], r[3]));
            }
    } else if (P.packed) {
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj)
                *reinterpret_cast<uint2*>(row + 32 * dt + 8 * jj + 4 * hh) = make_uint2(0, 0);
    }
}

template <int D>
hipError_t launch_all(const DevProblem& P, const BwdArgs& A, hipStream_t st) {
    const int seqs = P.nseq;
    // the coarse branch works on VSA blocks (64 * ratio tokens), the
    // attention kernels and the inverse lists on 64-token blocks
    const DevProblem CP = coarse_view(P);
    const int qgrid = P.packed ? P.total_q : P.nQB;
    const int maxq = P.packed ? P.max_q : P.nQB;
    const int maxkv = P.packed ? P.max_kv : P.nKVB;
    const int maxq64 = P.packed ? P.max_q * P.ratio : P.nQ;
    const int maxkv64 = P.packed ? P.max_kv * P.ratio : P.nKV;
    const double scale = 1.0 / sqrt((double)D);
    const float c_log2 = (float)(1.4426950408889634 * scale);
    hipError_t e;
    // 1. combine backward
    const dim3 cgrid(qgrid, P.H, P.packed ? 1 : seqs);
    switch (A.gate_mode) {
        case VSA_GATE_NONE:
            hipLaunchKernelGGL((bwd_combine_kernel<D, VSA_GATE_NONE>), cgrid, dim3(kThreads), 0, st, P, A.dout,
                               A.out_s, A.out_c, A.gate, A.gs0, A.gs1, A.gs2, A.lse, A.rs, A.doc, A.dgate);
            break;
        case VSA_GATE_TOKEN:
            hipLaunchKernelGGL((bwd_combine_kernel<D, VSA_GATE_TOKEN>), cgrid, dim3(kThreads), 0, st, P, A.dout,
                               A.out_s, A.out_c, A.gate, A.gs0, A.gs1, A.gs2, A.lse, A.rs, A.doc, A.dgate);
            break;
        case VSA_GATE_FULL:
            hipLaunchKernelGGL((bwd_combine_kernel<D, VSA_GATE_FULL>), cgrid, dim3(kThreads), 0, st, P, A.dout,
                               A.out_s, A.out_c, A.gate, A.gs0, A.gs1, A.gs2, A.lse, A.rs, A.doc, A.dgate);
            break;
        default: return hipErrorInvalidValue;
    }
    if ((e = hipGetLastError()) != hipSuccess) return e;
    // 2. block means (unless the caller passed the forward's)
    if (!A.pooled && (e = launch_pool(P, A.q, A.k, A.v, A.qc, A.kc, A.vc, st)) != hipSuccess) return e;
    // 3. coarse backward
    if ((e = launch_coarse_scores(CP, A.qc, A.kc, A.pbuf, st)) != hipSuccess) return e;
    if ((e = launch_coarse_scores(CP, A.doc, A.vc, A.dsbuf, st)) != hipSuccess) return e;
    const int64_t crows = (int64_t)seqs * P.H * maxq;
    hipLaunchKernelGGL(bwd_coarse_softmax_kernel, dim3((unsigned)((crows + 3) / 4)), dim3(kThreads), 0, st, CP,
                       A.pbuf, A.dsbuf, maxkv, maxq, scale);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL((bwd_coarse_mm_kernel<D, false>), dim3(kMmSplit * ((maxq + 63) / 64), P.H, seqs),
                       dim3(kThreads), 0, st,
                       CP, A.dsbuf, A.kc, A.dqc, maxkv, maxq, scale);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL((bwd_coarse_mm_kernel<D, true>), dim3(kMmSplit * ((maxkv + 63) / 64), P.H, seqs),
                       dim3(kThreads), 0, st,
                       CP, A.dsbuf, A.qc, A.dkc, maxkv, maxq, scale);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL((bwd_coarse_mm_kernel<D, true>), dim3(kMmSplit * ((maxkv + 63) / 64), P.H, seqs),
                       dim3(kThreads), 0, st,
                       CP, A.pbuf, A.doc, A.dvc, maxkv, maxq, 1.0);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    // 4. inverse routing (64-token blocks)
    hipLaunchKernelGGL(bwd_k2q_kernel, dim3((maxkv64 + 3) / 4, P.H, seqs), dim3(kThreads), 0, st, P, A.idx, A.num,
                       A.k2q, A.k2q_num, maxq64);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    // 5. dQ, 6. dK / dV
    const int64_t nq_all = P.packed ? (int64_t)P.total_q * P.ratio * P.H : (int64_t)P.nQ * P.H * P.nseq;
    const int64_t nkv_all = P.packed ? (int64_t)P.total_kv * P.ratio * P.H : (int64_t)P.nKV * P.H * P.nseq;
    hipLaunchKernelGGL(bwd_dq_kernel<D>, dim3((unsigned)nq_all), dim3(kAttnThreads), 0, st, P, A.q, A.k, A.v, A.dout,
                       A.rs, A.idx, A.num, A.dqc, A.dq, c_log2, (float)scale);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(bwd_dkdv_kernel<D>, dim3((unsigned)nkv_all), dim3(kDkdvThreads), 0, st, P, A.q, A.k, A.v,
                       A.dout, A.rs, A.k2q, A.k2q_num, maxq64, A.dkc, A.dvc, A.dk, A.dv, c_log2, (float)scale);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_backward(const DevProblem& P, const BwdArgs& A, hipStream_t st) {
    const int64_t nq_all = P.packed ? (int64_t)P.total_q * P.ratio * P.H : (int64_t)P.nQ * P.H * P.nseq;
    const int64_t nkv_all = P.packed ? (int64_t)P.total_kv * P.ratio * P.H : (int64_t)P.nKV * P.H * P.nseq;
    if (nq_all <= 0 || nq_all > 0x7fffffff || nkv_all <= 0 || nkv_all > 0x7fffffff) return hipErrorInvalidValue;
    return P.D == 128 ? launch_all<128>(P, A, st) : launch_all<64>(P, A, st);
}

}  // namespace vsa
