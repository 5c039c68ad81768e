// Block mean-pooling of Q, K and V into float64: the per-workgroup body,
// shared by the pool kernel and by the coarse score kernel, which pools V in
// workgroups of its own while the scores of the already pooled Q and K are
// computed.  (Kernel design notes in pool.hip.)
#pragma once

#include "vsa_internal.hpp"

namespace vsa {
namespace pool {

constexpr int kPoolThreads = 256;
constexpr int kUnroll = 16;
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
constexpr int kSlices = 4;  // threads sharing one (block, chunk)

__device__ __forceinline__ double bf16_lo(uint32_t w) { return (double)__uint_as_float(w << 16); }
__device__ __forceinline__ double bf16_hi(uint32_t w) { return (double)__uint_as_float(w & 0xffff0000u); }

// Pools the BPG blocks of workgroup column bx of tensor `which` (0 q, 1 k,
// 2 v) for batch item b (dense; 0 packed) and head h; kPoolThreads threads.
template <int D>
__device__ __forceinline__ void pool_group(const DevProblem& P, const uint16_t* __restrict__ q,
                                           const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
                                           double* __restrict__ qc, double* __restrict__ kc,
                                           double* __restrict__ vc, int which, int b, int h, int bx) {
    constexpr int CH = D / 8;                        // 16-byte chunks per token row
    constexpr int TPB = CH * kSlices;                // threads per block (64 or 32: within a wave)
    constexpr int BPG = kPoolThreads / TPB;          // blocks per workgroup
    const int blk = bx * BPG + threadIdx.x / TPB;
    const int c = threadIdx.x % CH;
    const int sl = (threadIdx.x % TPB) / CH;         // token slice

    int64_t off0, st, out_row;  // element offset of the block's first row, row stride
    int size;
    if (!P.packed) {
        const int nb = which == 0 ? P.nQB : P.nKVB;
        if (blk >= nb) return;
        const int S = which == 0 ? P.Sq : P.Skv;
        const int bt = kBlock * P.ratio;  // tokens per block
        size = min(bt, S - bt * blk);
        st = which == 0 ? P.q_st : P.kv_st;
        off0 = (which == 0 ? (int64_t)b * P.q_sb + (int64_t)h * P.q_sh : (int64_t)b * P.kv_sb + (int64_t)h * P.kv_sh) +
               (int64_t)bt * blk * st;
        out_row = ((int64_t)b * P.H + h) * nb + blk;
    } else {
        const int nb = which == 0 ? P.total_q : P.total_kv;
        if (blk >= nb) return;
        const int bt = kBlock * P.ratio;  // slots per block
        size = clampi(which == 0 ? P.bs_q[blk] : P.bs_kv[blk], 1, bt);
        st = D;
        off0 = ((int64_t)h * nb + blk) * bt * D;
        out_row = (int64_t)h * nb + blk;
    }
    const uint16_t* src = (which == 0 ? q : (which == 1 ? k : v)) + off0 + 8 * c;
    double* dst = which == 0 ? qc : (which == 1 ? kc : vc);

    double acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.0;
    for (int t0 = sl; t0 < size; t0 += kSlices * kUnroll) {
        uint4 w[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int t = t0 + kSlices * u;
            u32x4 x = {0, 0, 0, 0};
            if (t < size) x = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src + (int64_t)t * st));
            w[u] = make_uint4(x[0], x[1], x[2], x[3]);
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            acc[0] += bf16_lo(w[u].x); acc[1] += bf16_hi(w[u].x);
            acc[2] += bf16_lo(w[u].y); acc[3] += bf16_hi(w[u].y);
            acc[4] += bf16_lo(w[u].z); acc[5] += bf16_hi(w[u].z);
            acc[6] += bf16_lo(w[u].w); acc[7] += bf16_hi(w[u].w);
        }
    }
    // the slices of a chunk are lanes CH apart inside one wave
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        acc[e] += __shfl_xor(acc[e], CH);
        acc[e] += __shfl_xor(acc[e], 2 * CH);
    }
    if (sl != 0) return;
    const double cnt = (double)size;
    double2* o = reinterpret_cast<double2*>(dst + out_row * D + 8 * c);
#pragma unroll
    for (int e = 0; e < 4; ++e) o[e] = make_double2(acc[2 * e] / cnt, acc[2 * e + 1] / cnt);
}


// workgroup columns of the pool grid (blocks of one tensor, batch item and head)
__host__ __device__ inline int pool_columns(const DevProblem& P) {
    const int bpg = kPoolThreads / (P.D / 8 * kSlices);
    const int nb = P.packed ? max(P.total_q, P.total_kv) : max(P.nQB, P.nKVB);
    return (nb + bpg - 1) / bpg;
}

}  // namespace pool
}  // namespace vsa
