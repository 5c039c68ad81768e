// Block mean-pooling of Q, K and V into float64 (the compression branch's
// block means; "[perf] avoid full-sequence materialization in VSA
// coarse/sparse combine", Problem and Notes).
//
// One workgroup of 256 threads pools one 64-token block of one head of one
// tensor.  Thread (g, c) reads the 16-byte chunk c (8 consecutive d) of
// tokens g, g + G, ... and accumulates them in float64; the G partial sums of
// each d are then added through LDS.  Sums of at most 64 bf16 values in
// float64 are exact for any realistic data, so the result does not depend on
// the order of the additions; the mean is an IEEE division by the block's
// valid-token count.  HBM-bound: every input byte is read once.
#include "vsa_internal.hpp"

namespace vsa {
namespace {

constexpr int kPoolThreads = 256;

__device__ __forceinline__ double bf16_lo(uint32_t w) { return (double)__uint_as_float(w << 16); }
__device__ __forceinline__ double bf16_hi(uint32_t w) { return (double)__uint_as_float(w & 0xffff0000u); }

template <int D>
__global__ __launch_bounds__(kPoolThreads) void pool_kernel(DevProblem P, const uint16_t* __restrict__ q,
                                                            const uint16_t* __restrict__ k,
                                                            const uint16_t* __restrict__ v,
                                                            double* __restrict__ qc,
                                                            double* __restrict__ kc,
                                                            double* __restrict__ vc) {
    constexpr int CH = D / 8;                // 16-byte chunks per row
    constexpr int G = kPoolThreads / CH;     // token groups
    constexpr int TPG = kBlock / G;          // tokens per group
    __shared__ double part[G][D];

    const int which = blockIdx.z % 3;  // 0 q, 1 k, 2 v
    const int b = blockIdx.z / 3;      // batch item (dense) or 0 (packed)
    const int h = blockIdx.y;
    const int blk = blockIdx.x;

    const uint16_t* src;
    double* dst;
    int64_t row0, out_row;
    int size;
    if (!P.packed) {
        const int nb = which == 0 ? P.nQ : P.nKV;
        if (blk >= nb) return;
        const int S = which == 0 ? P.Sq : P.Skv;
        size = min(kBlock, S - kBlock * blk);
        const int64_t sh = (int64_t)b * P.H + h;
        row0 = sh * S + (int64_t)kBlock * blk;
        out_row = sh * nb + blk;
    } else {
        const int nb = which == 0 ? P.total_q : P.total_kv;
        if (blk >= nb) return;
        size = clampi(which == 0 ? P.bs_q[blk] : P.bs_kv[blk], 1, kBlock);
        row0 = ((int64_t)h * nb + blk) * kBlock;
        out_row = (int64_t)h * nb + blk;
    }
    src = which == 0 ? q : (which == 1 ? k : v);
    dst = which == 0 ? qc : (which == 1 ? kc : vc);

    const int c = threadIdx.x % CH;
    const int g = threadIdx.x / CH;
    double acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.0;
    uint4 w[TPG];
#pragma unroll
    for (int r = 0; r < TPG; ++r) {
        const int t = g + G * r;
        if (t < size)
            w[r] = *reinterpret_cast<const uint4*>(src + (row0 + t) * D + 8 * c);
        else
            w[r] = make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int r = 0; r < TPG; ++r) {
        acc[0] += bf16_lo(w[r].x); acc[1] += bf16_hi(w[r].x);
        acc[2] += bf16_lo(w[r].y); acc[3] += bf16_hi(w[r].y);
        acc[4] += bf16_lo(w[r].z); acc[5] += bf16_hi(w[r].z);
        acc[6] += bf16_lo(w[r].w); acc[7] += bf16_hi(w[r].w);
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) part[g][8 * c + e] = acc[e];
    __syncthreads();
    for (int d = threadIdx.x; d < D; d += kPoolThreads) {
        double s = 0.0;
#pragma unroll
        for (int gg = 0; gg < G; ++gg) s += part[gg][d];
        dst[out_row * D + d] = s / (double)size;
    }
}

}  // namespace

hipError_t launch_pool(const DevProblem& P, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                       double* qc, double* kc, double* vc, hipStream_t st) {
    dim3 grid, block(kPoolThreads);
    if (!P.packed)
        grid = dim3(max(P.nQ, P.nKV), P.H, 3 * P.nseq);
    else
        grid = dim3(max(P.total_q, P.total_kv), P.H, 3);
    if (P.D == 128)
        hipLaunchKernelGGL(pool_kernel<128>, grid, block, 0, st, P, q, k, v, qc, kc, vc);
    else
        hipLaunchKernelGGL(pool_kernel<64>, grid, block, 0, st, P, q, k, v, qc, kc, vc);
    return hipGetLastError();
}

}  // namespace vsa
