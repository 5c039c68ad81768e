// Block mean-pooling of Q, K and V into float64 (the compression branch's
// block means; "[perf] avoid full-sequence materialization in VSA
// coarse/sparse combine", Problem and Notes).
//
// HBM-bound streaming kernel.  Thread (block, slice s, c) owns the 16-byte
// chunk c (8 consecutive d) of tokens s, s + 4, s + 8, ... of one VSA block
// (64 * ratio tokens, ratio 1, 2 or 4) and walks them with independent,
// non-temporal 16-byte loads (16 in flight per thread: a whole 64-token block
// in one round; both measured 7 % faster than 8 cached loads), accumulating 8
// sums in float64 registers; the 4 slices of a
// chunk then add their sums with lane shuffles (no LDS).  The 4 CH threads of
// a block (CH = D/8) read 4 consecutive token rows per load instruction, 4
// contiguous 16*CH-byte segments, so every instruction of a wave is fully
// coalesced, and splitting a block over 4 slices gives the launch enough
// short workgroups to fill the chip evenly.  Sums of at most 256 bf16 values
// in float64 are exact for any realistic data, so the result does not depend
// on the order of the additions; the mean is an IEEE division by the block's
// valid-token count.
#include "vsa_internal.hpp"

namespace vsa {
namespace {

constexpr int kPoolThreads = 256;
constexpr int kUnroll = 16;
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
constexpr int kSlices = 4;  // threads sharing one (block, chunk)

__device__ __forceinline__ double bf16_lo(uint32_t w) { return (double)__uint_as_float(w << 16); }
__device__ __forceinline__ double bf16_hi(uint32_t w) { return (double)__uint_as_float(w & 0xffff0000u); }

template <int D>
__global__ __launch_bounds__(kPoolThreads) void pool_kernel(DevProblem P, const uint16_t* __restrict__ q,
                                                            const uint16_t* __restrict__ k,
                                                            const uint16_t* __restrict__ v,
                                                            double* __restrict__ qc,
                                                            double* __restrict__ kc,
                                                            double* __restrict__ vc) {
    constexpr int CH = D / 8;                        // 16-byte chunks per token row
    constexpr int TPB = CH * kSlices;                // threads per block (64 or 32: within a wave)
    constexpr int BPG = kPoolThreads / TPB;          // blocks per workgroup
    const int which = blockIdx.z % 3;                // 0 q, 1 k, 2 v
    const int b = blockIdx.z / 3;                    // batch item (dense) or 0 (packed)
    const int h = blockIdx.y;
    const int blk = blockIdx.x * BPG + threadIdx.x / TPB;
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

}  // namespace

hipError_t launch_pool(const DevProblem& P, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                       double* qc, double* kc, double* vc, hipStream_t st) {
    const int bpg = kPoolThreads / (P.D / 8 * kSlices);
    const int nb = P.packed ? max(P.total_q, P.total_kv) : max(P.nQB, P.nKVB);
    const dim3 grid((nb + bpg - 1) / bpg, P.H, P.packed ? 3 : 3 * P.nseq);
    if (P.D == 128)
        hipLaunchKernelGGL(pool_kernel<128>, grid, dim3(kPoolThreads), 0, st, P, q, k, v, qc, kc, vc);
    else
        hipLaunchKernelGGL(pool_kernel<64>, grid, dim3(kPoolThreads), 0, st, P, q, k, v, qc, kc, vc);
    return hipGetLastError();
}

}  // namespace vsa
