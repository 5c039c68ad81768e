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
#include "pool_common.hpp"

namespace vsa {
namespace {

using namespace pool;

// grid (columns, H, 3 or 2 tensors x batch items): z = tensor + ntens * b,
// tensors q, k (, v)
template <int D>
__global__ __launch_bounds__(kPoolThreads) void pool_kernel(DevProblem P, const uint16_t* __restrict__ q,
                                                            const uint16_t* __restrict__ k,
                                                            const uint16_t* __restrict__ v,
                                                            double* __restrict__ qc,
                                                            double* __restrict__ kc,
                                                            double* __restrict__ vc, int ntens) {
    pool_group<D>(P, q, k, v, qc, kc, vc, blockIdx.z % ntens, blockIdx.z / ntens, blockIdx.y, blockIdx.x);
}

hipError_t launch(const DevProblem& P, const uint16_t* q, const uint16_t* k, const uint16_t* v, double* qc,
                  double* kc, double* vc, int ntens, hipStream_t st) {
    const dim3 grid(pool_columns(P), P.H, P.packed ? ntens : ntens * P.nseq);
    if (P.D == 128)
        hipLaunchKernelGGL(pool_kernel<128>, grid, dim3(kPoolThreads), 0, st, P, q, k, v, qc, kc, vc, ntens);
    else
        hipLaunchKernelGGL(pool_kernel<64>, grid, dim3(kPoolThreads), 0, st, P, q, k, v, qc, kc, vc, ntens);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_pool(const DevProblem& P, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                       double* qc, double* kc, double* vc, hipStream_t st) {
    return launch(P, q, k, v, qc, kc, vc, 3, st);
}

hipError_t launch_pool_qk(const DevProblem& P, const uint16_t* q, const uint16_t* k, double* qc, double* kc,
                          hipStream_t st) {
    return launch(P, q, k, nullptr, qc, kc, nullptr, 2, st);
}

}  // namespace vsa
