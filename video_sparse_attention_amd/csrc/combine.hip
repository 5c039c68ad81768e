// In-place combine of the block-resolution coarse output with the sparse
// output: out = bf16(fma(out_c[block], gate, out)) or bf16(out_c[block] + out).
// ("[perf] avoid full-sequence materialization in VSA coarse/sparse combine",
// Problem and Change: out_c stays [.., n_blocks, 1, D] and broadcasts over the
// block's tokens, accumulated into the sparse output in place; follow-up:
// strict shapes, the gate accepted as a transposed view.)
//
// HBM-bound.  One workgroup of 256 threads updates one 64-token block: each
// thread owns one 16-byte chunk (8 consecutive d) for 4 tokens, keeps the
// matching 8 floats of out_c in registers, and streams out with 16-byte loads
// and stores, both non-temporal (each byte of out is touched once: keeping it
// out of the caches measured 10 % faster in the steady state).  No temporary
// is allocated; algorithmic traffic per block is 2 * size * D * 2 bytes of
// out, D * 4 bytes of out_c and the gate.
#include "vsa_internal.hpp"

namespace vsa {
namespace {

constexpr int kCombThreads = 256;
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float lo_f(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_f(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ uint32_t pack2(float a, float b) {
    const __bf16 x = (__bf16)a, y = (__bf16)b;
    return (uint32_t)__builtin_bit_cast(uint16_t, x) | ((uint32_t)__builtin_bit_cast(uint16_t, y) << 16);
}

template <int D, int MODE>
__global__ __launch_bounds__(kCombThreads) void combine_kernel(DevProblem P, const float* __restrict__ out_c,
                                                               const uint16_t* __restrict__ gate,
                                                               int64_t gs0, int64_t gs1, int64_t gs2,
                                                               uint16_t* __restrict__ out) {
    constexpr int CH = D / 8;
    constexpr int TG = kCombThreads / CH;  // token groups
    constexpr int TPT = kBlock / TG;       // tokens per thread

    int64_t off0, st, cb;  // element offset of the block's first row, row stride, row of out_c
    int size;
    int64_t g_base;        // gate element offset of token 0 of the block
    if (!P.packed) {
        const int blk = blockIdx.x, h = blockIdx.y, b = blockIdx.z;  // 64-token block
        if (blk >= P.nQ) return;
        const int64_t sh = (int64_t)b * P.H + h;
        size = min(kBlock, P.Sq - kBlock * blk);
        st = P.q_st;
        off0 = (int64_t)b * P.q_sb + (int64_t)h * P.q_sh + (int64_t)kBlock * blk * st;
        cb = sh * P.nQB + blk / P.ratio;  // out_c is at VSA-block resolution
        g_base = (int64_t)b * gs0 + (int64_t)h * gs1 + (int64_t)kBlock * blk * gs2;
    } else {  // 64-token block blk of the packed slots, in VSA block blk / ratio
        const int blk = blockIdx.x, h = blockIdx.y;
        const int lr = P.ratio >> 1;
        if (blk >= (P.total_q << lr)) return;
        size = packed_sub_size(P.bs_q[blk >> lr], blk & ((1 << lr) - 1));
        st = D;
        off0 = ((int64_t)h * (P.total_q << lr) + blk) * kBlock * D;
        cb = (int64_t)h * P.total_q + (blk >> lr);
        g_base = (int64_t)h * gs1 + (int64_t)kBlock * blk * gs2;
    }
    const int c = threadIdx.x % CH;
    const int tg = threadIdx.x / CH;
    const float4 ca = *reinterpret_cast<const float4*>(out_c + cb * D + 8 * c);
    const float4 cbv = *reinterpret_cast<const float4*>(out_c + cb * D + 8 * c + 4);
    const float oc[8] = {ca.x, ca.y, ca.z, ca.w, cbv.x, cbv.y, cbv.z, cbv.w};

    uint4 w[TPT];
    float gt[TPT];
    uint4 gf[TPT];
#pragma unroll
    for (int r = 0; r < TPT; ++r) {
        const int t = tg + TG * r;
        if (t < size) {
            const u32x4 x = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(out + off0 + t * st + 8 * c));
            w[r] = make_uint4(x[0], x[1], x[2], x[3]);
            if (MODE == 1) gt[r] = __uint_as_float((uint32_t)gate[g_base + (int64_t)t * gs2] << 16);
            if (MODE == 2) gf[r] = *reinterpret_cast<const uint4*>(gate + g_base + (int64_t)t * gs2 + 8 * c);
        }
    }
#pragma unroll
    for (int r = 0; r < TPT; ++r) {
        const int t = tg + TG * r;
        if (t >= size) continue;
        const uint32_t in[4] = {w[r].x, w[r].y, w[r].z, w[r].w};
        uint32_t res[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            float a = lo_f(in[e]), b = hi_f(in[e]);
            if (MODE == 0) {
                a = oc[2 * e] + a;
                b = oc[2 * e + 1] + b;
            } else if (MODE == 1) {
                a = __builtin_fmaf(oc[2 * e], gt[r], a);
                b = __builtin_fmaf(oc[2 * e + 1], gt[r], b);
            } else {
                const uint32_t gw = e == 0 ? gf[r].x : (e == 1 ? gf[r].y : (e == 2 ? gf[r].z : gf[r].w));
                a = __builtin_fmaf(oc[2 * e], lo_f(gw), a);
                b = __builtin_fmaf(oc[2 * e + 1], hi_f(gw), b);
            }
            res[e] = pack2(a, b);
        }
        const u32x4 y = {res[0], res[1], res[2], res[3]};
        __builtin_nontemporal_store(y, reinterpret_cast<u32x4*>(out + off0 + t * st + 8 * c));
    }
}

template <int D>
hipError_t launch_d(const DevProblem& P, const float* out_c, const uint16_t* gate, int mode,
                    int64_t gs0, int64_t gs1, int64_t gs2, uint16_t* out, hipStream_t st) {
    dim3 grid = P.packed ? dim3(P.total_q * P.ratio, P.H, 1) : dim3(P.nQ, P.H, P.nseq);
    dim3 block(kCombThreads);
    if (mode == 0)
        hipLaunchKernelGGL((combine_kernel<D, 0>), grid, block, 0, st, P, out_c, gate, gs0, gs1, gs2, out);
    else if (mode == 1)
        hipLaunchKernelGGL((combine_kernel<D, 1>), grid, block, 0, st, P, out_c, gate, gs0, gs1, gs2, out);
    else
        hipLaunchKernelGGL((combine_kernel<D, 2>), grid, block, 0, st, P, out_c, gate, gs0, gs1, gs2, out);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_combine(const DevProblem& P, const float* out_c, const uint16_t* gate, int mode,
                          int64_t gs0, int64_t gs1, int64_t gs2, uint16_t* out, hipStream_t st) {
    if (P.D == 128) return launch_d<128>(P, out_c, gate, mode, gs0, gs1, gs2, out, st);
    return launch_d<64>(P, out_c, gate, mode, gs0, gs1, gs2, out, st);
}

}  // namespace vsa
