// Index maps of the block-sparse attention kernel, usable on host and
// device so that their coverage and bank behaviour can be checked on a CPU.
#pragma once

#include <hip/hip_runtime.h>

namespace vsa {

// LDS position of KV token t inside its 16-token group.  The MFMA k-slot
// 8*hh + 4*jj + ii of the O^T = V^T P^T product stands for token
// 16*s + 8*jj + 4*hh + ii, which is where the S^T accumulator of lane half hh
// holds it; storing token t at this position makes each lane's 8 k-slots one
// contiguous 16-byte group.
__host__ __device__ inline int tok_pos(int t) {
    return (t & ~15) | (((t >> 2) & 1) << 3) | (((t >> 3) & 1) << 2) | (t & 3);
}

// Element offset of V^T[d][pos] in LDS: rows of 64 tokens (128 bytes), the
// eight 16-byte groups of a row XOR-swizzled by (d ^ d/8) mod 8 so that
// (a) eight consecutive rows read at one group hit eight different groups
// and (b) rows 8 apart written at one group do too.
__host__ __device__ inline int vt_off(int d, int pos) {
    const int swz = (d ^ (d >> 3)) & 7;
    return d * 64 + 8 * ((pos >> 3) ^ swz) + (pos & 7);
}

// Staging unit u (0 .. 16*CH-1) -> 4-token group g4 and 16-byte chunk c.
// Within a 16-lane quarter-wave the eight chunks pair with two token groups
// whose LDS positions differ by 4 elements, so a quarter-wave's ds_write_b64
// covers 16 distinct 8-byte bank pairs.
template <int CH>
__host__ __device__ inline void stage_unit(int u, int* g4, int* c) {
    const int ul = u & 63, uw = u >> 6;
    const int clo = ul & 7, gl = 2 * ((ul >> 3) & 1) + ((ul >> 4) & 1), b5 = ul >> 5;
    if (CH == 16) {
        *c = clo + 8 * b5;
        *g4 = 4 * uw + gl;
    } else {
        *c = clo;
        *g4 = 4 * (2 * uw + b5) + gl;
    }
}

// Workgroups are handed to the 8 XCDs round-robin by linear id.  Re-number
// them so that each XCD walks a contiguous range of logical work items (the
// query blocks of one head stay on one XCD and share its L2).  A bijection
// of [0, N).
__host__ __device__ inline int xcd_remap(int n, int N) {
    constexpr int X = 8;
    const int q = N / X, r = N % X;
    const int x = n % X, k = n / X;
    return (x < r) ? x * (q + 1) + k : r * (q + 1) + (x - r) * q + k;
}

}  // namespace vsa
