// Index maps of the block-sparse attention kernel, usable on host and
// device so that their coverage and LDS bank behaviour can be checked on a
// CPU.
//
// A KV block lives in LDS as two row-major tiles, K[64][D] and V[64][D]
// (bf16), written 16 bytes per lane by direct global->LDS loads.  Lane l of
// a wave's load instruction always lands at LDS byte base + 16 l, so the
// layout is chosen by which global 16-byte chunk each lane fetches: the
// chunks of every row are XOR-permuted by a function of the row so that the
// MFMA operand reads hit distinct banks.
#pragma once

#include <hip/hip_runtime.h>

namespace vsa {

// XOR applied to the 16-byte chunk index of K row `row` (CH chunks per row).
// The S^T = K Q^T A operand reads one chunk of 32 consecutive rows per
// instruction (ds_read_b128); with 64 banks a pass serves 16 lanes = 16
// consecutive rows, which then fall on 16 different chunk columns.  Copy
// instruction n of a lane covers row 8n + r0 (D = 128) or 16n + r0 (D = 64),
// so the swizzle seen by a lane only depends on n through bit 3 of the row
// (D = 128): its source offset is lane_off[n & 1] + 2048 n.
template <int CH>
__host__ __device__ inline int k_swz(int row) {
    return CH == 16 ? (row & 15) : ((row & 7) ^ ((row >> 3) & 1));
}

// XOR applied to the chunk index of V row `row`.  The O^T = V^T P^T A
// operand is read with ds_read_b64_tr_b16: each 16-lane group fetches a
// 4-token x 16-d sub-block; rows 4a..4a+3 are spread over four disjoint
// chunk pairs (and four disjoint chunk quads for the 32 lanes of a pass).
// Depends on row & 3 only.
template <int CH>
__host__ __device__ inline int v_swz(int row) {
    return (4 * (row & 3) + 2 * ((row >> 1) & 1)) & (CH - 1);
}

// XOR for a tile read both ways: by rows (ds_read_b128, as K above) and
// transposed (ds_read_b64_tr_b16, as V above), which the backward kernels do
// with K, Q and dO.  Row reads need distinct values over 16 consecutive rows
// (D = 128) or over the 8 rows of one parity among 16 (D = 64, two rows per
// 256 bytes); a transposed read of rows 4a..4a+3 needs the four (D = 128) or
// the two same-parity (D = 64) rows in different groups of four chunks.
// D = 128: 4 (row & 3) + ((row >> 2) & 3); D = 64: 4 ((row >> 1) & 1) +
// ((row >> 2) & 3).  Depends on the row only through bits 0..3, and for D = 128
// on copy instruction n only through n & 1 (as k_swz).
template <int CH>
__host__ __device__ inline int dual_swz(int row) {
    return CH == 16 ? 4 * (row & 3) + ((row >> 2) & 3) : 4 * ((row >> 1) & 1) + ((row >> 2) & 3);
}

// Swizzle kinds of a tile: read by rows, transposed, or both.
enum { kSwzRow = 0, kSwzTr = 1, kSwzDual = 2 };

template <int CH, int SW>
__host__ __device__ inline int tile_swz(int row) {
    return SW == kSwzRow ? k_swz<CH>(row) : (SW == kSwzTr ? v_swz<CH>(row) : dual_swz<CH>(row));
}

// Element offset of logical chunk c of row `row` in a [64][8*CH] tile.
template <int CH>
__host__ __device__ inline int tile_off(int row, int c, int swz) {
    return row * CH * 8 + 8 * (c ^ swz);
}

// Direct-load instruction n of wave w (2 waves, 64 lanes) fills LDS chunk
// p = (2 n + w) * 64 + lane; that physical chunk holds logical chunk
// (p % CH) ^ swz(p / CH) of row p / CH.
__host__ __device__ inline int load_chunk_pos(int n, int wave, int lane) { return (2 * n + wave) * 64 + lane; }

// The same for a tile copied by NW = 4 or 8 waves: instruction n of wave w
// fills LDS chunks p = (NW n + w) * 64 + lane.  Rows per instruction step:
// 64 NW / CH (16, 32 or 64), so the swizzle (low 4 row bits) seen by a lane
// is the same for every n.
template <int NW>
__host__ __device__ inline int load_chunk_posN(int n, int wave, int lane) {
    return (NW * n + wave) * 64 + lane;
}
__host__ __device__ inline int load_chunk_pos4(int n, int wave, int lane) { return load_chunk_posN<4>(n, wave, lane); }

// Byte offset, inside a block of contiguous rows, of the chunk that copy
// instruction 0 of (wave, lane) fetches; instruction n fetches the one
// 1024 NW n bytes further.
template <int CH, int SW, int NW>
__host__ __device__ inline int lane_src_offsetN(int wave, int lane) {
    const int p = load_chunk_posN<NW>(0, wave, lane);
    const int row = p / CH;
    return row * CH * 16 + 16 * ((p % CH) ^ tile_swz<CH, SW>(row));
}
template <int CH, int SW>
__host__ __device__ inline int lane_src_offset4(int wave, int lane) {
    return lane_src_offsetN<CH, SW, 4>(wave, lane);
}

// Byte offset, inside a full 64-row block of the source tensor, of the chunk
// that copy instruction n (n = 0 or 1) of (wave, lane) fetches; instruction
// n + 2m fetches the one 4096 m bytes further (rows are 16 * CH bytes).
template <int CH, int SW>
__host__ __device__ inline int lane_src_offset(int wave, int lane, int n) {
    const int p = load_chunk_pos(n, wave, lane);
    const int row = p / CH;
    const int sw = tile_swz<CH, SW>(row);
    return row * CH * 16 + 16 * ((p % CH) ^ sw);
}

// Source lane of ds_read_b64_tr_b16 inside its 16-lane group: lane L reads
// the 8 bytes holding d = d0 + 4 (L & 3) .. +3 of token base + (L >> 2); after
// the transpose lane i holds d = d0 + i of tokens base .. base + 3.
__host__ __device__ inline int tr_token(int L) { return L >> 2; }
__host__ __device__ inline int tr_dquad(int L) { return L & 3; }

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
