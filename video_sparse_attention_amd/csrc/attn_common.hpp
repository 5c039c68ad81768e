// Device helpers shared by the block-sparse attention kernels (forward and
// backward): MFMA operand types, bf16 packing, half-wave exchanges, explicit
// vmcnt waits and workgroup barriers, and the direct global -> LDS copies of
// 64-row KV tiles into the swizzled layouts of attn_layout.hpp.
#pragma once

#include "attn_layout.hpp"
#include "vsa_internal.hpp"

namespace vsa {
namespace attn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short s16x4 __attribute__((ext_vector_type(4)));

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 u) { return __builtin_bit_cast(bf16x8, u); }

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// two floats -> two bf16 (round to nearest even) in one v_cvt_pk_bf16_f32
__device__ __forceinline__ uint32_t bf16pair(float a, float b) {
    const f32x2 v = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// max / sum of x over lanes l and l ^ 32 (v_permlane32_swap: the two halves
// of the wave trade places, so the pair of results holds both halves)
__device__ __forceinline__ float max_with_lane_xor32(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_with_lane_xor32(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
// acc + the two bf16 values packed in w (one v_dot2 against (1, 1))
__device__ __forceinline__ float sum_bf16_pair(uint32_t w, float acc) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w), __builtin_bit_cast(bf16x2, 0x3F803F80u), acc,
                                           false);
}

// Wait until at most N vector-memory operations of this wave are in flight
// (loads complete in issue order).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
// Workgroup barrier that first waits for this wave's own LDS reads, so that
// no wave can start overwriting a tile while another's read is in flight.
__device__ __forceinline__ void wg_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// A pointer every lane holds the same value of, moved to scalar registers.
template <typename T>
__device__ __forceinline__ const T* uniform_ptr(const T* p) {
    const uint64_t v = (uint64_t)p;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    return (const T*)(((uint64_t)hi << 32) | lo);
}

// Read-only, wave-uniform data (the block list, block sizes) is read through
// the constant address space so the compiler uses scalar loads, which are
// counted by lgkmcnt and never wait for the direct-to-LDS copies in flight.
typedef const __attribute__((address_space(4))) int const_int;

// Direct global -> LDS copy of 16 bytes per lane (global_load_lds_dwordx4,
// scalar base + per-lane 32-bit offset): lane l's bytes land at LDS byte
// lds_base + 16 l.  Written as inline assembly (it has no output register)
// so that the compiler does not add its own conservative waits for the LDS
// write before every LDS read; the kernel orders these copies with explicit
// vmcnt waits and barriers.  M0 (the LDS base of the copy) is saved and
// restored inside the block.
__device__ __forceinline__ void dma_16B(const void* sbase, uint32_t voff, uint32_t lds_base) {
    uint32_t saved;
    // the LDS base is wave-uniform; readfirstlane keeps it in a scalar register
    // even when the compiler has placed the value in a vector one
    lds_base = __builtin_amdgcn_readfirstlane(lds_base);
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %3\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %1, %2\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(voff), "s"(sbase), "s"(lds_base)
        : "memory");
}

// Two direct copies sharing one M0: the immediate offset of the second
// (2048) is added to both its global and its LDS address, so with voff_b =
// (wanted source offset) - 2048 it lands 2048 bytes after the first.
__device__ __forceinline__ void dma_16B_pair(const void* sbase, uint32_t voff_a, uint32_t voff_b,
                                             uint32_t lds_base) {
    uint32_t saved;
    lds_base = __builtin_amdgcn_readfirstlane(lds_base);
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %4\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %1, %3\n\t"
        "global_load_lds_dwordx4 %2, %3 offset:2048\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(voff_a), "v"(voff_b), "s"(sbase), "s"(lds_base)
        : "memory");
}

// Copy one 64-row KV block starting at `block` (rows `pitch` bytes apart)
// into a swizzled tile.  Full blocks of contiguous rows: instructions 2m and
// 2m + 1 of a lane fetch lane_off0 + 4096 m and lane_off1 + 4096 m (passed as
// lane_off1_m2k = lane_off1 - 2048, see dma_16B_pair) into LDS bytes
// lds0 + 4096 m and lds0 + 4096 m + 2048.  Otherwise one copy per instruction
// with the row clamped: rows past valid - 1 repeat that row, so every address
// stays inside the tensor and every LDS value is finite.
template <int D, int SW>
__device__ __forceinline__ void load_tile(uint32_t lds0, const uint16_t* block, int valid, int wave,
                                          int lane, uint32_t lane_off0, uint32_t lane_off1_m2k,
                                          uint32_t pitch = 2u * D) {
    constexpr int CH = D / 8;
    const char* base = (const char*)uniform_ptr(block);
    if (valid == kBlock && pitch == 2u * D) {
#pragma unroll
        for (int m = 0; m < CH / 4; ++m)
            dma_16B_pair(base + 4096 * m, lane_off0, lane_off1_m2k, lds0 + 4096u * m);
    } else {
        // instruction n covers physical rows row0 + RSTEP n; the swizzles
        // depend on n only through n & 1 (bit 3 of the row for CH = 16), so a
        // lane needs row0 and two chunk numbers, and the clamp is
        // min(row0, valid - 1 - RSTEP n) + RSTEP n with a scalar bound
        constexpr int RSTEP = 128 / CH;
        const int p0 = load_chunk_pos(0, wave, lane);
        const int row0 = p0 / CH;
        const int c0 = (p0 % CH) ^ tile_swz<CH, SW>(row0);
        const int c1 = (p0 % CH) ^ tile_swz<CH, SW>(row0 + RSTEP);
#pragma unroll
        for (int n = 0; n < CH / 2; ++n) {
            const int r = min(row0, valid - 1 - RSTEP * n) + RSTEP * n;
            dma_16B(base, (uint32_t)r * pitch + 16u * ((n & 1) ? c1 : c0), lds0 + 2048u * n);
        }
    }
}

// The same copy of the first ROWS (64 or 32) rows of a block by NW = 4 or 8
// waves (load_chunk_posN): each wave issues ROWS CH / (64 NW) instructions;
// instruction n of a block of contiguous rows with every row valid fetches
// lane_off + 1024 NW n into LDS byte lds0 + 1024 NW n (lds0 = tile + 1024
// wave).  Otherwise (a partial block, or rows `pitch` bytes apart) row
// row0 + RSTEP n is fetched with the row clamped: rows at or past `valid`
// repeat row valid - 1, as in load_tile.
template <int D, int SW, int ROWS, int NW>
__device__ __forceinline__ void load_tile_n(uint32_t lds0, const uint16_t* block, int valid, int wave, int lane,
                                            uint32_t lane_off, uint32_t pitch = 2u * D) {
    constexpr int CH = D / 8;
    constexpr int NI = ROWS * CH / (64 * NW);  // instructions per wave
    constexpr int RSTEP = 64 * NW / CH;        // rows between a lane's instructions
    static_assert(NI >= 1 && NI * 64 * NW == ROWS * CH, "tile rows must fill whole instructions");
    static_assert(RSTEP % 16 == 0, "the swizzle must not change between a lane's instructions");
    const char* base = (const char*)uniform_ptr(block);
    if (valid >= ROWS && pitch == 2u * D) {
#pragma unroll
        for (int n = 0; n < NI; ++n) dma_16B(base + 1024 * NW * n, lane_off, lds0 + 1024u * NW * n);
    } else {
        const int p0 = load_chunk_posN<NW>(0, wave, lane);
        const int row0 = p0 / CH;
        const int c0 = (p0 % CH) ^ tile_swz<CH, SW>(row0);
#pragma unroll
        for (int n = 0; n < NI; ++n) {
            const int r = min(row0, valid - 1 - RSTEP * n) + RSTEP * n;
            dma_16B(base, (uint32_t)r * pitch + 16u * c0, lds0 + 1024u * NW * n);
        }
    }
}

template <int D, int SW, int ROWS>
__device__ __forceinline__ void load_tile4(uint32_t lds0, const uint16_t* block, int valid, int wave, int lane,
                                           uint32_t lane_off) {
    load_tile_n<D, SW, ROWS, 4>(lds0, block, valid, wave, lane, lane_off);
}

}  // namespace attn
}  // namespace vsa
