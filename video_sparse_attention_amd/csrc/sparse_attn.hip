// Block-sparse flash attention over the KV blocks listed per query block.
// ("[chore] release fastvideo-kernel 0.3.0", Block-sparse / VSA attention
// improvements: block_sparse_attn_from_indices(q, k, v, q2k_idx, q2k_num,
// variable_block_sizes) and the varlen variant; "[perf] avoid full-sequence
// materialization ...", follow-up: the sparse kernel dominates the forward.)
//
// Work decomposition (gfx950, 64-wide waves, bf16 MFMA 32x32x16):
//   * one workgroup = 2 waves = one 64-token query block of one head; wave w
//     owns query rows 32w .. 32w+31 and keeps its Q fragment in registers;
//   * with VSA blocks of 128 or 256 tokens the 64-token query blocks of one
//     VSA block share its block list: one workgroup of 4 waves
//     serves two of them, copies each selected KV tile into LDS once (each
//     wave issues a quarter of the copy) and both wave pairs read it, which
//     halves the L2 -> LDS traffic (sharing among all four blocks of a
//     256-token VSA block in one 8-wave workgroup measured slower);
//   * scores are computed transposed, S^T = K Q^T, so the accumulator layout
//     of v_mfma_f32_32x32x16_bf16 gives every lane ONE query column and 32
//     of its KV tokens: the running max and sum of the online softmax stay
//     in the lane (one exchange with lane ^ 32 per KV block);
//   * the output is accumulated transposed too, O^T = V^T P^T: the bf16
//     probabilities feed the B operand straight from the S^T accumulator
//     registers (the k-slots of both operands are relabelled the same way)
//     and the rescale by exp(m_old - m_new) is in-lane;
//   * each selected KV block is copied global -> LDS by direct loads
//     (global_load_lds_dwordx4, no register staging) into row-major K and V
//     tiles with XOR-swizzled 16-byte chunks; K operands come from
//     ds_read_b128, the transposed V operands from ds_read_b64_tr_b16;
//   * the block list is walked from a rotated start (see kSweep) so that
//     concurrently running workgroups share KV blocks in L2;
//   * software pipeline per KV block t: wait K_t, S = K_t Q^T, release the K
//     tile and start loading K_{t+1}; softmax; wait V_t, O += V_t^T P^T,
//     release the V tile and start loading V_{t+1} - so each load overlaps
//     half an iteration of this workgroup plus the work of the other
//     workgroups on the CU;
//   * float32 accumulation and softmax (exp2 with log2(e)/sqrt(D) folded
//     into one FMA); the running max moves lazily (only when a block raises
//     it by more than 2^8), so most blocks skip the rescale of the output;
//     one bf16 rounding per output element.
#include "attn_common.hpp"

namespace vsa {
namespace {

using namespace attn;

constexpr int kAttnThreads = 128;  // per 64-token query block
// Workgroups resident on one XCD at a time (32 CUs x 4 workgroups).  Query
// block i starts its walk over its block list at entry (i mod kSweep) * n /
// kSweep and wraps around, so the workgroups running together on an XCD read
// nearby entries of their (ascending) lists at the same time and share them
// in L2, instead of all starting at the front while earlier ones are deep
// into theirs.  Only the order of the online-softmax updates changes.
constexpr int kSweep = 128;

// Epilogue of the kernel: write the sparse output itself, or fuse the
// combine with the block's coarse row (no gate, a per-token gate, or a full
// [.., D] gate).
enum CombineMode { kSparseOnly = -1, kAddCoarse = 0, kTokenGate = 1, kFullGate = 2 };

// Where the combine's inputs live (unused for kSparseOnly), and the optional
// extra outputs a training forward keeps for the backward pass.
struct CombineArgs {
    const float* out_c;     // block-resolution coarse output
    const uint16_t* gate;   // bf16 gate
    int64_t gs0, gs1, gs2;  // gate element strides: batch, head, token
    uint16_t* out_s;        // if set (fused modes): the sparse output O / l, bf16
    float* lse;             // if set: log2 of the softmax denominator of each
                            // query row in exp2 units of the scaled scores
};

// R = 64-token query blocks per workgroup: 1, or 2 for problems with 128- or
// 256-token VSA blocks (blocks 2J and 2J + 1 then lie in one VSA block and
// share its list).  Two waves per SIMD.
template <int D, int CMODE, int R>
__global__ __launch_bounds__(kAttnThreads * R, 2) void sparse_attn_kernel(
    DevProblem P, const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const int* __restrict__ idx, const int* __restrict__ num,
    uint16_t* __restrict__ out, float c_log2, CombineArgs C) {
    static_assert(R == 1 || R == 2, "1 or 2 query blocks per workgroup");
    constexpr int KS = D / 16;      // MFMA k-steps over d for S^T
    constexpr int DT = D / 32;      // 32-row d tiles of O^T
    constexpr int CH = D / 8;       // 16-byte chunks per token row
    constexpr int NW = 2 * R;       // waves sharing (and copying) each tile
    constexpr int LOADS = CH / NW;  // direct-load instructions per wave per tile
    // The running max is only moved when a block's max exceeds it by more than
    // kLazy (in log2 units): probabilities then stay <= 2^kLazy, far from any
    // float32/bf16 range limit, and most blocks skip the rescale entirely.
    constexpr float kLazy = 8.0f;
    __shared__ __attribute__((aligned(1024))) uint16_t k_tile[kBlock * D];
    __shared__ __attribute__((aligned(1024))) uint16_t v_tile[kBlock * D];

    const int tid = threadIdx.x;
    const int wave = tid >> 6;  // 0 .. 2R-1
    const int lane = tid & 63;
    const int l32 = lane & 31;
    const int hh = lane >> 5;

    // VSA blocks of 64 * ratio tokens: the routing and out_c are per VSA
    // block; a selected VSA block J stands for the 64-token KV blocks
    // J ratio .. J ratio + ratio - 1
    const int lr = P.ratio >> 1;  // log2(ratio) for ratio 1, 2, 4

    // ---- which query block -------------------------------------------------
    int s, h, i;
    SeqView sv;
    if (R > 1 && !P.packed) {  // 64-token query blocks 2J and 2J + 1 of one VSA block
        const int nJ = (P.nQ + 1) / 2;
        const int N = nJ * P.H * P.nseq;
        const int lin = xcd_remap(blockIdx.x, N);
        const int J = lin % nJ;
        const int rest = lin / nJ;
        h = rest % P.H;
        s = rest / P.H;
        sv = seq_view(P, s, h);
        i = 2 * J + (wave >> 1);  // this wave pair's query block (may be past the end)
    } else if (R > 1) {  // packed: every VSA block holds ratio / 2 pairs
        const int npair = P.total_q << (lr - 1);
        const int N = npair * P.H;
        const int lin = xcd_remap(blockIdx.x, N);
        const int gJ = lin % npair;
        h = lin / npair;
        s = seq_of_qblock(P, gJ >> (lr - 1));
        sv = seq_view(P, s, h);
        i = 2 * gJ + (wave >> 1) - (sv.qblk0 << lr);
        if (i < 0 || i >= sv.nq) return;  // block outside every sequence (both pairs alike)
    } else if (!P.packed) {
        const int N = P.nQ * P.H * P.nseq;
        const int lin = xcd_remap(blockIdx.x, N);
        i = lin % P.nQ;
        const int rest = lin / P.nQ;
        h = rest % P.H;
        s = rest / P.H;
        sv = seq_view(P, s, h);
    } else {
        const int N = (P.total_q << lr) * P.H;
        const int lin = xcd_remap(blockIdx.x, N);
        const int g = lin % (P.total_q << lr);
        h = lin / (P.total_q << lr);
        s = seq_of_qblock(P, g >> lr);
        sv = seq_view(P, s, h);
        i = g - (sv.qblk0 << lr);
        if (i < 0 || i >= sv.nq) return;  // block outside every sequence
    }
    // a query block past the end of a dense sequence (last VSA block) or an
    // empty one of a packed VSA block has no rows; its waves still take part
    // in the shared copies and barriers
    const int qsize = (R > 1 && i >= sv.nq) ? 0 : q_block_size(P, sv, i);
    // the first query block of the workgroup is the fullest: when it is empty
    // (packed) no block list is walked
    const int lead_size = R > 1 ? q_block_size(P, sv, i & ~1) : qsize;
    const int64_t qrow0 = sv.qrow_base + (int64_t)kBlock * i;    // row index (lse)
    const int64_t qoff0 = sv.q_off + (int64_t)kBlock * i * sv.q_st;  // element offset of row 0

    // ---- Q operand: B of S^T, column = query row, k-slots = 8 d values ----
    const int qr = 32 * (wave & 1) + l32;
    bf16x8 qf[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        uint4 u = make_uint4(0, 0, 0, 0);
        if (qr < qsize) u = *reinterpret_cast<const uint4*>(q + qoff0 + qr * sv.q_st + 16 * ks + 8 * hh);
        qf[ks] = as_bf16x8(u);
    }

    f32x16 o[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int e = 0; e < 16; ++e) o[dt][e] = 0.f;
    float m = -INFINITY;  // running (lazy) max of raw scores for this lane's query
    float l = 0.f;        // this lane's share of the running sum

    // VSA block of this query block in the block-resolution arrays
    const int64_t qb = sv.qvsa_base + (i >> lr);
    const int nsel = __builtin_amdgcn_readfirstlane(lead_size > 0 ? clampi(num[qb], 0, P.idx_row) : 0);
    const int n = nsel << lr;  // 64-token KV blocks to visit
    const_int* list = (const_int*)uniform_ptr(idx + qb * P.idx_row);
    const_int* bs_kv = (const_int*)(P.packed ? uniform_ptr(P.bs_kv + sv.kvblk0) : nullptr);
    const int rebase = __builtin_amdgcn_readfirstlane(sv.idx_rebase);
    const int nkv = __builtin_amdgcn_readfirstlane(sv.nkv);
    const float lazy_raw = kLazy / c_log2;  // kLazy in raw-score units

    // Q is in registers before the first direct-to-LDS copy is issued, so the
    // copies in flight are the only vector-memory operations the pipeline's
    // vmcnt waits count.
    __builtin_amdgcn_s_waitcnt(0);

    // the walk visits positions (t0 + t) mod n for t = 0 .. n-1 of the list
    // expanded to 64-token blocks; entries are local 64-token KV blocks
    const int t0 = n > 0 ? (((i >> lr) % kSweep) * n) / kSweep : 0;
    auto entry = [&](int t) -> int {
        int pos = t0 + t;
        if (pos >= n) pos -= n;
        const int J = list[pos >> lr] - rebase;
        // no sequence has 2^28 VSA blocks: such an entry (or a negative one)
        // is out of range, and is kept from wrapping into range by the shift
        if ((unsigned)J >= (1u << 28)) return -1;
        return (J << lr) + (pos & ((1 << lr) - 1));
    };
    // The entry of walk step pre_t is loaded one step ahead, so the scalar
    // load's latency is hidden behind a whole block of work.
    int pre_t = 0;
    int pre = n > 0 ? entry(0) : 0;
    // valid tokens of local KV block j (packed: 0 for an empty 64-token
    // block of a VSA block)
    auto kv_size = [&](int j) -> int {
        return P.packed ? packed_sub_size(bs_kv[j >> lr], j & ((1 << lr) - 1)) : min(kBlock, P.Skv - kBlock * j);
    };
    // next valid, non-empty entry at or after walk step t (-1: none)
    auto next_valid = [&](int& t) -> int {
        for (; t < n; ++t) {
            const int j = t == pre_t ? pre : entry(t);
            if (t + 1 < n) {
                pre = entry(t + 1);
                pre_t = t + 1;
            }
            if (j >= 0 && j < nkv && (lr == 0 || !P.packed || kv_size(j) > 0)) return j;
        }
        return -1;
    };

    // per-lane positions inside the tiles (copies by 2 waves: two offsets,
    // see load_tile; by 4 or 8 waves: one, see load_tile_n)
    uint32_t koff0, koff1 = 0, voff0, voff1 = 0;
    if constexpr (R == 1) {
        koff0 = (uint32_t)lane_src_offset<CH, kSwzRow>(wave, lane, 0);
        koff1 = (uint32_t)lane_src_offset<CH, kSwzRow>(wave, lane, 1) - 2048u;
        voff0 = (uint32_t)lane_src_offset<CH, kSwzTr>(wave, lane, 0);
        voff1 = (uint32_t)lane_src_offset<CH, kSwzTr>(wave, lane, 1) - 2048u;
    } else {
        koff0 = (uint32_t)lane_src_offsetN<CH, kSwzRow, NW>(wave, lane);
        voff0 = (uint32_t)lane_src_offsetN<CH, kSwzTr, NW>(wave, lane);
    }
    const uint32_t pitch = __builtin_amdgcn_readfirstlane((uint32_t)(2 * sv.kv_st));  // bytes between KV rows
    // this wave's LDS byte base inside each tile
    const uint32_t k_lds = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)k_tile + 1024u * wave);
    const uint32_t v_lds = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)v_tile + 1024u * wave);
    // V^T operand via transpose reads: 16-lane group g16 covers d0 .. d0+15
    const int g16 = lane >> 4, L16 = lane & 15;
    const int tr_r = tr_token(L16), tr_a = tr_dquad(L16);
    const int tr_d = 16 * (g16 & 1) + 4 * tr_a;  // + 32 dt

    // Pipeline.  Each pass issues the loads of block `jn` (if any) and computes
    // block `j` (if any); the first pass only issues.
    int t = 0;
    int j = -1, kvsize = 0;
    int jn = next_valid(t);
    int kvsize_n = jn >= 0 ? kv_size(jn) : 0;
    bool first = true;
    while (j >= 0 || first) {
        const bool cur = j >= 0;
        const bool more = jn >= 0;
        const int64_t off_n = more ? sv.kv_off + (int64_t)kBlock * jn * sv.kv_st : 0;

        // ---- S^T = K Q^T ----------------------------------------------------
        f32x16 sacc[2];
        if (cur) {
            wait_vmcnt<LOADS>();  // this wave's part of K_t is in LDS (V_t may be in flight)
            wg_barrier();         // ... and the other wave's part
#pragma unroll
            for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                for (int e = 0; e < 16; ++e) sacc[mt][e] = 0.f;
            // K operands are read two k-steps ahead of their MFMAs (the two
            // 32-token tiles alternate), so each read has four MFMAs of time
            auto k_read = [&](int mt, int ks) -> uint4 {
                const int row = 32 * mt + l32;
                return *reinterpret_cast<const uint4*>(k_tile + tile_off<CH>(row, 2 * ks + hh, k_swz<CH>(row)));
            };
            uint4 ka[3][2];
#pragma unroll
            for (int ks = 0; ks < 2; ++ks)
#pragma unroll
                for (int mt = 0; mt < 2; ++mt) ka[ks][mt] = k_read(mt, ks);
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                if (ks + 2 < KS) {
#pragma unroll
                    for (int mt = 0; mt < 2; ++mt) ka[(ks + 2) % 3][mt] = k_read(mt, ks + 2);
                }
                // keep the scheduler from sinking the reads next to their use
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int mt = 0; mt < 2; ++mt)
                    sacc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(ka[ks % 3][mt]), qf[ks], sacc[mt], 0, 0, 0);
                __builtin_amdgcn_sched_barrier(0);
            }
            wg_barrier();  // both waves are done with the K tile
        }
        if (more) {
            if constexpr (R == 1) load_tile<D, kSwzRow>(k_lds, k + off_n, kvsize_n, wave, lane, koff0, koff1, pitch);
            else load_tile_n<D, kSwzRow, kBlock, NW>(k_lds, k + off_n, kvsize_n, wave, lane, koff0, pitch);
        }

        if (cur) {
            // ---- online softmax; acc e of tile mt is token 32 mt + 8 (e/4) + 4 hh + e%4
            if (kvsize < kBlock) {
#pragma unroll
                for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                    for (int e = 0; e < 16; ++e) {
                        const int tok = 32 * mt + 8 * (e >> 2) + 4 * hh + (e & 3);
                        if (tok >= kvsize) sacc[mt][e] = -INFINITY;
                    }
            }
            float bm = -INFINITY;
#pragma unroll
            for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                for (int e = 0; e < 16; ++e) bm = fmaxf(bm, sacc[mt][e]);
            bm = max_with_lane_xor32(bm);
            if (__ballot(bm > m + lazy_raw)) {  // some query's max moved: rescale
                const float m_new = fmaxf(m, bm);
                const float alpha = __builtin_amdgcn_exp2f((m - m_new) * c_log2);
                m = m_new;
                l *= alpha;
#pragma unroll
                for (int dt = 0; dt < DT; ++dt)
#pragma unroll
                    for (int e = 0; e < 16; ++e) o[dt][e] *= alpha;
            }
            const float mc = m * c_log2;
#pragma unroll
            for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                for (int e = 0; e < 16; ++e) sacc[mt][e] = __builtin_amdgcn_exp2f(fmaf(sacc[mt][e], c_log2, -mc));
            // bf16 probabilities, the B operand of O^T += V^T P^T; the row sum
            // is taken over these rounded values (two per dot2 instruction)
            uint32_t pw[4][4];
#pragma unroll
            for (int s4 = 0; s4 < 4; ++s4)
#pragma unroll
                for (int w = 0; w < 4; ++w)
                    pw[s4][w] = bf16pair(sacc[s4 >> 1][8 * (s4 & 1) + 2 * w], sacc[s4 >> 1][8 * (s4 & 1) + 2 * w + 1]);
#pragma unroll
            for (int s4 = 0; s4 < 4; ++s4)
#pragma unroll
                for (int w = 0; w < 4; ++w) l = sum_bf16_pair(pw[s4][w], l);

            // ---- O^T += V^T P^T over 4 k-steps of 16 tokens -----------------
            if (more) wait_vmcnt<LOADS>(); else wait_vmcnt<0>();  // V_t landed (K_{t+1} may be in flight)
            wg_barrier();
#pragma unroll
            for (int s4 = 0; s4 < 4; ++s4) {
                const bf16x8 pb = as_bf16x8(make_uint4(pw[s4][0], pw[s4][1], pw[s4][2], pw[s4][3]));
#pragma unroll
                for (int dt = 0; dt < DT; ++dt) {
                    const int d = 32 * dt + tr_d;
                    s16x4 half[2];
#pragma unroll
                    for (int jj = 0; jj < 2; ++jj) {
                        const int tok = 16 * s4 + 8 * jj + 4 * hh + tr_r;
                        const int off = tile_off<CH>(tok, d >> 3, v_swz<CH>(tok)) + (d & 7);
                        half[jj] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                            (lds_s16x4*)((__attribute__((address_space(3))) uint16_t*)v_tile + off));
                    }
                    const uint2 h0 = __builtin_bit_cast(uint2, half[0]);
                    const uint2 h1 = __builtin_bit_cast(uint2, half[1]);
                    const uint4 va = make_uint4(h0.x, h0.y, h1.x, h1.y);
                    o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(va), pb, o[dt], 0, 0, 0);
                }
            }
            wg_barrier();  // both waves are done with the V tile
        }
        if (more) {
            if constexpr (R == 1) load_tile<D, kSwzTr>(v_lds, v + off_n, kvsize_n, wave, lane, voff0, voff1, pitch);
            else load_tile_n<D, kSwzTr, kBlock, NW>(v_lds, v + off_n, kvsize_n, wave, lane, voff0, pitch);
        }

        first = false;
        j = jn;
        kvsize = kvsize_n;
        if (more) {
            ++t;
            jn = next_valid(t);
            kvsize_n = jn >= 0 ? kv_size(jn) : 0;
        }
    }

    // ---- normalise and store: lane holds O[qr][32 dt + 8 j + 4 hh + 0..3] ----
    const float lt = sum_with_lane_xor32(l);
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    // P[t][u] = exp2(s[t][u] c_log2 - lse[t]) for the row's selected tokens
    if (C.lse && hh == 0 && qr < qsize) C.lse[qrow0 + qr] = m * c_log2 + __log2f(lt);
    if (CMODE != kSparseOnly && C.out_s && qr < qsize) {
        uint16_t* srow = C.out_s + qoff0 + qr * sv.q_st;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                uint2 w2;
                w2.x = bf16pair(o[dt][4 * jj + 0] * inv, o[dt][4 * jj + 1] * inv);
                w2.y = bf16pair(o[dt][4 * jj + 2] * inv, o[dt][4 * jj + 3] * inv);
                *reinterpret_cast<uint2*>(srow + 32 * dt + 8 * jj + 4 * hh) = w2;
            }
    } else if (CMODE != kSparseOnly && C.out_s && P.packed) {
        uint16_t* srow = C.out_s + qoff0 + qr * sv.q_st;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj)
                *reinterpret_cast<uint2*>(srow + 32 * dt + 8 * jj + 4 * hh) = make_uint2(0, 0);
    }
    if (qr < qsize && CMODE == kSparseOnly) {
        uint16_t* orow = out + qoff0 + qr * sv.q_st;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                uint2 w2;
                w2.x = bf16pair(o[dt][4 * jj + 0] * inv, o[dt][4 * jj + 1] * inv);
                w2.y = bf16pair(o[dt][4 * jj + 2] * inv, o[dt][4 * jj + 3] * inv);
                *reinterpret_cast<uint2*>(orow + 32 * dt + 8 * jj + 4 * hh) = w2;
            }
    } else if (qr < qsize) {
        // fused combine: out = out_c[block] * gate + O / l in float32 (FMA),
        // one rounding to bf16
        uint16_t* orow = out + qoff0 + qr * sv.q_st;
        const float* ocr = C.out_c + qb * D;
        // token index of this row along the gate's token axis
        const int64_t tok = (int64_t)kBlock * (P.packed ? (sv.qblk0 << lr) + i : i) + qr;
        const int64_t goff = (P.packed ? 0 : (int64_t)s * C.gs0) + (int64_t)h * C.gs1 + tok * C.gs2;
        float g = 1.f;
        if (CMODE == kTokenGate) g = __uint_as_float((uint32_t)C.gate[goff] << 16);
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const int d0 = 32 * dt + 8 * jj + 4 * hh;
                const float4 c4 = *reinterpret_cast<const float4*>(ocr + d0);
                float r[4];
                const float cc[4] = {c4.x, c4.y, c4.z, c4.w};
                if (CMODE == kFullGate) {
                    const uint2 gw = *reinterpret_cast<const uint2*>(C.gate + goff + d0);
                    const float gg[4] = {__uint_as_float(gw.x << 16), __uint_as_float(gw.x & 0xffff0000u),
                                         __uint_as_float(gw.y << 16), __uint_as_float(gw.y & 0xffff0000u)};
#pragma unroll
                    for (int e = 0; e < 4; ++e) r[e] = __builtin_fmaf(cc[e], gg[e], o[dt][4 * jj + e] * inv);
                } else if (CMODE == kTokenGate) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) r[e] = __builtin_fmaf(cc[e], g, o[dt][4 * jj + e] * inv);
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e) r[e] = cc[e] + o[dt][4 * jj + e] * inv;
                }
                uint2 w2;
                w2.x = bf16pair(r[0], r[1]);
                w2.y = bf16pair(r[2], r[3]);
                *reinterpret_cast<uint2*>(orow + d0) = w2;
            }
    } else if (P.packed) {
        uint16_t* orow = out + qoff0 + qr * sv.q_st;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj)
                *reinterpret_cast<uint2*>(orow + 32 * dt + 8 * jj + 4 * hh) = make_uint2(0, 0);
    }
}

template <int D, int CMODE, int R>
hipError_t launch_r(const DevProblem& P, unsigned grid, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                    const int* idx, const int* num, uint16_t* out, float c, const CombineArgs& C, hipStream_t st) {
    hipLaunchKernelGGL((sparse_attn_kernel<D, CMODE, R>), dim3(grid), dim3(kAttnThreads * R), 0, st, P, q, k, v, idx,
                       num, out, c, C);
    return hipGetLastError();
}

template <int D, int CMODE>
hipError_t launch_d(const DevProblem& P, const uint16_t* q, const uint16_t* k, const uint16_t* v, const int* idx,
                    const int* num, uint16_t* out, float c, const CombineArgs& C, hipStream_t st) {
    // 128/256-token VSA blocks: one workgroup per pair of 64-token query
    // blocks
    const bool pairs = P.ratio >= 2;
    const int64_t N = P.packed ? (int64_t)P.total_q * P.ratio / (pairs ? 2 : 1) * P.H
                               : (int64_t)(pairs ? (P.nQ + 1) / 2 : P.nQ) * P.H * P.nseq;
    if (N <= 0 || N > 0x7fffffff) return hipErrorInvalidValue;
    if (pairs) return launch_r<D, CMODE, 2>(P, (unsigned)N, q, k, v, idx, num, out, c, C, st);
    return launch_r<D, CMODE, 1>(P, (unsigned)N, q, k, v, idx, num, out, c, C, st);
}

template <int CMODE>
hipError_t launch_mode(const DevProblem& P, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                       const int* idx, const int* num, uint16_t* out, const CombineArgs& C, hipStream_t st) {
    const float c = (float)(1.4426950408889634 / sqrt((double)P.D));
    if (P.D == 128) return launch_d<128, CMODE>(P, q, k, v, idx, num, out, c, C, st);
    return launch_d<64, CMODE>(P, q, k, v, idx, num, out, c, C, st);
}

}  // namespace

hipError_t launch_sparse_attn(const DevProblem& P, const uint16_t* q, const uint16_t* k,
                              const uint16_t* v, const int* idx, const int* num, uint16_t* out,
                              hipStream_t st) {
    return launch_mode<kSparseOnly>(P, q, k, v, idx, num, out,
                                    CombineArgs{nullptr, nullptr, 0, 0, 0, nullptr, nullptr}, st);
}

hipError_t launch_sparse_attn_combine(const DevProblem& P, const uint16_t* q, const uint16_t* k,
                                      const uint16_t* v, const int* idx, const int* num, const float* out_c,
                                      const uint16_t* gate, int mode, int64_t gs0, int64_t gs1, int64_t gs2,
                                      uint16_t* out, uint16_t* out_s, float* lse, hipStream_t st) {
    const CombineArgs C{out_c, gate, gs0, gs1, gs2, out_s, lse};
    switch (mode) {
        case 0: return launch_mode<kAddCoarse>(P, q, k, v, idx, num, out, C, st);
        case 1: return launch_mode<kTokenGate>(P, q, k, v, idx, num, out, C, st);
        case 2: return launch_mode<kFullGate>(P, q, k, v, idx, num, out, C, st);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace vsa
