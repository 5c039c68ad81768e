// Block-sparse flash attention over the KV blocks listed per query block.
// ("[chore] release fastvideo-kernel 0.3.0", Block-sparse / VSA attention
// improvements: block_sparse_attn_from_indices(q, k, v, q2k_idx, q2k_num,
// variable_block_sizes) and the varlen variant; "[perf] avoid full-sequence
// materialization ...", follow-up: the sparse kernel dominates the forward.)
//
// Work decomposition (gfx950, 64-wide waves, bf16 MFMA 32x32x16):
//   * one workgroup = 2 waves = one 64-token query block of one head; wave w
//     owns query rows 32w .. 32w+31;
//   * scores are computed transposed, S^T = K Q^T, so the accumulator layout
//     of v_mfma_f32_32x32x16_bf16 gives every lane ONE query column and 32
//     of its KV tokens: the running max / sum of the online softmax stay in
//     the lane (one cross-lane step with lane ^ 32 per KV block);
//   * the output is accumulated transposed as well, O^T = V^T P^T, so the
//     bf16 probabilities feed the B operand straight from the S^T
//     accumulator registers (k-slots are relabelled consistently on both
//     operands) and the per-query rescale by exp(m_old - m_new) is in-lane;
//   * K (A operand of S^T: row = KV token, k = d) is loaded from global
//     memory straight into MFMA registers, 16 bytes per lane;
//   * V must be contracted over tokens, so it is staged once per KV block
//     into LDS transposed, V^T[d][token], with the tokens of each 16-token
//     group permuted so that a lane's 8 k-slots are one 16-byte ds_read and
//     the 16-byte groups XOR-swizzled by the row so that the transposing
//     ds_write_b64 and the ds_read_b128 stay free of bank conflicts;
//   * Q stays in registers for the whole block list; float32 accumulation and
//     softmax (exp2 with log2(e)/sqrt(D) folded into one FMA); one bf16
//     rounding per output element.
#include "attn_layout.hpp"
#include "vsa_internal.hpp"

namespace vsa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short s16x8 __attribute__((ext_vector_type(8)));

constexpr int kAttnThreads = 128;

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 u) { return __builtin_bit_cast(bf16x8, u); }

__device__ __forceinline__ uint32_t pack_lo(uint32_t a, uint32_t b) { return (a & 0xffffu) | (b << 16); }
__device__ __forceinline__ uint32_t pack_hi(uint32_t a, uint32_t b) { return (a >> 16) | (b & 0xffff0000u); }

__device__ __forceinline__ uint32_t word(const uint4& u, int w) {
    return w == 0 ? u.x : (w == 1 ? u.y : (w == 2 ? u.z : u.w));
}

__device__ __forceinline__ uint32_t bf16pair(float a, float b) {
    const __bf16 x = (__bf16)a, y = (__bf16)b;
    return (uint32_t)__builtin_bit_cast(uint16_t, x) | ((uint32_t)__builtin_bit_cast(uint16_t, y) << 16);
}

template <int D>
__global__ __launch_bounds__(kAttnThreads, 2) void sparse_attn_kernel(
    DevProblem P, const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const int* __restrict__ idx, const int* __restrict__ num,
    uint16_t* __restrict__ out, float c_log2) {
    constexpr int KS = D / 16;        // MFMA k-steps over d for S^T
    constexpr int DT = D / 32;        // 32-row d tiles of O^T
    constexpr int CH = D / 8;         // 16-byte chunks per token row
    constexpr int UNITS = 16 * CH;    // (4-token group, chunk) staging units
    constexpr int UPT = UNITS / kAttnThreads;
    __shared__ __attribute__((aligned(16))) uint16_t vt[D * kBlock];

    // ---- which query block -------------------------------------------------
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
        const int N = P.total_q * P.H;
        const int lin = xcd_remap(blockIdx.x, N);
        const int g = lin % P.total_q;
        h = lin / P.total_q;
        s = seq_of_qblock(P, g);
        sv = seq_view(P, s, h);
        i = g - sv.qblk0;
        if (i < 0 || i >= sv.nq) return;  // block outside every sequence
    }
    const int qsize = q_block_size(P, sv, i);
    const int64_t qrow0 = sv.qrow_base + (int64_t)kBlock * i;

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int l32 = lane & 31;
    const int hh = lane >> 5;

    // ---- Q operand: B of S^T, column = query row, k-slots = 8 d values ----
    const int qr = 32 * wave + l32;
    bf16x8 qf[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        uint4 u = make_uint4(0, 0, 0, 0);
        if (qr < qsize) u = *reinterpret_cast<const uint4*>(q + (qrow0 + qr) * D + 16 * ks + 8 * hh);
        qf[ks] = as_bf16x8(u);
    }

    f32x16 o[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int e = 0; e < 16; ++e) o[dt][e] = 0.f;
    float m = -INFINITY;  // running max of raw scores for this lane's query
    float l = 0.f;        // this lane's share of the running sum

    const int64_t qb = sv.qblk_base + i;
    const int n = clampi(num[qb], 0, P.idx_row);
    const int* list = idx + qb * P.idx_row;

    for (int t = 0; t < n; ++t) {
        const int j = list[t] - sv.idx_rebase;
        if (j < 0 || j >= sv.nkv) continue;
        const int kvsize = kv_block_size(P, sv, j);
        const int64_t kvrow0 = sv.kvrow_base + (int64_t)kBlock * j;

        // K operand: A of S^T, row = KV token 32 mt + l32, k-slots = d
        bf16x8 kf[2][KS];
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
            const int r = 32 * mt + l32;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                uint4 u = make_uint4(0, 0, 0, 0);
                if (r < kvsize) u = *reinterpret_cast<const uint4*>(k + (kvrow0 + r) * D + 16 * ks + 8 * hh);
                kf[mt][ks] = as_bf16x8(u);
            }
        }

        // V block -> registers (4 tokens x 8 d per unit)
        uint4 vr[UPT][4];
        int ug4[UPT], uc[UPT];
#pragma unroll
        for (int r = 0; r < UPT; ++r) {
            const int u = tid + kAttnThreads * r;
            int c, g4;
            stage_unit<CH>(u, &g4, &c);
            ug4[r] = g4;
            uc[r] = c;
#pragma unroll
            for (int ii = 0; ii < 4; ++ii) {
                const int tok = 4 * g4 + ii;
                uint4 w = make_uint4(0, 0, 0, 0);
                if (tok < kvsize) w = *reinterpret_cast<const uint4*>(v + (kvrow0 + tok) * D + 8 * c);
                vr[r][ii] = w;
            }
        }

        __syncthreads();  // every wave is done reading the previous V^T
#pragma unroll
        for (int r = 0; r < UPT; ++r) {
            const int pos = tok_pos(4 * ug4[r]);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int d = 8 * uc[r] + e;
                uint2 w2;
                if ((e & 1) == 0) {
                    w2.x = pack_lo(word(vr[r][0], e >> 1), word(vr[r][1], e >> 1));
                    w2.y = pack_lo(word(vr[r][2], e >> 1), word(vr[r][3], e >> 1));
                } else {
                    w2.x = pack_hi(word(vr[r][0], e >> 1), word(vr[r][1], e >> 1));
                    w2.y = pack_hi(word(vr[r][2], e >> 1), word(vr[r][3], e >> 1));
                }
                *reinterpret_cast<uint2*>(&vt[vt_off(d, pos)]) = w2;
            }
        }
        __syncthreads();

        // S^T = K Q^T : two 32x32 tiles over the block's 64 tokens
        f32x16 sacc[2];
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
            for (int e = 0; e < 16; ++e) sacc[mt][e] = 0.f;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                sacc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[mt][ks], qf[ks], sacc[mt], 0, 0, 0);
        }

        // online softmax; accumulator e of tile mt is token 32 mt + 8 (e/4) + 4 hh + e%4
        float bm = -INFINITY;
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int tok = 32 * mt + 8 * (e >> 2) + 4 * hh + (e & 3);
                if (tok >= kvsize) sacc[mt][e] = -INFINITY;
                bm = fmaxf(bm, sacc[mt][e]);
            }
        bm = fmaxf(bm, __shfl_xor(bm, 32));
        const float m_new = fmaxf(m, bm);
        const float alpha = __builtin_amdgcn_exp2f((m - m_new) * c_log2);
        m = m_new;
        const float mc = m_new * c_log2;
        float ps = 0.f;
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const float p = __builtin_amdgcn_exp2f(fmaf(sacc[mt][e], c_log2, -mc));
                sacc[mt][e] = p;
                ps += p;
            }
        l = fmaf(l, alpha, ps);
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int e = 0; e < 16; ++e) o[dt][e] *= alpha;

        // O^T += V^T P^T over 4 k-steps of 16 tokens
#pragma unroll
        for (int s4 = 0; s4 < 4; ++s4) {
            const f32x16& sa = sacc[s4 >> 1];
            const int base = 8 * (s4 & 1);
            uint4 pw;
            pw.x = bf16pair(sa[base + 0], sa[base + 1]);
            pw.y = bf16pair(sa[base + 2], sa[base + 3]);
            pw.z = bf16pair(sa[base + 4], sa[base + 5]);
            pw.w = bf16pair(sa[base + 6], sa[base + 7]);
            const bf16x8 pb = as_bf16x8(pw);
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) {
                const int d = 32 * dt + l32;
                const uint4 va = *reinterpret_cast<const uint4*>(&vt[vt_off(d, 16 * s4 + 8 * hh)]);
                o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(va), pb, o[dt], 0, 0, 0);
            }
        }
    }

    // ---- normalise and store: lane holds O[qr][32 dt + 8 j + 4 hh + 0..3] ----
    const float lt = l + __shfl_xor(l, 32);
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    if (qr < qsize) {
        uint16_t* orow = out + (qrow0 + qr) * D;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                uint2 w2;
                w2.x = bf16pair(o[dt][4 * jj + 0] * inv, o[dt][4 * jj + 1] * inv);
                w2.y = bf16pair(o[dt][4 * jj + 2] * inv, o[dt][4 * jj + 3] * inv);
                *reinterpret_cast<uint2*>(orow + 32 * dt + 8 * jj + 4 * hh) = w2;
            }
    } else if (P.packed) {
        uint16_t* orow = out + (qrow0 + qr) * D;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj)
                *reinterpret_cast<uint2*>(orow + 32 * dt + 8 * jj + 4 * hh) = make_uint2(0, 0);
    }
}

}  // namespace

hipError_t launch_sparse_attn(const DevProblem& P, const uint16_t* q, const uint16_t* k,
                              const uint16_t* v, const int* idx, const int* num, uint16_t* out,
                              hipStream_t st) {
    const int64_t N = P.packed ? (int64_t)P.total_q * P.H : (int64_t)P.nQ * P.H * P.nseq;
    if (N <= 0 || N > 0x7fffffff) return hipErrorInvalidValue;
    const float c = (float)(1.4426950408889634 / sqrt((double)P.D));
    if (P.D == 128)
        hipLaunchKernelGGL(sparse_attn_kernel<128>, dim3((unsigned)N), dim3(kAttnThreads), 0, st, P, q,
                           k, v, idx, num, out, c);
    else
        hipLaunchKernelGGL(sparse_attn_kernel<64>, dim3((unsigned)N), dim3(kAttnThreads), 0, st, P, q,
                           k, v, idx, num, out, c);
    return hipGetLastError();
}

}  // namespace vsa
