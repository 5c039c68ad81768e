// Coarse attention over pooled blocks and exact top-k routing.
// ("[perf] avoid full-sequence materialization in VSA coarse/sparse combine",
// Problem and Change: the per-block coarse output; Correctness: top-k
// selection.  "[chore] release fastvideo-kernel 0.3.0", Block-sparse / VSA
// attention improvements: q2k_idx / q2k_num.)
//
// One workgroup (4 waves) handles R consecutive query blocks of one sequence
// and head:
//   1. the R pooled query rows are staged in LDS;
//   2. raw float64 dot products Qc[i] . Kc[j] for every KV block j of the
//      sequence land in LDS (thread j reads Kc[j] once and serves R rows);
//   3. one wave per row selects the top-k exactly: the row's order-preserving
//      64-bit keys sit in registers (up to 64 per lane), the k-th largest is
//      found bit by bit with wave-wide ballot counts (32 rounds on the high
//      halves, 32 more on the low halves only when needed), ties at the
//      threshold go to the lowest indices, and the indices are emitted in
//      ascending order with ballot prefix counts;
//   4. the same wave turns the row into softmax weights exp((s - max)/sqrt(D))
//      and their sum, in float64;
//   5. out_c[i][d] = sum_j w[i][j] Vc[j][d] / sum_j w[i][j], rounded once to
//      float32; each thread owns 4 d of 2 rows.
// Scores, softmax and the coarse product stay in float64 so that the
// selected set matches a float64 reference on any input whose k-th and
// (k+1)-th scores are not within a few ulps of each other.
#include "vsa_internal.hpp"

namespace vsa {
namespace {

constexpr int kCoarseThreads = 256;
constexpr int kCoarseWaves = kCoarseThreads / 64;
constexpr size_t kCoarseLdsBudget = 60 * 1024;

__device__ __forceinline__ uint64_t order_key(double s) {
    // -0.0 and +0.0 compare equal as doubles; fold them before the bit map.
    const uint64_t b = (uint64_t)__double_as_longlong(s + 0.0);
    return (b >> 63) ? ~b : (b | 0x8000000000000000ull);
}

__device__ __forceinline__ int lane_id() { return __lane_id(); }

__device__ __forceinline__ int prefix_popc(uint64_t mask) {
    const int l = lane_id();
    const uint64_t below = l == 0 ? 0ull : (mask & ((~0ull) >> (64 - l)));
    return __popcll(below);
}

__device__ __forceinline__ double wave_max(double x) {
    for (int o = 32; o > 0; o >>= 1) x = fmax(x, __shfl_xor(x, o));
    return x;
}
__device__ __forceinline__ double wave_sum(double x) {
    for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
    return x;
}

template <int D, int R, int KPL>
__global__ __launch_bounds__(kCoarseThreads) void coarse_topk_kernel(
    DevProblem P, const double* __restrict__ qc, const double* __restrict__ kc,
    const double* __restrict__ vc, float* __restrict__ out_c, int* __restrict__ idx_out,
    int* __restrict__ num_out, int kv_cap, double scale) {
    extern __shared__ double lds[];
    double* qrow = lds;              // [R][D]
    double* sc = lds + R * D;        // [R][kv_cap]
    __shared__ double lsum[R];

    const int s = blockIdx.z;
    const int h = blockIdx.y;
    const SeqView sv = seq_view(P, s, h);
    const int i0 = blockIdx.x * R;
    if (i0 >= sv.nq) return;
    const int nr = min(R, sv.nq - i0);
    const int nkv = min(min(sv.nkv, kv_cap), 64 * KPL);
    const int tid = threadIdx.x;

    // 1. pooled query rows
    for (int e = tid; e < R * D; e += kCoarseThreads) {
        const int r = e / D;
        qrow[e] = r < nr ? qc[(sv.qblk_base + i0 + r) * D + (e % D)] : 0.0;
    }
    __syncthreads();

    // 2. raw scores: thread j reads Kc[j] once and serves all R rows
    for (int j = tid; j < nkv; j += kCoarseThreads) {
        double acc[R];
#pragma unroll
        for (int r = 0; r < R; ++r) acc[r] = 0.0;
        const double2* kr = reinterpret_cast<const double2*>(kc + (sv.kvblk_base + j) * D);
#pragma unroll 4
        for (int d2 = 0; d2 < D / 2; ++d2) {
            const double2 kv = kr[d2];
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const double2 qv = *reinterpret_cast<const double2*>(&qrow[r * D + 2 * d2]);
                acc[r] = fma(qv.x, kv.x, acc[r]);
                acc[r] = fma(qv.y, kv.y, acc[r]);
            }
        }
#pragma unroll
        for (int r = 0; r < R; ++r) sc[r * kv_cap + j] = acc[r];
    }
    __syncthreads();

    // 3 + 4. per row (one wave): exact top-k on keys held in registers, then
    // softmax weights written back in place
    const int wave = tid / 64;
    const int lane = tid % 64;
    for (int r = wave; r < nr; r += kCoarseWaves) {
        double* row = sc + r * kv_cap;
        const int k = sv.k;
        const int64_t qb = sv.qblk_base + i0 + r;
        int* orow = idx_out + qb * P.idx_row;

        uint64_t key[KPL];  // 0 marks "no block": below the key of any double
#pragma unroll
        for (int e = 0; e < KPL; ++e) {
            const int j = 64 * e + lane;
            key[e] = j < nkv ? order_key(row[j]) : 0ull;
        }
        // T = the k-th largest key.  First the k-th largest of the high 32 bits
        // (Th) by bitwise bisection on 32-bit compares; the low 32 bits only
        // need a second bisection when the candidates sharing Th are more than
        // the number still to be chosen.
        uint32_t Th = 0;
        for (int bit = 31; bit >= 0; --bit) {
            const uint32_t cand = Th | (1u << bit);
            int cnt = 0;
#pragma unroll
            for (int e = 0; e < KPL; ++e)
                if (64 * e < nkv) cnt += __popcll(__ballot((uint32_t)(key[e] >> 32) >= cand));
            if (cnt >= k) Th = cand;
        }
        int gt_hi = 0, eq_hi = 0;
#pragma unroll
        for (int e = 0; e < KPL; ++e)
            if (64 * e < nkv) {
                const uint32_t hi = (uint32_t)(key[e] >> 32);
                gt_hi += __popcll(__ballot(hi > Th));
                eq_hi += __popcll(__ballot(hi == Th));
            }
        const int need_hi = k - gt_hi;  // >= 1 and <= eq_hi
        uint32_t Tl = 0;
        if (eq_hi != need_hi) {
            for (int bit = 31; bit >= 0; --bit) {
                const uint32_t cand = Tl | (1u << bit);
                int cnt = 0;
#pragma unroll
                for (int e = 0; e < KPL; ++e)
                    if (64 * e < nkv)
                        cnt += __popcll(__ballot((uint32_t)(key[e] >> 32) == Th && (uint32_t)key[e] >= cand));
                if (cnt >= need_hi) Tl = cand;
            }
        }
        // (when every candidate is chosen, T = Th:0 selects all of them below)
        const uint64_t T = ((uint64_t)Th << 32) | Tl;
        int n_gt = 0;
#pragma unroll
        for (int e = 0; e < KPL; ++e)
            if (64 * e < nkv) n_gt += __popcll(__ballot(key[e] > T));
        const int need_eq = k - n_gt;
        int n_sel = 0, n_eq = 0;
#pragma unroll
        for (int e = 0; e < KPL; ++e) {
            if (64 * e >= nkv) break;
            const int j = 64 * e + lane;
            const bool eq = key[e] == T;
            const uint64_t eq_mask = __ballot(eq);
            const bool sel = key[e] > T || (eq && n_eq + prefix_popc(eq_mask) < need_eq);
            const uint64_t sel_mask = __ballot(sel);
            if (sel) orow[n_sel + prefix_popc(sel_mask)] = j + sv.idx_rebase;
            n_sel += __popcll(sel_mask);
            n_eq += __popcll(eq_mask);
        }
        for (int t = n_sel + lane; t < P.idx_row; t += 64) orow[t] = -1;
        if (lane == 0) num_out[qb] = n_sel;

        double m = -INFINITY;
        for (int j = lane; j < nkv; j += 64) m = fmax(m, row[j]);
        m = wave_max(m);
        double l = 0.0;
        for (int j = lane; j < nkv; j += 64) {
            const double w = exp((row[j] - m) * scale);
            row[j] = w;
            l += w;
        }
        l = wave_sum(l);
        if (lane == 0) lsum[r] = l;
    }
    __syncthreads();

    // 5. coarse output: thread (quad, pair) owns d = 4 quad .. +3 of rows
    // 2 pair, 2 pair + 1 (and further pairs when R > 2 * groups): per KV block
    // two 16-byte loads of Vc and two LDS reads of weights feed 8 FMAs.
    constexpr int QUADS = D / 4;
    constexpr int PAIRS = kCoarseThreads / QUADS;  // row pairs handled at once
    const int quad = tid % QUADS;
    const int pair = tid / QUADS;
    for (int r0 = 2 * pair; r0 < nr; r0 += 2 * PAIRS) {
        const bool two = r0 + 1 < nr;
        const double* w0 = sc + r0 * kv_cap;
        const double* w1 = sc + (two ? r0 + 1 : r0) * kv_cap;
        double a0[4] = {0.0, 0.0, 0.0, 0.0}, a1[4] = {0.0, 0.0, 0.0, 0.0};
        const double2* vcol = reinterpret_cast<const double2*>(vc + sv.kvblk_base * D + 4 * quad);
#pragma unroll 4
        for (int j = 0; j < nkv; ++j) {
            const double2 x = vcol[j * (D / 2)];
            const double2 y = vcol[j * (D / 2) + 1];
            const double p0 = w0[j], p1 = w1[j];
            a0[0] = fma(p0, x.x, a0[0]); a0[1] = fma(p0, x.y, a0[1]);
            a0[2] = fma(p0, y.x, a0[2]); a0[3] = fma(p0, y.y, a0[3]);
            a1[0] = fma(p1, x.x, a1[0]); a1[1] = fma(p1, x.y, a1[1]);
            a1[2] = fma(p1, y.x, a1[2]); a1[3] = fma(p1, y.y, a1[3]);
        }
        float* o0 = out_c + (sv.qblk_base + i0 + r0) * D + 4 * quad;
        const double l0 = lsum[r0];
        *reinterpret_cast<float4*>(o0) =
            make_float4((float)(a0[0] / l0), (float)(a0[1] / l0), (float)(a0[2] / l0), (float)(a0[3] / l0));
        if (two) {
            const double l1 = lsum[r0 + 1];
            *reinterpret_cast<float4*>(o0 + D) =
                make_float4((float)(a1[0] / l1), (float)(a1[1] / l1), (float)(a1[2] / l1), (float)(a1[3] / l1));
        }
    }
}

template <int D>
size_t coarse_lds_bytes(int R, int kv_cap) {
    return (size_t)8 * R * (D + kv_cap);
}

template <int D, int R, int KPL>
hipError_t launch_rk(const DevProblem& P, const double* qc, const double* kc, const double* vc,
                     float* out_c, int* idx, int* num, hipStream_t st) {
    const int max_nq = P.packed ? P.max_q : P.nQ;
    const int kv_cap = P.packed ? P.max_kv : P.nKV;
    dim3 grid((max_nq + R - 1) / R, P.H, P.nseq);
    const size_t lds = coarse_lds_bytes<D>(R, kv_cap);
    hipLaunchKernelGGL((coarse_topk_kernel<D, R, KPL>), grid, dim3(kCoarseThreads), lds, st, P, qc,
                       kc, vc, out_c, idx, num, kv_cap, 1.0 / sqrt((double)D));
    return hipGetLastError();
}

template <int D, int R>
hipError_t launch_r(const DevProblem& P, const double* qc, const double* kc, const double* vc,
                    float* out_c, int* idx, int* num, hipStream_t st) {
    const int kv_cap = P.packed ? P.max_kv : P.nKV;
    if (kv_cap <= 4 * 64) return launch_rk<D, R, 4>(P, qc, kc, vc, out_c, idx, num, st);
    if (kv_cap <= 16 * 64) return launch_rk<D, R, 16>(P, qc, kc, vc, out_c, idx, num, st);
    return launch_rk<D, R, 64>(P, qc, kc, vc, out_c, idx, num, st);
}

template <int D>
hipError_t launch_d(const DevProblem& P, const double* qc, const double* kc, const double* vc,
                    float* out_c, int* idx, int* num, hipStream_t st) {
    const int kv_cap = P.packed ? P.max_kv : P.nKV;
    const int R = coarse_rows_per_group(kv_cap, D);
    switch (R) {
        case 16: return launch_r<D, 16>(P, qc, kc, vc, out_c, idx, num, st);
        case 8: return launch_r<D, 8>(P, qc, kc, vc, out_c, idx, num, st);
        case 4: return launch_r<D, 4>(P, qc, kc, vc, out_c, idx, num, st);
        case 2: return launch_r<D, 2>(P, qc, kc, vc, out_c, idx, num, st);
        case 1: return launch_r<D, 1>(P, qc, kc, vc, out_c, idx, num, st);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

int coarse_rows_per_group(int max_kv_blocks, int D) {
    if (max_kv_blocks < 1 || max_kv_blocks > kMaxKvBlocks) return 0;
    const size_t per_row = (size_t)8 * (D + max_kv_blocks);
    size_t r = kCoarseLdsBudget / per_row;
    if (r >= 16) return 16;
    if (r >= 8) return 8;
    if (r >= 4) return 4;
    if (r >= 2) return 2;
    if (r >= 1) return 1;
    return 0;
}

hipError_t launch_coarse_topk(const DevProblem& P, const double* qc, const double* kc,
                              const double* vc, float* out_c, int* idx, int* num, hipStream_t st) {
    if (P.D == 128) return launch_d<128>(P, qc, kc, vc, out_c, idx, num, st);
    return launch_d<64>(P, qc, kc, vc, out_c, idx, num, st);
}

}  // namespace vsa
