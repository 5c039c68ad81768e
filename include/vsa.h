/*
 * vsa.h - C ABI of libvsa, the forward pass of video sparse attention (VSA)
 * on AMD Instinct MI355X (gfx950).
 *
 * The method (taken from the FastVideo pages listed per entry point):
 *   1. Q, K and V are cut into 64-token blocks;
 *   2. a coarse branch pools every block to its mean and runs softmax
 *      attention of the pooled queries over the pooled keys/values, giving one
 *      coarse output row per query block (out_c, kept at block resolution);
 *   3. for every query block the top-k KV blocks by coarse score are selected
 *      (q2k_idx, q2k_num);
 *   4. a block-sparse attention runs each query block over only its selected
 *      KV blocks (out_s);
 *   5. out = out_c * gate + out_s, out_c broadcast over the block's tokens
 *      (out_c + out_s without a gate);
 *   6. several sequences of different lengths can be packed, block-aligned,
 *      into one tensor and handled in one launch per stage.
 *
 * Conventions shared by every entry point:
 *   - bf16 tensors are passed as uint16_t storage (vsa_bf16), device memory;
 *   - every device pointer must be 16-byte aligned unless stated otherwise;
 *   - the caller owns every buffer; the library allocates no device memory
 *     and keeps no state between calls except a per-thread error message;
 *   - every call is asynchronous on `stream` (a hipStream_t; NULL is the
 *     null stream) and performs no host-device synchronisation;
 *   - all arguments are validated on the host before anything is launched; a
 *     negative return value is an error code (VSA_ERR_*), nothing has been
 *     launched in that case, and vsa_last_error() describes it;
 *   - head_dim is 64 or 128; block_size (the VSA block: pooling, routing and
 *     the KV granularity of the sparse attention) is 64, 128 or 256 in every
 *     layout ("[chore] release fastvideo-kernel 0.3.0", Block-sparse / VSA
 *     attention improvements: 256-token KV blocks and the variable-block-size
 *     variants; "[perf] avoid full-sequence materialization ...", Change: the
 *     64/128/256 dispatch).
 *
 * Layouts:
 *   DENSE   q [B, H, Sq, D], k/v [B, H, Skv, D], out [B, H, Sq, D], each batch
 *           item one sequence; block i of a sequence holds tokens
 *           [bs i, min(bs i + bs, S)) for block_size bs.
 *   BSHD    the same with q [B, Sq, H, D], k/v [B, Skv, H, D], out [B, Sq, H, D]
 *           ("[chore] release fastvideo-kernel 0.3.0", the BSHD-native entry
 *           that avoids layout round trips); a token gate defaults to
 *           [B, Sq, H], a full gate to [B, Sq, H, D].
 *   PACKED  block-padded packing of num_seqs sequences: q [H, bs*Nq, D],
 *           k/v [H, bs*Nkv, D] with bs = block_size and Nq/Nkv the total
 *           block counts; sequence s owns global query blocks
 *           [cu_blocks_q[s], cu_blocks_q[s+1]) and KV blocks
 *           [cu_blocks_kv[s], cu_blocks_kv[s+1]); global block g starts at
 *           slot bs g and its first block_sizes_*[g] slots are valid tokens
 *           (the rest is padding, never read).
 *   Block-resolution tensors: out_c is float32 [B, H, nQ, D] (DENSE, BSHD;
 *   nQ = ceil(Sq / block_size)) or [H, Nq, D] (PACKED); q2k_num is int32
 *   [B, H, nQ] or [H, Nq]; q2k_idx is int32 [B, H, nQ, kk] with kk = min(topk,
 *   nKV) and per-sequence KV block numbers (DENSE, BSHD), or [H, Nq, max_topk]
 *   with GLOBAL KV block numbers and -1 after the first q2k_num entries
 *   (PACKED).  Selected indices are stored in ascending order.
 */
#ifndef VSA_H
#define VSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef uint16_t vsa_bf16; /* bfloat16 bit pattern */
typedef void *vsa_stream;  /* hipStream_t */

/* tokens per attention tile; VSA blocks (the unit of pooling, routing and
   out_c) are VSA_BLOCK, 2 VSA_BLOCK or 4 VSA_BLOCK tokens (block_size) */
#define VSA_BLOCK 64

/* status codes */
#define VSA_OK 0
#define VSA_ERR_NULL (-1)        /* a required pointer is NULL */
#define VSA_ERR_UNSUPPORTED (-2) /* block_size, layout or head_dim not supported, or a size over a limit */
#define VSA_ERR_TOPK (-3)        /* topk < 1 */
#define VSA_ERR_SHAPE (-4)       /* empty batch, zero-length sequence, inconsistent block counts */
#define VSA_ERR_GATE (-5)        /* bad gate mode or strides */
#define VSA_ERR_WORKSPACE (-6)   /* workspace missing or too small */
#define VSA_ERR_ALIGN (-7)       /* pointer or stride not aligned as required */
#define VSA_ERR_ALIAS (-8)       /* out overlaps an input */
#define VSA_ERR_HIP (-9)         /* a HIP runtime call or kernel launch failed */

/* layouts */
#define VSA_LAYOUT_DENSE 0
#define VSA_LAYOUT_PACKED 1
#define VSA_LAYOUT_BSHD 2

/* gate modes: none; one value per (token, head) broadcast over D; full */
#define VSA_GATE_NONE 0
#define VSA_GATE_TOKEN 1
#define VSA_GATE_FULL 2

/*
 * A problem description shared by the stage entry points.  For DENSE and BSHD
 * fill batch, seqlen_q, seqlen_kv and topk; the PACKED fields are ignored.  For
 * PACKED fill the num_seqs..topk_per_seq block (device arrays as produced by
 * vsa_build_metadata and copied to the device); batch/seqlen/topk are
 * ignored.  The kernels never read outside the arrays whose lengths are given
 * here, whatever values the device arrays hold: block sizes are clamped to
 * [1, block_size], per-sequence top-k to [1, min(max_topk, KV blocks)], and
 * indices outside a query block's own sequence are skipped.
 */
typedef struct vsa_problem {
    int32_t layout;     /* VSA_LAYOUT_DENSE, VSA_LAYOUT_BSHD or VSA_LAYOUT_PACKED */
    int32_t heads;      /* H >= 1 */
    int32_t head_dim;   /* D: 64 or 128 */
    int32_t block_size; /* 64, 128 or 256 */
    /* DENSE */
    int32_t batch;     /* B >= 1 */
    int32_t seqlen_q;  /* Sq >= 1 */
    int32_t seqlen_kv; /* Skv >= 1 */
    int32_t topk;      /* >= 1, clamped to ceil(Skv/block_size) */
    /* PACKED */
    int32_t num_seqs;        /* >= 1 */
    int32_t total_q_blocks;  /* Nq = cu_blocks_q[num_seqs] */
    int32_t total_kv_blocks; /* Nkv = cu_blocks_kv[num_seqs] */
    int32_t max_q_blocks;    /* max over sequences of query blocks */
    int32_t max_kv_blocks;   /* max over sequences of KV blocks */
    int32_t max_topk;        /* row length of q2k_idx, >= every per-sequence top-k */
    const int32_t *cu_blocks_q;    /* device, [num_seqs + 1] */
    const int32_t *cu_blocks_kv;   /* device, [num_seqs + 1] */
    const int32_t *block_sizes_q;  /* device, [Nq], 1..block_size */
    const int32_t *block_sizes_kv; /* device, [Nkv], 1..block_size */
    const int32_t *topk_per_seq;   /* device, [num_seqs] */
} vsa_problem;

/* Sizes reported by vsa_build_metadata. */
typedef struct vsa_meta_sizes {
    int32_t num_seqs;
    int32_t total_q_blocks;
    int32_t total_kv_blocks;
    int32_t max_q_blocks;
    int32_t max_kv_blocks;
    int32_t max_topk; /* max over sequences of min(topk, KV blocks) */
    int64_t q_slots;  /* block_size * total_q_blocks: rows per head of packed q/out */
    int64_t kv_slots; /* block_size * total_kv_blocks */
} vsa_meta_sizes;

/*
 * vsa_build_metadata - host-side block metadata for PACKED sequences.
 * ("[kernel] Add varlen support for block-sparse attention", Summary / How it
 * works: block-aligned packing with 64 slots per block and rebasing of
 * q2k_idx to global block offsets; "[kernel] Extract VSA utility functions
 * into fastvideo_kernel": build_vsa_metadata, variable block sizes.)
 *
 * seqlens_q/seqlens_kv/topk are host arrays of num_seqs entries
 * (seqlens_kv NULL means equal to seqlens_q); block_size (64, 128 or 256)
 * is the VSA block, the slots each block occupies.  `sizes` is always
 * filled.
 * The five output arrays are host arrays the caller allocates from `sizes`
 * (pass all NULL to size them first): cu_blocks_q/kv [num_seqs + 1],
 * block_sizes_q [total_q_blocks], block_sizes_kv [total_kv_blocks],
 * topk_clamped [num_seqs] = min(topk[s], KV blocks of s).
 * Errors: VSA_ERR_NULL (seqlens_q, topk or sizes NULL; some but not all
 * outputs NULL), VSA_ERR_UNSUPPORTED (block_size), VSA_ERR_SHAPE
 * (num_seqs < 1, a length < 1, totals beyond 2^31 slots), VSA_ERR_TOPK (a
 * topk < 1).  No device memory is touched.
 */
int vsa_build_metadata(int32_t num_seqs, const int32_t *seqlens_q, const int32_t *seqlens_kv,
                       const int32_t *topk, int32_t block_size, vsa_meta_sizes *sizes, int32_t *cu_blocks_q,
                       int32_t *cu_blocks_kv, int32_t *block_sizes_q, int32_t *block_sizes_kv,
                       int32_t *topk_clamped);

/*
 * vsa_workspace_size - bytes of device workspace the problem needs
 * (vsa_coarse_topk, vsa_forward, vsa_forward_varlen).  It holds only
 * block-resolution data, no full-sequence temporary ("[perf] avoid
 * full-sequence materialization in VSA coarse/sparse combine", Change):
 * pooled Q/K/V in float64, the float64 block-level score matrix of a chunk of
 * query blocks (the coarse stage runs chunk by chunk so that this matrix
 * stays below max(128 MiB, 1/8 of the bytes of q)) and, for the two forward
 * calls, the float32 coarse output and the routing indices when the caller
 * does not ask for them.  Returns 0 when the problem is invalid.
 */
size_t vsa_workspace_size(const vsa_problem *problem);

/*
 * vsa_coarse_topk - pool + coarse attention + top-k routing (steps 1-3).
 * ("[perf] avoid full-sequence materialization in VSA coarse/sparse
 * combine", Problem / Change / Correctness; "[chore] release fastvideo-kernel
 * 0.3.0", Block-sparse / VSA attention improvements.)
 *
 * Reads q, k, v (bf16, layout per problem).  Writes out_c (float32,
 * block-resolution), q2k_idx and q2k_num (int32, layouts above).  The pooled
 * means and the coarse scores are computed in float64 and ties between equal
 * scores go to the lower KV block.  workspace must hold
 * vsa_workspace_size(problem) bytes (256-byte aligned).
 * Limits: at most 4096 KV blocks per sequence (VSA_ERR_UNSUPPORTED).
 */
int vsa_coarse_topk(const vsa_problem *problem, const vsa_bf16 *q, const vsa_bf16 *k,
                    const vsa_bf16 *v, float *out_c, int32_t *q2k_idx, int32_t *q2k_num,
                    void *workspace, size_t workspace_bytes, vsa_stream stream);

/*
 * vsa_sparse_attn_from_indices - block-sparse attention of every query block
 * over the KV blocks listed for it (step 4).  ("[chore] release
 * fastvideo-kernel 0.3.0", Block-sparse / VSA attention improvements:
 * block_sparse_attn_from_indices(q, k, v, q2k_idx, q2k_num,
 * variable_block_sizes); PACKED is block_sparse_attn_varlen.)
 *
 * q2k_idx/q2k_num as written by vsa_coarse_topk (or any caller-made list in
 * the same layout; row length min(topk, nKV) for DENSE, max_topk for
 * PACKED).  Writes out (bf16, query layout): softmax over the valid tokens of
 * the listed blocks, bf16 matrix products with float32 accumulation and
 * float32 softmax.  In PACKED layout padding slots of out are written with 0.
 * A query block whose list holds no valid block gets 0.  out must not overlap
 * q, k or v (VSA_ERR_ALIAS).
 */
int vsa_sparse_attn_from_indices(const vsa_problem *problem, const vsa_bf16 *q,
                                 const vsa_bf16 *k, const vsa_bf16 *v, const int32_t *q2k_idx,
                                 const int32_t *q2k_num, vsa_bf16 *out, vsa_stream stream);

/*
 * vsa_combine - in place out = bf16(fma(out_c, gate, out)) (step 5), or
 * bf16(out_c + out) for VSA_GATE_NONE; float32 arithmetic, one rounding;
 * out_c is broadcast over the tokens of its block and never expanded.
 * ("[perf] avoid full-sequence materialization in VSA coarse/sparse
 * combine", Problem, Change and the follow-up comment on strict shapes and
 * the gate passed as a transposed view.)
 *
 * gate_mode VSA_GATE_TOKEN: gate[b*s0 + h*s1 + t*s2] for DENSE and
 * gate[h*s1 + slot*s2] for PACKED; VSA_GATE_FULL: the same plus d (stride 1);
 * gate_strides = {s0, s1, s2} in elements, or NULL for the contiguous
 * [B, H, Sq(, D)] / [H, slots(, D)] layout.  A transposed [B, S, H(, D)]
 * view is accepted without a copy.  FULL requires the three strides to be
 * multiples of 8 (VSA_ERR_ALIGN); strides must be >= 0 (VSA_ERR_GATE).
 * Padding slots of PACKED out are left untouched.
 */
int vsa_combine(const vsa_problem *problem, const float *out_c, const vsa_bf16 *gate,
                int32_t gate_mode, const int64_t *gate_strides, vsa_bf16 *out,
                vsa_stream stream);

/*
 * vsa_sparse_attn_combine - steps 4 and 5 in one kernel: the block-sparse
 * attention of vsa_sparse_attn_from_indices whose epilogue adds the block's
 * coarse row, out = bf16(fma(out_c, gate, O)) (bf16(out_c + O) for
 * VSA_GATE_NONE), with O the float32 normalised attention output, so the
 * sparse output is rounded once instead of twice and is never written to
 * memory on its own.  ("[perf] avoid full-sequence materialization in VSA
 * coarse/sparse combine", Change, and the review thread: the fused combine of
 * another backend, which moves gated values towards the float32 result.)
 *
 * Arguments as for vsa_sparse_attn_from_indices plus out_c, gate,
 * gate_mode and gate_strides as for vsa_combine (same checks and errors).
 * Padding slots of PACKED out are written with 0.  out must not overlap q,
 * k, v or gate.
 */
int vsa_sparse_attn_combine(const vsa_problem *problem, const vsa_bf16 *q, const vsa_bf16 *k,
                            const vsa_bf16 *v, const int32_t *q2k_idx, const int32_t *q2k_num,
                            const float *out_c, const vsa_bf16 *gate, int32_t gate_mode,
                            const int64_t *gate_strides, vsa_bf16 *out, vsa_stream stream);

/*
 * vsa_forward - the whole DENSE forward: vsa_coarse_topk, then
 * vsa_sparse_attn_combine into out.
 * ("FastVideo Kernel" README, Usage: video_sparse_attn(q, k, v, block_sizes,
 * block_sizes, topk); "[perf] avoid full-sequence materialization ...",
 * Problem.)
 *
 * q [B,H,Sq,D], k/v [B,H,Skv,D], out [B,H,Sq,D], bf16.  gate as in
 * vsa_combine (gate_strides may be NULL).  q2k_idx, q2k_num and out_c are
 * optional outputs (NULL: kept in the workspace).  workspace must hold
 * vsa_workspace_size() bytes for the matching DENSE problem.
 */
int vsa_forward(const vsa_bf16 *q, const vsa_bf16 *k, const vsa_bf16 *v, const vsa_bf16 *gate,
                int32_t gate_mode, const int64_t *gate_strides, vsa_bf16 *out, int32_t *q2k_idx,
                int32_t *q2k_num, float *out_c, int32_t batch, int32_t heads, int32_t seqlen_q,
                int32_t seqlen_kv, int32_t head_dim, int32_t block_size, int32_t topk,
                void *workspace, size_t workspace_bytes, vsa_stream stream);

/*
 * vsa_forward_noalloc - vsa_forward without a caller-provided workspace, for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc).  The workspace is a
 * file-scope device array of vsa_noalloc_scratch_bytes() bytes (96 MiB),
 * which every GPU the library runs on holds from the library's first use on
 * it until the process ends; its device address is taken once per device, on
 * the first call with that device current.  The call allocates nothing
 * (no hipMalloc, hipFree or allocating library routine).
 *
 * Arguments, outputs and errors as for vsa_forward (DENSE [B,H,S,D] tensors);
 * VSA_ERR_WORKSPACE when the problem's vsa_workspace_size() exceeds the array
 * (checked before any device call).  All calls on one GPU share that GPU's
 * array: calls that overlap in time on one GPU (other streams, other host
 * threads) race and must be serialised by the caller.  Nothing in the array
 * needs clearing between calls.
 */
size_t vsa_noalloc_scratch_bytes(void);
int vsa_forward_noalloc(const vsa_bf16 *q, const vsa_bf16 *k, const vsa_bf16 *v, const vsa_bf16 *gate,
                        int32_t gate_mode, const int64_t *gate_strides, vsa_bf16 *out, int32_t *q2k_idx,
                        int32_t *q2k_num, float *out_c, int32_t batch, int32_t heads, int32_t seqlen_q,
                        int32_t seqlen_kv, int32_t head_dim, int32_t block_size, int32_t topk,
                        vsa_stream stream);

/*
 * vsa_forward_bshd - vsa_forward for [B, S, H, D] tensors (BSHD layout):
 * q [B,Sq,H,D], k/v [B,Skv,H,D], out [B,Sq,H,D]; everything else, including
 * block_size 64, 128 or 256, as vsa_forward.  ("[chore] release
 * fastvideo-kernel 0.3.0", Block-sparse / VSA attention improvements: the
 * BSHD-native video_sparse_attn_bshd() entry point.)
 */
int vsa_forward_bshd(const vsa_bf16 *q, const vsa_bf16 *k, const vsa_bf16 *v, const vsa_bf16 *gate,
                     int32_t gate_mode, const int64_t *gate_strides, vsa_bf16 *out, int32_t *q2k_idx,
                     int32_t *q2k_num, float *out_c, int32_t batch, int32_t heads, int32_t seqlen_q,
                     int32_t seqlen_kv, int32_t head_dim, int32_t block_size, int32_t topk,
                     void *workspace, size_t workspace_bytes, vsa_stream stream);

/*
 * vsa_forward_varlen - the whole PACKED forward in one launch per stage over
 * all sequences ("[kernel] Add varlen support for block-sparse attention",
 * Summary / How it works; "[chore] release fastvideo-kernel 0.3.0",
 * varlen block-sparse attention with Q/KV length mismatch).
 *
 * q [H, bs*Nq, D], k/v [H, bs*Nkv, D], out [H, bs*Nq, D] with bs =
 * block_size (padding slots of out are written with 0).  The device metadata
 * arrays and sizes are those of vsa_build_metadata for the same block_size
 * (topk_per_seq = its topk_clamped).  q2k_idx holds global
 * KV block numbers.  Optional outputs and workspace as for vsa_forward.
 */
int vsa_forward_varlen(const vsa_bf16 *q, const vsa_bf16 *k, const vsa_bf16 *v,
                       const vsa_bf16 *gate, int32_t gate_mode, const int64_t *gate_strides,
                       vsa_bf16 *out, int32_t *q2k_idx, int32_t *q2k_num, float *out_c,
                       const int32_t *cu_blocks_q, const int32_t *cu_blocks_kv,
                       const int32_t *block_sizes_q, const int32_t *block_sizes_kv,
                       const int32_t *topk_per_seq, int32_t num_seqs, int32_t total_q_blocks,
                       int32_t total_kv_blocks, int32_t max_q_blocks, int32_t max_kv_blocks,
                       int32_t max_topk, int32_t heads, int32_t head_dim, int32_t block_size,
                       void *workspace, size_t workspace_bytes, vsa_stream stream);

/*
 * Training: the forward that keeps what the backward needs, and the backward.
 * ("[kernel] Add varlen support for block-sparse attention", Test plan:
 * backward correctness of the block-sparse attention against per-sequence
 * references; "[chore] release fastvideo-kernel 0.3.0", Block-sparse / VSA
 * attention improvements: block-sparse attention forward and backward.)
 * The backward is the gradient of the forward with the routing (q2k_idx)
 * held fixed: the top-k choice is piecewise constant and carries none.
 * Both take every problem the forward takes: every layout, VSA blocks of
 * 64, 128 or 256 tokens.
 */

/*
 * vsa_sparse_attn_combine_train - vsa_sparse_attn_combine that also writes
 * out_s, the bf16 normalised block-sparse attention output on its own (query
 * layout, padding slots of PACKED written with 0), and lse, float32, one per
 * query row ([B, H, Sq] for DENSE and for BSHD, [H, bs*Nq] PACKED, padding
 * slots not written):
 * log2 of the softmax denominator of the row in units where the row's
 * probabilities are exp2(s * log2(e) / sqrt(D) - lse) for raw scores s = q.k
 * (-inf for a row whose list holds no valid block).  Arguments, checks and
 * errors as vsa_sparse_attn_combine; out_s and lse must not be NULL, out_s
 * 16-byte aligned, lse 4-byte aligned, and neither may overlap an input or
 * out (VSA_ERR_ALIAS).
 */
int vsa_sparse_attn_combine_train(const vsa_problem *problem, const vsa_bf16 *q, const vsa_bf16 *k,
                                  const vsa_bf16 *v, const int32_t *q2k_idx, const int32_t *q2k_num,
                                  const float *out_c, const vsa_bf16 *gate, int32_t gate_mode,
                                  const int64_t *gate_strides, vsa_bf16 *out, vsa_bf16 *out_s, float *lse,
                                  vsa_stream stream);

/*
 * vsa_backward_workspace_size - bytes of device workspace vsa_backward needs:
 * float64 block means of Q, K, V and their gradients, the coarse output
 * gradient (one row per VSA block), two float64 block-level matrices (VSA
 * query blocks x the most VSA KV blocks of a sequence: the coarse softmax and
 * its score gradient), 128 float32 row statistics per 64-token query block
 * and the inverse routing (64-token KV blocks x the most 64-token query
 * blocks of a sequence, int32).  Returns 0 when the problem is invalid.
 */
size_t vsa_backward_workspace_size(const vsa_problem *problem);

/*
 * vsa_backward - gradients of sum(out * dout) for the forward
 * out = out_c * gate + out_s run with these q, k, v, gate and routing.
 *
 * Inputs: q, k, v (bf16, layouts above); q2k_idx / q2k_num as written by
 * vsa_coarse_topk (each list strictly ascending); out_c (float32) from
 * vsa_coarse_topk; gate, gate_mode, gate_strides as for vsa_combine; out_s
 * and lse from vsa_sparse_attn_combine_train; dout (bf16, query layout; its
 * padding slots are not read).
 * Outputs (bf16, written in full, PACKED padding slots with 0): dq in the
 * query layout, dk and dv in the KV layout, and for a gate dgate, contiguous
 * in the query layout whatever gate_strides were: [B, H, Sq] (BSHD:
 * [B, Sq, H]) / [H, bs*Nq] for VSA_GATE_TOKEN, the same with a trailing D for
 * VSA_GATE_FULL (NULL and unused for VSA_GATE_NONE).  With VSA blocks of 128
 * or 256 tokens the gradients through the block means spread dQc, dKc, dVc
 * over the valid tokens of each VSA block.
 * Arithmetic: the coarse branch and the gradients through the block means
 * in float64; the block-sparse part as bf16 matrix products with float32
 * accumulation (probabilities recomputed from lse, rounded to bf16 as
 * product operands); one rounding per output element.  No atomics: results
 * are bit-for-bit repeatable.
 * Errors as vsa_sparse_attn_combine, plus VSA_ERR_NULL (a required pointer
 * NULL), VSA_ERR_ALIGN (tensors not 16-byte aligned, lse not 4-byte aligned,
 * workspace not 256-byte aligned), VSA_ERR_ALIAS (an output overlapping an
 * input or another output), VSA_ERR_WORKSPACE (fewer than
 * vsa_backward_workspace_size bytes).
 */
int vsa_backward(const vsa_problem *problem, const vsa_bf16 *q, const vsa_bf16 *k, const vsa_bf16 *v,
                 const int32_t *q2k_idx, const int32_t *q2k_num, const float *out_c, const vsa_bf16 *gate,
                 int32_t gate_mode, const int64_t *gate_strides, const vsa_bf16 *out_s, const float *lse,
                 const vsa_bf16 *dout, vsa_bf16 *dq, vsa_bf16 *dk, vsa_bf16 *dv, vsa_bf16 *dgate,
                 void *workspace, size_t workspace_bytes, vsa_stream stream);

/*
 * vsa_backward_pooled - vsa_backward that reads the float64 block means of
 * q, k and v from the forward instead of pooling q, k and v again (one pass
 * over the three tensors fewer; the gradients are bit-identical to
 * vsa_backward's).
 *
 * forward_workspace: the workspace (at least its first vsa_workspace_size
 * bytes, 256-byte aligned) of the vsa_coarse_topk or vsa_forward call that
 * produced q2k_idx, q2k_num and out_c for these q, k, v and this problem,
 * unchanged since; the library reads its block means and writes nothing to
 * it.  Not the scratch of vsa_forward_noalloc, which the next call reuses.
 * Every other argument as vsa_backward.
 * Errors as vsa_backward, plus VSA_ERR_WORKSPACE (forward_workspace NULL or
 * smaller than the forward's block means need), VSA_ERR_ALIGN (not 256-byte
 * aligned) and VSA_ERR_ALIAS (an output or the backward workspace overlapping
 * the forward's block means).
 */
int vsa_backward_pooled(const vsa_problem *problem, const vsa_bf16 *q, const vsa_bf16 *k, const vsa_bf16 *v,
                        const int32_t *q2k_idx, const int32_t *q2k_num, const float *out_c, const vsa_bf16 *gate,
                        int32_t gate_mode, const int64_t *gate_strides, const vsa_bf16 *out_s, const float *lse,
                        const vsa_bf16 *dout, vsa_bf16 *dq, vsa_bf16 *dk, vsa_bf16 *dv, vsa_bf16 *dgate,
                        const void *forward_workspace, size_t forward_workspace_bytes, void *workspace,
                        size_t workspace_bytes, vsa_stream stream);

/*
 * 3-D tile partition of video latents ("[kernel] Extract VSA utility
 * functions into fastvideo_kernel", Summary, Design decisions and review
 * thread: tile partition indices and their inverse, variable block sizes with
 * the tile size a parameter, the non-pad index, one-call metadata).
 *
 * A latent is a T x H x W grid of tokens flattened in raster order (w
 * fastest).  It is cut into tiles of tile_t x tile_h x tile_w tokens (at most
 * 256; 4 x 4 x 4 is the usual choice, 4 x 4 x 8 and 4 x 8 x 8 those of the
 * 128/256-token variants of "[chore] release fastvideo-kernel 0.3.0"), the
 * last tile along an axis shorter when the extent is not a multiple; tiles
 * are ordered in raster order of their tile coordinates and the tokens of a
 * tile in raster order.  Each tile is one VSA block of the PACKED layout:
 * bs = 64 slots for tiles of at most 64 tokens, else 128 or 256 (the
 * smallest that holds the tile), its first tile-size slots valid; the
 * block_size of the forward problem is bs.
 */

/*
 * vsa_tile_partition - host index arrays of the partition.
 * *num_tiles is always written.  Each output may be NULL:
 *   tile_sizes [num_tiles]                      valid tokens of each tile
 *   tile_partition_indices [T*H*W]              raster index of tiled position p
 *   reverse_tile_partition_indices [T*H*W]      tiled position of raster index r
 *   non_pad_index [T*H*W]                       slot bs*tile + rank of position p
 * Errors: VSA_ERR_NULL (num_tiles NULL), VSA_ERR_SHAPE (an extent < 1, a tile
 * of more than 256 tokens, more than 2^31 - 1 tokens or slots).
 */
int vsa_tile_partition(int32_t T, int32_t H, int32_t W, int32_t tile_t, int32_t tile_h, int32_t tile_w,
                       int32_t *num_tiles, int32_t *tile_sizes, int64_t *tile_partition_indices,
                       int64_t *reverse_tile_partition_indices, int64_t *non_pad_index);

/*
 * vsa_build_tile_metadata - the PACKED-layout metadata (same outputs and
 * conventions as vsa_build_metadata) of num_videos videos of one grid packed
 * one after another, queries and keys/values on the same tiles, top-k
 * clamped to the tile count; the slot counts in `sizes` are for blocks of bs
 * slots (the forward's block_size).  Errors as vsa_build_metadata and
 * vsa_tile_partition; VSA_ERR_UNSUPPORTED beyond 4096 tiles per video.
 */
int vsa_build_tile_metadata(int32_t num_videos, int32_t T, int32_t H, int32_t W, int32_t tile_t,
                            int32_t tile_h, int32_t tile_w, int32_t topk, vsa_meta_sizes *sizes,
                            int32_t *cu_blocks_q, int32_t *cu_blocks_kv, int32_t *block_sizes_q,
                            int32_t *block_sizes_kv, int32_t *topk_clamped);

/*
 * vsa_tile_gather - x [batch, heads, T*H*W, elems] (raster order, contiguous,
 * bf16) -> y [heads, batch * bs * num_tiles, elems] in tile order, video b at
 * slots [b * bs * num_tiles, (b + 1) * bs * num_tiles), padding slots written
 * with 0: the PACKED input of vsa_forward_varlen for the metadata of
 * vsa_build_tile_metadata (elems = head_dim for q/k/v, 1 for a per-token
 * gate, head_dim for a full gate).
 * vsa_tile_scatter - the inverse, y -> x (padding slots are not read).
 * Device pointers, asynchronous on stream.  elems a multiple of 8 needs
 * 16-byte aligned tensors, otherwise 2-byte.  Errors: VSA_ERR_NULL,
 * VSA_ERR_SHAPE, VSA_ERR_ALIGN, VSA_ERR_ALIAS (x and y overlap), VSA_ERR_HIP.
 */
int vsa_tile_gather(const vsa_bf16 *x, vsa_bf16 *y, int32_t batch, int32_t heads, int32_t T, int32_t H,
                    int32_t W, int32_t tile_t, int32_t tile_h, int32_t tile_w, int32_t elems,
                    vsa_stream stream);
int vsa_tile_scatter(const vsa_bf16 *y, vsa_bf16 *x, int32_t batch, int32_t heads, int32_t T, int32_t H,
                     int32_t W, int32_t tile_t, int32_t tile_h, int32_t tile_w, int32_t elems,
                     vsa_stream stream);

/* Text for a status code (static storage). */
const char *vsa_status_string(int status);

/* Detail of the last error on the calling thread ("" if none). */
const char *vsa_last_error(void);

/* Library version string. */
const char *vsa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* VSA_H */
