// Host side of libvsa: argument validation, block metadata, workspace
// partitioning and the launch sequence of every C entry point declared in
// vsa.h.  Nothing here allocates device memory or synchronises the stream.
#include <stdarg.h>
#include <stdio.h>

#include <algorithm>
#include <mutex>
#include <string>

#include "vsa_internal.hpp"

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_err = buf;
    return code;
}

int ok() {
    g_err.clear();
    return VSA_OK;
}

constexpr int64_t kGridYZMax = 65535;
constexpr size_t kAlign = 256;

size_t round_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Validate a problem and build its kernel-side view.
int make_problem(const vsa_problem* pr, vsa::DevProblem* P) {
    if (!pr) return fail(VSA_ERR_NULL, "problem is NULL");
    const bool dense = pr->layout == VSA_LAYOUT_DENSE || pr->layout == VSA_LAYOUT_BSHD;
    if (pr->block_size != VSA_BLOCK && pr->block_size != 128 && pr->block_size != 256)
        return fail(VSA_ERR_UNSUPPORTED, "block_size %d unsupported (64, 128 or 256)", pr->block_size);
    if (pr->head_dim != 64 && pr->head_dim != 128)
        return fail(VSA_ERR_UNSUPPORTED, "head_dim %d unsupported (64 or 128)", pr->head_dim);
    if (pr->heads < 1) return fail(VSA_ERR_SHAPE, "heads must be >= 1 (got %d)", pr->heads);
    if (pr->heads > kGridYZMax) return fail(VSA_ERR_UNSUPPORTED, "heads > %lld", (long long)kGridYZMax);
    *P = vsa::DevProblem{};
    P->H = pr->heads;
    P->D = pr->head_dim;
    P->ratio = pr->block_size / VSA_BLOCK;
    if (dense) {
        if (pr->batch < 1) return fail(VSA_ERR_SHAPE, "empty batch (batch=%d)", pr->batch);
        if (3LL * pr->batch > kGridYZMax) return fail(VSA_ERR_UNSUPPORTED, "batch too large");
        if (pr->seqlen_q < 1 || pr->seqlen_kv < 1)
            return fail(VSA_ERR_SHAPE, "zero-length sequence (Sq=%d, Skv=%d)", pr->seqlen_q, pr->seqlen_kv);
        if (pr->topk < 1) return fail(VSA_ERR_TOPK, "topk must be >= 1 (got %d)", pr->topk);
        P->packed = 0;
        P->nseq = pr->batch;
        P->Sq = pr->seqlen_q;
        P->Skv = pr->seqlen_kv;
        const int64_t sq = pr->seqlen_q, skv = pr->seqlen_kv, bs = pr->block_size;
        P->nQ = (int)((sq + VSA_BLOCK - 1) / VSA_BLOCK);
        P->nKV = (int)((skv + VSA_BLOCK - 1) / VSA_BLOCK);
        P->nQB = (int)((sq + bs - 1) / bs);
        P->nKVB = (int)((skv + bs - 1) / bs);
        if (P->nKVB > vsa::kMaxKvBlocks)
            return fail(VSA_ERR_UNSUPPORTED, "%d KV blocks per sequence exceeds %d", P->nKVB, vsa::kMaxKvBlocks);
        P->kk = std::min(pr->topk, P->nKVB);
        P->idx_row = P->kk;
        if ((int64_t)P->nQ * P->H * P->nseq > 0x7fffffffLL)
            return fail(VSA_ERR_UNSUPPORTED, "too many query blocks in one launch");
        const int64_t H = P->H, D = P->D, Sq = P->Sq, Skv = P->Skv;
        if (pr->layout == VSA_LAYOUT_DENSE) {  // [B, H, S, D]
            P->q_sb = H * Sq * D, P->q_sh = Sq * D, P->q_st = D;
            P->kv_sb = H * Skv * D, P->kv_sh = Skv * D, P->kv_st = D;
        } else {  // [B, S, H, D]
            P->bshd = 1;
            P->q_sb = Sq * H * D, P->q_sh = D, P->q_st = H * D;
            P->kv_sb = Skv * H * D, P->kv_sh = D, P->kv_st = H * D;
        }
    } else if (pr->layout == VSA_LAYOUT_PACKED) {
        if (pr->num_seqs < 1) return fail(VSA_ERR_SHAPE, "empty batch (num_seqs=%d)", pr->num_seqs);
        if (pr->num_seqs > kGridYZMax) return fail(VSA_ERR_UNSUPPORTED, "num_seqs > %lld", (long long)kGridYZMax);
        if (!pr->cu_blocks_q || !pr->cu_blocks_kv || !pr->block_sizes_q || !pr->block_sizes_kv ||
            !pr->topk_per_seq)
            return fail(VSA_ERR_NULL, "packed metadata array is NULL");
        if (pr->total_q_blocks < pr->num_seqs || pr->total_kv_blocks < pr->num_seqs)
            return fail(VSA_ERR_SHAPE, "every sequence needs at least one block (Nq=%d, Nkv=%d, seqs=%d)",
                        pr->total_q_blocks, pr->total_kv_blocks, pr->num_seqs);
        if (pr->max_q_blocks < 1 || pr->max_q_blocks > pr->total_q_blocks || pr->max_kv_blocks < 1 ||
            pr->max_kv_blocks > pr->total_kv_blocks)
            return fail(VSA_ERR_SHAPE, "max block counts inconsistent with totals");
        if (pr->max_kv_blocks > vsa::kMaxKvBlocks)
            return fail(VSA_ERR_UNSUPPORTED, "%d KV blocks per sequence exceeds %d", pr->max_kv_blocks,
                        vsa::kMaxKvBlocks);
        if (pr->max_topk < 1) return fail(VSA_ERR_TOPK, "max_topk must be >= 1 (got %d)", pr->max_topk);
        if ((int64_t)pr->total_q_blocks * pr->heads * P->ratio > 0x7fffffffLL)
            return fail(VSA_ERR_UNSUPPORTED, "too many query blocks in one launch");
        if ((int64_t)std::max(pr->total_q_blocks, pr->total_kv_blocks) * pr->block_size > 0x7fffffffLL)
            return fail(VSA_ERR_SHAPE, "packed length exceeds 2^31 slots");
        P->packed = 1;
        P->nseq = pr->num_seqs;
        P->cu_q = pr->cu_blocks_q;
        P->cu_kv = pr->cu_blocks_kv;
        P->bs_q = pr->block_sizes_q;
        P->bs_kv = pr->block_sizes_kv;
        P->topk_s = pr->topk_per_seq;
        P->total_q = pr->total_q_blocks;
        P->total_kv = pr->total_kv_blocks;
        P->max_q = pr->max_q_blocks;
        P->max_kv = pr->max_kv_blocks;
        P->max_topk = pr->max_topk;
        P->idx_row = pr->max_topk;
        P->q_st = P->kv_st = P->D;  // rows of the packed layout are contiguous
        P->q_sh = (int64_t)pr->total_q_blocks * pr->block_size * P->D;
        P->kv_sh = (int64_t)pr->total_kv_blocks * pr->block_size * P->D;
    } else {
        return fail(VSA_ERR_UNSUPPORTED, "unknown layout %d", pr->layout);
    }
    return VSA_OK;
}

// element counts of the token-resolution tensors
int64_t q_elems(const vsa::DevProblem& P) {
    return P.packed ? (int64_t)P.H * P.total_q * P.ratio * VSA_BLOCK * P.D : (int64_t)P.nseq * P.H * P.Sq * P.D;
}
int64_t kv_elems(const vsa::DevProblem& P) {
    return P.packed ? (int64_t)P.H * P.total_kv * P.ratio * VSA_BLOCK * P.D : (int64_t)P.nseq * P.H * P.Skv * P.D;
}
// 64-token block counts (the attention kernels' granularity)
int64_t qblocks64(const vsa::DevProblem& P) {
    return P.packed ? (int64_t)P.H * P.total_q * P.ratio : (int64_t)P.nseq * P.H * P.nQ;
}
int64_t kvblocks64(const vsa::DevProblem& P) {
    return P.packed ? (int64_t)P.H * P.total_kv * P.ratio : (int64_t)P.nseq * P.H * P.nKV;
}
// block-resolution array lengths (VSA blocks)
int64_t qblocks(const vsa::DevProblem& P) {
    return P.packed ? (int64_t)P.H * P.total_q : (int64_t)P.nseq * P.H * P.nQB;
}
int64_t kvblocks(const vsa::DevProblem& P) {
    return P.packed ? (int64_t)P.H * P.total_kv : (int64_t)P.nseq * P.H * P.nKVB;
}

struct Workspace {
    double *qc, *kc, *vc;
    double* coarse;  // block-level scores / weights and their row sums
    float* out_c;
    int *idx, *num;
    size_t coarse_bytes, total_bytes;
};

Workspace plan_workspace(const vsa::DevProblem& P, void* base) {
    Workspace w{};
    char* p = (char*)base;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        char* r = p ? p + off : nullptr;
        off += round_up(bytes);
        return r;
    };
    w.qc = (double*)take(sizeof(double) * qblocks(P) * P.D);
    w.kc = (double*)take(sizeof(double) * kvblocks(P) * P.D);
    w.vc = (double*)take(sizeof(double) * kvblocks(P) * P.D);
    w.coarse = (double*)take(sizeof(double) * vsa::coarse_scratch_doubles(vsa::coarse_view(P)));
    w.coarse_bytes = off;
    w.out_c = (float*)take(sizeof(float) * qblocks(P) * P.D);
    w.idx = (int*)take(sizeof(int) * qblocks(P) * P.idx_row);
    w.num = (int*)take(sizeof(int) * qblocks(P));
    w.total_bytes = off;
    return w;
}

struct BwdWorkspace {
    double *qc, *kc, *vc, *doc, *dqc, *dkc, *dvc, *pbuf, *dsbuf;
    float* rs;
    int *k2q, *k2q_num;
    size_t total_bytes;
};

BwdWorkspace plan_bwd_workspace(const vsa::DevProblem& P, void* base) {
    BwdWorkspace w{};
    char* p = (char*)base;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        char* r = p ? p + off : nullptr;
        off += round_up(bytes);
        return r;
    };
    // coarse matrices per VSA block; statistics and inverse lists per 64-token block
    const int64_t maxq = P.packed ? P.max_q : P.nQB, maxkv = P.packed ? P.max_kv : P.nKVB;
    const int64_t maxq64 = P.packed ? (int64_t)P.max_q * P.ratio : P.nQ;
    const size_t qd = sizeof(double) * qblocks(P) * P.D, kd = sizeof(double) * kvblocks(P) * P.D;
    w.qc = (double*)take(qd);
    w.kc = (double*)take(kd);
    w.vc = (double*)take(kd);
    w.doc = (double*)take(qd);
    w.dqc = (double*)take(qd);
    w.dkc = (double*)take(kd);
    w.dvc = (double*)take(kd);
    const int64_t coarse_rows = (int64_t)P.nseq * P.H * maxq;
    w.pbuf = (double*)take(sizeof(double) * coarse_rows * maxkv);
    w.dsbuf = (double*)take(sizeof(double) * coarse_rows * maxkv);
    w.rs = (float*)take(sizeof(float) * qblocks64(P) * vsa::kStatRow);
    w.k2q = (int*)take(sizeof(int) * kvblocks64(P) * maxq64);
    w.k2q_num = (int*)take(sizeof(int) * kvblocks64(P));
    w.total_bytes = off;
    return w;
}

bool overlaps(const void* a, int64_t abytes, const void* b, int64_t bbytes) {
    const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
    return a0 < b0 + (uintptr_t)bbytes && b0 < a0 + (uintptr_t)abytes;
}

int check_qkv(const vsa::DevProblem&, const void* q, const void* k, const void* v) {
    if (!q || !k || !v) return fail(VSA_ERR_NULL, "q, k or v is NULL");
    if (!aligned16(q) || !aligned16(k) || !aligned16(v)) return fail(VSA_ERR_ALIGN, "q, k and v must be 16-byte aligned");
    return VSA_OK;
}

int check_out_alias(const vsa::DevProblem& P, const void* out, const void* q, const void* k, const void* v) {
    const int64_t qb = 2 * q_elems(P), kb = 2 * kv_elems(P);
    if (overlaps(out, qb, q, qb) || overlaps(out, qb, k, kb) || overlaps(out, qb, v, kb))
        return fail(VSA_ERR_ALIAS, "out overlaps q, k or v");
    return VSA_OK;
}

int hip_status(hipError_t e, const char* what) {
    if (e == hipSuccess) return VSA_OK;
    return fail(VSA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

int gate_strides(const vsa::DevProblem& P, const uint16_t* gate, int mode, const int64_t* gs,
                 int64_t out[3]) {
    out[0] = out[1] = out[2] = 0;
    if (mode == VSA_GATE_NONE) return VSA_OK;
    if (mode != VSA_GATE_TOKEN && mode != VSA_GATE_FULL) return fail(VSA_ERR_GATE, "unknown gate mode %d", mode);
    if (!gate) return fail(VSA_ERR_NULL, "gate is NULL with gate_mode %d", mode);
    const int64_t dmul = mode == VSA_GATE_FULL ? P.D : 1;
    if (gs) {
        for (int i = 0; i < 3; ++i) {
            if (gs[i] < 0) return fail(VSA_ERR_GATE, "negative gate stride");
            out[i] = gs[i];
        }
        if (!P.packed && P.Sq > 1 && out[2] == 0) return fail(VSA_ERR_GATE, "gate token stride is 0");
        if (P.H > 1 && out[1] == 0) return fail(VSA_ERR_GATE, "gate head stride is 0");
    } else if (!P.packed && !P.bshd) {  // [B, H, Sq(, D)]
        out[2] = dmul;
        out[1] = (int64_t)P.Sq * dmul;
        out[0] = (int64_t)P.H * P.Sq * dmul;
    } else if (!P.packed) {  // [B, Sq, H(, D)]
        out[2] = (int64_t)P.H * dmul;
        out[1] = dmul;
        out[0] = (int64_t)P.Sq * P.H * dmul;
    } else {
        out[2] = dmul;
        out[1] = (int64_t)P.total_q * P.ratio * VSA_BLOCK * dmul;
        out[0] = 0;
    }
    if (mode == VSA_GATE_FULL) {
        if (!aligned16(gate)) return fail(VSA_ERR_ALIGN, "full gate must be 16-byte aligned");
        for (int i = 0; i < 3; ++i)
            if (out[i] % 8) return fail(VSA_ERR_ALIGN, "full gate strides must be multiples of 8 elements");
    } else if (((uintptr_t)gate & 1u) != 0) {
        return fail(VSA_ERR_ALIGN, "gate must be 2-byte aligned");
    }
    return VSA_OK;
}

int run_coarse(const vsa::DevProblem& P, const uint16_t* q, const uint16_t* k, const uint16_t* v,
               float* out_c, int* idx, int* num, const Workspace& w, hipStream_t st) {
    // Q and K are pooled first; V is pooled by workgroups of the first score
    // launch, which needs only Q and K and, being latency-bound, leaves most
    // of the HBM bandwidth to them
    int rc = hip_status(vsa::launch_pool_qk(P, q, k, w.qc, w.kc, st), "pool launch");
    if (rc) return rc;
    return hip_status(vsa::launch_coarse_topk(vsa::coarse_view(P), w.qc, w.kc, w.vc, out_c, idx, num, w.coarse, st,
                                              &P, v),
                      "coarse/top-k launch");
}

int check_tiles(int32_t T, int32_t H, int32_t W, int32_t tt, int32_t th, int32_t tw, vsa::TileGrid* g) {
    if (T < 1 || H < 1 || W < 1) return fail(VSA_ERR_SHAPE, "grid extents must be >= 1 (got %d x %d x %d)", T, H, W);
    if (tt < 1 || th < 1 || tw < 1 || (int64_t)tt * th * tw > 4 * VSA_BLOCK)
        return fail(VSA_ERR_SHAPE, "tile %d x %d x %d: extents must be >= 1 and the tile at most %d tokens", tt, th,
                    tw, 4 * VSA_BLOCK);
    if ((int64_t)T * H * W > 0x7fffffffLL) return fail(VSA_ERR_SHAPE, "grid exceeds 2^31 - 1 tokens");
    *g = vsa::make_tile_grid(T, H, W, tt, th, tw);
    if ((int64_t)g->ntiles * g->blk > 0x7fffffffLL) return fail(VSA_ERR_SHAPE, "padded length exceeds 2^31 slots");
    return VSA_OK;
}

int tile_copy(const vsa_bf16* src, vsa_bf16* dst, int32_t batch, int32_t heads, int32_t T, int32_t H, int32_t W,
              int32_t tt, int32_t th, int32_t tw, int32_t elems, bool scatter, vsa_stream stream) {
    vsa::TileGrid g;
    int rc = check_tiles(T, H, W, tt, th, tw, &g);
    if (rc) return rc;
    if (batch < 1 || heads < 1 || elems < 1)
        return fail(VSA_ERR_SHAPE, "batch, heads and elems must be >= 1 (got %d, %d, %d)", batch, heads, elems);
    if ((int64_t)batch * g.ntiles * g.blk > 0x7fffffffLL)
        return fail(VSA_ERR_SHAPE, "packed length exceeds 2^31 slots");
    if (!src || !dst) return fail(VSA_ERR_NULL, "source or destination is NULL");
    const bool vec = elems % 8 == 0;
    const uintptr_t mask = vec ? 15u : 1u;
    if (((uintptr_t)src & mask) || ((uintptr_t)dst & mask))
        return fail(VSA_ERR_ALIGN, "tensors must be %d-byte aligned", vec ? 16 : 2);
    const int64_t raster_bytes = 2LL * batch * heads * ((int64_t)T * H * W) * elems;
    const int64_t tiled_bytes = 2LL * batch * heads * ((int64_t)g.ntiles * g.blk) * elems;
    const int64_t sb = scatter ? tiled_bytes : raster_bytes, db = scatter ? raster_bytes : tiled_bytes;
    if (overlaps(src, sb, dst, db)) return fail(VSA_ERR_ALIAS, "source and destination overlap");
    rc = hip_status(vsa::launch_tile_copy(g, src, dst, batch, heads, elems, scatter, (hipStream_t)stream),
                    scatter ? "tile scatter launch" : "tile gather launch");
    return rc ? rc : ok();
}

}  // namespace

// ---------------------------------------------------------------------------
// vsa_forward_noalloc: vsa_forward with its workspace in a file-scope device
// array instead of a caller-provided buffer, for callers that cannot allocate
// device memory (HIP graph capture, tight serving loops).  Every GPU the
// library runs on holds its own copy of the array (kNoAllocScratchBytes) from
// the module's load until the process ends.  In host code `scratch` names a
// host-side stand-in, not a device address: the array's device address is
// taken once per device with hipGetSymbolAddress, with that device current,
// and only that address is handed to kernels.
// ---------------------------------------------------------------------------
constexpr size_t kNoAllocScratchBytes = (size_t)96 << 20;
static __device__ __attribute__((aligned(256))) unsigned char scratch[kNoAllocScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};  // device address of `scratch` per device, set once

// The current device's address of `scratch` (taken on the first call on that
// device).  Returns VSA_OK or an error code with the detail set.
int scratch_address(void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return fail(VSA_ERR_HIP, "hipGetDevice failed");
    if (dev >= kMaxDevices) return fail(VSA_ERR_UNSUPPORTED, "device %d beyond %d", dev, kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return fail(VSA_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return VSA_OK;
}
}  // namespace

extern "C" {

const char* vsa_status_string(int status) {
    switch (status) {
        case VSA_OK: return "ok";
        case VSA_ERR_NULL: return "NULL pointer";
        case VSA_ERR_UNSUPPORTED: return "unsupported configuration";
        case VSA_ERR_TOPK: return "invalid topk";
        case VSA_ERR_SHAPE: return "invalid shape";
        case VSA_ERR_GATE: return "invalid gate";
        case VSA_ERR_WORKSPACE: return "workspace missing or too small";
        case VSA_ERR_ALIGN: return "misaligned pointer or stride";
        case VSA_ERR_ALIAS: return "output overlaps an input";
        case VSA_ERR_HIP: return "HIP runtime error";
        default: return "unknown status";
    }
}

const char* vsa_last_error(void) { return g_err.c_str(); }

const char* vsa_version(void) { return "libvsa 0.1.0 gfx950"; }

int vsa_build_metadata(int32_t num_seqs, const int32_t* seqlens_q, const int32_t* seqlens_kv,
                       const int32_t* topk, int32_t block_size, vsa_meta_sizes* sizes, int32_t* cu_blocks_q,
                       int32_t* cu_blocks_kv, int32_t* block_sizes_q, int32_t* block_sizes_kv,
                       int32_t* topk_clamped) {
    if (!sizes) return fail(VSA_ERR_NULL, "sizes is NULL");
    *sizes = vsa_meta_sizes{};
    if (block_size != VSA_BLOCK && block_size != 128 && block_size != 256)
        return fail(VSA_ERR_UNSUPPORTED, "block_size %d unsupported (64, 128 or 256)", block_size);
    const int bs = block_size;
    if (num_seqs < 1) return fail(VSA_ERR_SHAPE, "empty batch (num_seqs=%d)", num_seqs);
    if (!seqlens_q || !topk) return fail(VSA_ERR_NULL, "seqlens_q or topk is NULL");
    const int nout = !!cu_blocks_q + !!cu_blocks_kv + !!block_sizes_q + !!block_sizes_kv + !!topk_clamped;
    if (nout != 0 && nout != 5) return fail(VSA_ERR_NULL, "pass all five output arrays or none");
    if (!seqlens_kv) seqlens_kv = seqlens_q;
    int64_t tq = 0, tkv = 0;
    int32_t mq = 0, mkv = 0, mk = 0;
    for (int s = 0; s < num_seqs; ++s) {
        if (seqlens_q[s] < 1 || seqlens_kv[s] < 1)
            return fail(VSA_ERR_SHAPE, "sequence %d has zero length (q=%d, kv=%d)", s, seqlens_q[s], seqlens_kv[s]);
        if (topk[s] < 1) return fail(VSA_ERR_TOPK, "sequence %d: topk must be >= 1 (got %d)", s, topk[s]);
        const int32_t nq = (int32_t)(((int64_t)seqlens_q[s] + bs - 1) / bs);
        const int32_t nkv = (int32_t)(((int64_t)seqlens_kv[s] + bs - 1) / bs);
        tq += nq;
        tkv += nkv;
        mq = std::max(mq, nq);
        mkv = std::max(mkv, nkv);
        mk = std::max(mk, std::min(topk[s], nkv));
    }
    if (tq * bs > 0x7fffffffLL || tkv * bs > 0x7fffffffLL)
        return fail(VSA_ERR_SHAPE, "packed length exceeds 2^31 slots");
    sizes->num_seqs = num_seqs;
    sizes->total_q_blocks = (int32_t)tq;
    sizes->total_kv_blocks = (int32_t)tkv;
    sizes->max_q_blocks = mq;
    sizes->max_kv_blocks = mkv;
    sizes->max_topk = mk;
    sizes->q_slots = tq * bs;
    sizes->kv_slots = tkv * bs;
    if (nout == 0) return ok();
    int32_t oq = 0, okv = 0;
    for (int s = 0; s < num_seqs; ++s) {
        const int32_t nq = (seqlens_q[s] + bs - 1) / bs;
        const int32_t nkv = (seqlens_kv[s] + bs - 1) / bs;
        cu_blocks_q[s] = oq;
        cu_blocks_kv[s] = okv;
        for (int i = 0; i < nq; ++i) block_sizes_q[oq + i] = std::min(bs, seqlens_q[s] - bs * i);
        for (int j = 0; j < nkv; ++j) block_sizes_kv[okv + j] = std::min(bs, seqlens_kv[s] - bs * j);
        topk_clamped[s] = std::min(topk[s], nkv);
        oq += nq;
        okv += nkv;
    }
    cu_blocks_q[num_seqs] = oq;
    cu_blocks_kv[num_seqs] = okv;
    return ok();
}

size_t vsa_workspace_size(const vsa_problem* problem) {
    vsa::DevProblem P;
    if (make_problem(problem, &P) != VSA_OK) return 0;
    return plan_workspace(P, nullptr).total_bytes;
}

int vsa_coarse_topk(const vsa_problem* problem, const vsa_bf16* q, const vsa_bf16* k, const vsa_bf16* v,
                    float* out_c, int32_t* q2k_idx, int32_t* q2k_num, void* workspace,
                    size_t workspace_bytes, vsa_stream stream) {
    vsa::DevProblem P;
    int rc = make_problem(problem, &P);
    if (rc) return rc;
    if ((rc = check_qkv(P, q, k, v))) return rc;
    if (!out_c || !q2k_idx || !q2k_num) return fail(VSA_ERR_NULL, "out_c, q2k_idx or q2k_num is NULL");
    if (!aligned16(out_c)) return fail(VSA_ERR_ALIGN, "out_c must be 16-byte aligned");
    if (((uintptr_t)q2k_idx & 3u) || ((uintptr_t)q2k_num & 3u)) return fail(VSA_ERR_ALIGN, "index arrays must be 4-byte aligned");
    if (!workspace) return fail(VSA_ERR_WORKSPACE, "workspace is NULL");
    if ((uintptr_t)workspace % kAlign) return fail(VSA_ERR_ALIGN, "workspace must be 256-byte aligned");
    const Workspace w = plan_workspace(P, workspace);
    if (workspace_bytes < w.coarse_bytes)
        return fail(VSA_ERR_WORKSPACE, "workspace holds %zu bytes, needs %zu", workspace_bytes, w.coarse_bytes);
    rc = run_coarse(P, q, k, v, out_c, q2k_idx, q2k_num, w, (hipStream_t)stream);
    return rc ? rc : ok();
}

int vsa_sparse_attn_from_indices(const vsa_problem* problem, const vsa_bf16* q, const vsa_bf16* k,
                                 const vsa_bf16* v, const int32_t* q2k_idx, const int32_t* q2k_num,
                                 vsa_bf16* out, vsa_stream stream) {
    vsa::DevProblem P;
    int rc = make_problem(problem, &P);
    if (rc) return rc;
    if ((rc = check_qkv(P, q, k, v))) return rc;
    if (!q2k_idx || !q2k_num || !out) return fail(VSA_ERR_NULL, "q2k_idx, q2k_num or out is NULL");
    if (!aligned16(out)) return fail(VSA_ERR_ALIGN, "out must be 16-byte aligned");
    if ((rc = check_out_alias(P, out, q, k, v))) return rc;
    rc = hip_status(vsa::launch_sparse_attn(P, q, k, v, q2k_idx, q2k_num, out, (hipStream_t)stream),
                    "sparse attention launch");
    return rc ? rc : ok();
}

int vsa_sparse_attn_combine(const vsa_problem* problem, const vsa_bf16* q, const vsa_bf16* k,
                            const vsa_bf16* v, const int32_t* q2k_idx, const int32_t* q2k_num,
                            const float* out_c, const vsa_bf16* gate, int32_t gate_mode,
                            const int64_t* gate_strides_in, vsa_bf16* out, vsa_stream stream) {
    vsa::DevProblem P;
    int rc = make_problem(problem, &P);
    if (rc) return rc;
    if ((rc = check_qkv(P, q, k, v))) return rc;
    if (!q2k_idx || !q2k_num || !out || !out_c) return fail(VSA_ERR_NULL, "q2k_idx, q2k_num, out_c or out is NULL");
    if (!aligned16(out) || !aligned16(out_c)) return fail(VSA_ERR_ALIGN, "out_c and out must be 16-byte aligned");
    if ((rc = check_out_alias(P, out, q, k, v))) return rc;
    int64_t gs[3];
    if ((rc = gate_strides(P, gate, gate_mode, gate_strides_in, gs))) return rc;
    if (gate_mode != VSA_GATE_NONE && overlaps(out, 2 * q_elems(P), gate, 2))
        return fail(VSA_ERR_ALIAS, "gate overlaps out");
    rc = hip_status(vsa::launch_sparse_attn_combine(P, q, k, v, q2k_idx, q2k_num, out_c, gate, gate_mode, gs[0],
                                                    gs[1], gs[2], out, nullptr, nullptr, (hipStream_t)stream),
                    "fused sparse attention launch");
    return rc ? rc : ok();
}

int vsa_sparse_attn_combine_train(const vsa_problem* problem, const vsa_bf16* q, const vsa_bf16* k,
                                  const vsa_bf16* v, const int32_t* q2k_idx, const int32_t* q2k_num,
                                  const float* out_c, const vsa_bf16* gate, int32_t gate_mode,
                                  const int64_t* gate_strides_in, vsa_bf16* out, vsa_bf16* out_s, float* lse,
                                  vsa_stream stream) {
    vsa::DevProblem P;
    int rc = make_problem(problem, &P);
    if (rc) return rc;
    if ((rc = check_qkv(P, q, k, v))) return rc;
    if (!q2k_idx || !q2k_num || !out || !out_c || !out_s || !lse)
        return fail(VSA_ERR_NULL, "q2k_idx, q2k_num, out_c, out, out_s or lse is NULL");
    if (!aligned16(out) || !aligned16(out_c) || !aligned16(out_s))
        return fail(VSA_ERR_ALIGN, "out_c, out and out_s must be 16-byte aligned");
    if ((uintptr_t)lse & 3u) return fail(VSA_ERR_ALIGN, "lse must be 4-byte aligned");
    if ((rc = check_out_alias(P, out, q, k, v))) return rc;
    if ((rc = check_out_alias(P, out_s, q, k, v))) return rc;
    const int64_t ob = 2 * q_elems(P), lb = 4 * (q_elems(P) / P.D);
    if (overlaps(out, ob, out_s, ob)) return fail(VSA_ERR_ALIAS, "out_s overlaps out");
    if (overlaps(lse, lb, q, ob) || overlaps(lse, lb, k, 2 * kv_elems(P)) || overlaps(lse, lb, v, 2 * kv_elems(P)) ||
        overlaps(lse, lb, out, ob) || overlaps(lse, lb, out_s, ob))
        return fail(VSA_ERR_ALIAS, "lse overlaps an input, out or out_s");
    int64_t gs[3];
    if ((rc = gate_strides(P, gate, gate_mode, gate_strides_in, gs))) return rc;
    if (gate_mode != VSA_GATE_NONE && (overlaps(out, ob, gate, 2) || overlaps(out_s, ob, gate, 2)))
        return fail(VSA_ERR_ALIAS, "gate overlaps out or out_s");
    rc = hip_status(vsa::launch_sparse_attn_combine(P, q, k, v, q2k_idx, q2k_num, out_c, gate, gate_mode, gs[0],
                                                    gs[1], gs[2], out, out_s, lse, (hipStream_t)stream),
                    "fused sparse attention launch");
    return rc ? rc : ok();
}

size_t vsa_backward_workspace_size(const vsa_problem* problem) {
    vsa::DevProblem P;
    if (make_problem(problem, &P) != VSA_OK) return 0;
    return plan_bwd_workspace(P, nullptr).total_bytes;
}

// The backward; with forward_workspace (the workspace of the forward call that
// produced the routing) the block means of q, k and v are read from it
// instead of being pooled again.
static int backward_common(const vsa_problem* problem, const vsa_bf16* q, const vsa_bf16* k, const vsa_bf16* v,
                           const int32_t* q2k_idx, const int32_t* q2k_num, const float* out_c,
                           const vsa_bf16* gate, int32_t gate_mode, const int64_t* gate_strides_in,
                           const vsa_bf16* out_s, const float* lse, const vsa_bf16* dout, vsa_bf16* dq,
                           vsa_bf16* dk, vsa_bf16* dv, vsa_bf16* dgate, void* workspace, size_t workspace_bytes,
                           const void* forward_workspace, size_t forward_workspace_bytes, bool use_forward,
                           vsa_stream stream) {
    vsa::DevProblem P;
    int rc = make_problem(problem, &P);
    if (rc) return rc;
    if ((rc = check_qkv(P, q, k, v))) return rc;
    if (!q2k_idx || !q2k_num || !out_c || !out_s || !lse || !dout || !dq || !dk || !dv)
        return fail(VSA_ERR_NULL, "a required input or output pointer is NULL");
    if (!aligned16(out_c) || !aligned16(out_s) || !aligned16(dout) || !aligned16(dq) || !aligned16(dk) ||
        !aligned16(dv))
        return fail(VSA_ERR_ALIGN, "out_c, out_s, dout, dq, dk and dv must be 16-byte aligned");
    if ((uintptr_t)lse & 3u) return fail(VSA_ERR_ALIGN, "lse must be 4-byte aligned");
    if (((uintptr_t)q2k_idx & 3u) || ((uintptr_t)q2k_num & 3u))
        return fail(VSA_ERR_ALIGN, "index arrays must be 4-byte aligned");
    int64_t gs[3];
    if ((rc = gate_strides(P, gate, gate_mode, gate_strides_in, gs))) return rc;
    if (gate_mode != VSA_GATE_NONE) {
        if (!dgate) return fail(VSA_ERR_NULL, "dgate is NULL with gate_mode %d", gate_mode);
        if (gate_mode == VSA_GATE_FULL ? !aligned16(dgate) : ((uintptr_t)dgate & 1u) != 0)
            return fail(VSA_ERR_ALIGN, "dgate must be %d-byte aligned", gate_mode == VSA_GATE_FULL ? 16 : 2);
    }
    // every output against every input and the other outputs
    const int64_t qbytes = 2 * q_elems(P), kbytes = 2 * kv_elems(P), rows = q_elems(P) / P.D;
    const int64_t gbytes = gate_mode == VSA_GATE_FULL ? qbytes : 2 * rows;
    struct Span {
        const void* p;
        int64_t n;
    };
    const Span ins[] = {{q, qbytes},        {k, kbytes},       {v, kbytes},
                        {dout, qbytes},     {out_s, qbytes},   {lse, 4 * rows},
                        {out_c, 4 * qblocks(P) * P.D},         {gate, gate_mode != VSA_GATE_NONE ? 2 : 0}};
    const Span outs[] = {{dq, qbytes}, {dk, kbytes}, {dv, kbytes}, {dgate, gate_mode != VSA_GATE_NONE ? gbytes : 0}};
    for (int a = 0; a < 4; ++a) {
        if (!outs[a].n) continue;
        for (const Span& in : ins)
            if (in.n && overlaps(outs[a].p, outs[a].n, in.p, in.n))
                return fail(VSA_ERR_ALIAS, "an output of the backward overlaps one of its inputs");
        for (int b = a + 1; b < 4; ++b)
            if (outs[b].n && overlaps(outs[a].p, outs[a].n, outs[b].p, outs[b].n))
                return fail(VSA_ERR_ALIAS, "two outputs of the backward overlap");
    }
    if (!workspace) return fail(VSA_ERR_WORKSPACE, "workspace is NULL");
    if ((uintptr_t)workspace % kAlign) return fail(VSA_ERR_ALIGN, "workspace must be 256-byte aligned");
    const BwdWorkspace w = plan_bwd_workspace(P, workspace);
    if (workspace_bytes < w.total_bytes)
        return fail(VSA_ERR_WORKSPACE, "workspace holds %zu bytes, needs %zu", workspace_bytes, w.total_bytes);
    // the forward's block means: Qc, Kc, Vc at the start of its workspace
    Workspace fw{};
    if (use_forward) {
        if (!forward_workspace) return fail(VSA_ERR_WORKSPACE, "forward workspace is NULL");
        if ((uintptr_t)forward_workspace % kAlign)
            return fail(VSA_ERR_ALIGN, "forward workspace must be 256-byte aligned");
        fw = plan_workspace(P, const_cast<void*>(forward_workspace));
        if (forward_workspace_bytes < fw.coarse_bytes)
            return fail(VSA_ERR_WORKSPACE, "forward workspace holds %zu bytes, needs %zu", forward_workspace_bytes,
                        fw.coarse_bytes);
        const int64_t pooled_bytes = (const char*)fw.coarse - (const char*)forward_workspace;
        for (const Span& o : outs)
            if (o.n && overlaps(o.p, o.n, forward_workspace, pooled_bytes))
                return fail(VSA_ERR_ALIAS, "an output of the backward overlaps the forward workspace");
        if (overlaps(workspace, (int64_t)w.total_bytes, forward_workspace, pooled_bytes))
            return fail(VSA_ERR_ALIAS, "the backward workspace overlaps the forward workspace");
    }
    vsa::BwdArgs A{};
    A.q = q;
    A.k = k;
    A.v = v;
    A.dout = dout;
    A.out_s = out_s;
    A.gate = gate;
    A.out_c = out_c;
    A.lse = lse;
    A.idx = q2k_idx;
    A.num = q2k_num;
    A.gate_mode = gate_mode;
    A.gs0 = gs[0];
    A.gs1 = gs[1];
    A.gs2 = gs[2];
    A.dq = dq;
    A.dk = dk;
    A.dv = dv;
    A.dgate = dgate;
    A.qc = use_forward ? fw.qc : w.qc;
    A.kc = use_forward ? fw.kc : w.kc;
    A.vc = use_forward ? fw.vc : w.vc;
    A.pooled = use_forward;
    A.doc = w.doc;
    A.dqc = w.dqc;
    A.dkc = w.dkc;
    A.dvc = w.dvc;
    A.pbuf = w.pbuf;
    A.dsbuf = w.dsbuf;
    A.rs = w.rs;
    A.k2q = w.k2q;
    A.k2q_num = w.k2q_num;
    rc = hip_status(vsa::launch_backward(P, A, (hipStream_t)stream), "backward launch");
    return rc ? rc : ok();
}

int vsa_backward(const vsa_problem* problem, const vsa_bf16* q, const vsa_bf16* k, const vsa_bf16* v,
                 const int32_t* q2k_idx, const int32_t* q2k_num, const float* out_c, const vsa_bf16* gate,
                 int32_t gate_mode, const int64_t* gate_strides_in, const vsa_bf16* out_s, const float* lse,
                 const vsa_bf16* dout, vsa_bf16* dq, vsa_bf16* dk, vsa_bf16* dv, vsa_bf16* dgate, void* workspace,
                 size_t workspace_bytes, vsa_stream stream) {
    return backward_common(problem, q, k, v, q2k_idx, q2k_num, out_c, gate, gate_mode, gate_strides_in, out_s, lse,
                           dout, dq, dk, dv, dgate, workspace, workspace_bytes, nullptr, 0, false, stream);
}

int vsa_backward_pooled(const vsa_problem* problem, const vsa_bf16* q, const vsa_bf16* k, const vsa_bf16* v,
                        const int32_t* q2k_idx, const int32_t* q2k_num, const float* out_c, const vsa_bf16* gate,
                        int32_t gate_mode, const int64_t* gate_strides_in, const vsa_bf16* out_s, const float* lse,
                        const vsa_bf16* dout, vsa_bf16* dq, vsa_bf16* dk, vsa_bf16* dv, vsa_bf16* dgate,
                        const void* forward_workspace, size_t forward_workspace_bytes, void* workspace,
                        size_t workspace_bytes, vsa_stream stream) {
    return backward_common(problem, q, k, v, q2k_idx, q2k_num, out_c, gate, gate_mode, gate_strides_in, out_s, lse,
                           dout, dq, dk, dv, dgate, workspace, workspace_bytes, forward_workspace,
                           forward_workspace_bytes, true, stream);
}

int vsa_combine(const vsa_problem* problem, const float* out_c, const vsa_bf16* gate, int32_t gate_mode,
                const int64_t* gate_strides_in, vsa_bf16* out, vsa_stream stream) {
    vsa::DevProblem P;
    int rc = make_problem(problem, &P);
    if (rc) return rc;
    if (!out_c || !out) return fail(VSA_ERR_NULL, "out_c or out is NULL");
    if (!aligned16(out_c) || !aligned16(out)) return fail(VSA_ERR_ALIGN, "out_c and out must be 16-byte aligned");
    int64_t gs[3];
    if ((rc = gate_strides(P, gate, gate_mode, gate_strides_in, gs))) return rc;
    if (gate_mode != VSA_GATE_NONE) {
        const int64_t ob = 2 * q_elems(P);
        if (overlaps(out, ob, gate, 2)) return fail(VSA_ERR_ALIAS, "gate overlaps out");
    }
    rc = hip_status(vsa::launch_combine(P, out_c, gate, gate_mode, gs[0], gs[1], gs[2], out, (hipStream_t)stream),
                    "combine launch");
    return rc ? rc : ok();
}

static int forward_common(const vsa_problem* pr, const vsa_bf16* q, const vsa_bf16* k, const vsa_bf16* v,
                          const vsa_bf16* gate, int32_t gate_mode, const int64_t* gate_strides_in,
                          vsa_bf16* out, int32_t* q2k_idx, int32_t* q2k_num, float* out_c,
                          void* workspace, size_t workspace_bytes, vsa_stream stream) {
    vsa::DevProblem P;
    int rc = make_problem(pr, &P);
    if (rc) return rc;
    if ((rc = check_qkv(P, q, k, v))) return rc;
    if (!out) return fail(VSA_ERR_NULL, "out is NULL");
    if (!aligned16(out)) return fail(VSA_ERR_ALIGN, "out must be 16-byte aligned");
    if ((rc = check_out_alias(P, out, q, k, v))) return rc;
    int64_t gs[3];
    if ((rc = gate_strides(P, gate, gate_mode, gate_strides_in, gs))) return rc;
    if (gate_mode != VSA_GATE_NONE && overlaps(out, 2 * q_elems(P), gate, 2))
        return fail(VSA_ERR_ALIAS, "gate overlaps out");
    if (out_c && !aligned16(out_c)) return fail(VSA_ERR_ALIGN, "out_c must be 16-byte aligned");
    if ((q2k_idx && ((uintptr_t)q2k_idx & 3u)) || (q2k_num && ((uintptr_t)q2k_num & 3u)))
        return fail(VSA_ERR_ALIGN, "index arrays must be 4-byte aligned");
    if (!workspace) return fail(VSA_ERR_WORKSPACE, "workspace is NULL");
    if ((uintptr_t)workspace % kAlign) return fail(VSA_ERR_ALIGN, "workspace must be 256-byte aligned");
    const Workspace w = plan_workspace(P, workspace);
    if (workspace_bytes < w.total_bytes)
        return fail(VSA_ERR_WORKSPACE, "workspace holds %zu bytes, needs %zu", workspace_bytes, w.total_bytes);
    float* oc = out_c ? out_c : w.out_c;
    int* idx = q2k_idx ? q2k_idx : w.idx;
    int* num = q2k_num ? q2k_num : w.num;
    hipStream_t st = (hipStream_t)stream;
    if ((rc = run_coarse(P, q, k, v, oc, idx, num, w, st))) return rc;
    if ((rc = hip_status(vsa::launch_sparse_attn_combine(P, q, k, v, idx, num, oc, gate, gate_mode, gs[0], gs[1],
                                                         gs[2], out, nullptr, nullptr, st),
                         "fused sparse attention launch")))
        return rc;
    return ok();
}

int vsa_forward(const vsa_bf16* q, const vsa_bf16* k, const vsa_bf16* v, const vsa_bf16* gate,
                int32_t gate_mode, const int64_t* gate_strides, vsa_bf16* out, int32_t* q2k_idx,
                int32_t* q2k_num, float* out_c, int32_t batch, int32_t heads, int32_t seqlen_q,
                int32_t seqlen_kv, int32_t head_dim, int32_t block_size, int32_t topk, void* workspace,
                size_t workspace_bytes, vsa_stream stream) {
    vsa_problem pr{};
    pr.layout = VSA_LAYOUT_DENSE;
    pr.heads = heads;
    pr.head_dim = head_dim;
    pr.block_size = block_size;
    pr.batch = batch;
    pr.seqlen_q = seqlen_q;
    pr.seqlen_kv = seqlen_kv;
    pr.topk = topk;
    return forward_common(&pr, q, k, v, gate, gate_mode, gate_strides, out, q2k_idx, q2k_num, out_c, workspace,
                          workspace_bytes, stream);
}

size_t vsa_noalloc_scratch_bytes(void) { return kNoAllocScratchBytes; }

int vsa_forward_noalloc(const vsa_bf16* q, const vsa_bf16* k, const vsa_bf16* v, const vsa_bf16* gate,
                        int32_t gate_mode, const int64_t* gate_strides, vsa_bf16* out, int32_t* q2k_idx,
                        int32_t* q2k_num, float* out_c, int32_t batch, int32_t heads, int32_t seqlen_q,
                        int32_t seqlen_kv, int32_t head_dim, int32_t block_size, int32_t topk,
                        vsa_stream stream) {
    vsa_problem pr{};
    pr.layout = VSA_LAYOUT_DENSE;
    pr.heads = heads;
    pr.head_dim = head_dim;
    pr.block_size = block_size;
    pr.batch = batch;
    pr.seqlen_q = seqlen_q;
    pr.seqlen_kv = seqlen_kv;
    pr.topk = topk;
    // the size check comes first: a problem past the array is rejected
    // before any device is touched
    vsa::DevProblem P;
    int rc = make_problem(&pr, &P);
    if (rc) return rc;
    const size_t need = plan_workspace(P, nullptr).total_bytes;
    if (need > kNoAllocScratchBytes)
        return fail(VSA_ERR_WORKSPACE, "problem needs %zu bytes of scratch, vsa_forward_noalloc has %zu", need,
                    kNoAllocScratchBytes);
    void* ws = nullptr;
    if ((rc = scratch_address(&ws))) return rc;
    // the forward writes every scratch value before reading it (pooled
    // blocks, scores, routing), so nothing needs clearing between calls
    return forward_common(&pr, q, k, v, gate, gate_mode, gate_strides, out, q2k_idx, q2k_num, out_c, ws,
                          kNoAllocScratchBytes, stream);
}

int vsa_forward_bshd(const vsa_bf16* q, const vsa_bf16* k, const vsa_bf16* v, const vsa_bf16* gate,
                     int32_t gate_mode, const int64_t* gate_strides, vsa_bf16* out, int32_t* q2k_idx,
                     int32_t* q2k_num, float* out_c, int32_t batch, int32_t heads, int32_t seqlen_q,
                     int32_t seqlen_kv, int32_t head_dim, int32_t block_size, int32_t topk, void* workspace,
                     size_t workspace_bytes, vsa_stream stream) {
    vsa_problem pr{};
    pr.layout = VSA_LAYOUT_BSHD;
    pr.heads = heads;
    pr.head_dim = head_dim;
    pr.block_size = block_size;
    pr.batch = batch;
    pr.seqlen_q = seqlen_q;
    pr.seqlen_kv = seqlen_kv;
    pr.topk = topk;
    return forward_common(&pr, q, k, v, gate, gate_mode, gate_strides, out, q2k_idx, q2k_num, out_c, workspace,
                          workspace_bytes, stream);
}

int vsa_forward_varlen(const vsa_bf16* q, const vsa_bf16* k, const vsa_bf16* v, const vsa_bf16* gate,
                       int32_t gate_mode, const int64_t* gate_strides, vsa_bf16* out, int32_t* q2k_idx,
                       int32_t* q2k_num, float* out_c, const int32_t* cu_blocks_q, const int32_t* cu_blocks_kv,
                       const int32_t* block_sizes_q, const int32_t* block_sizes_kv,
                       const int32_t* topk_per_seq, int32_t num_seqs, int32_t total_q_blocks,
                       int32_t total_kv_blocks, int32_t max_q_blocks, int32_t max_kv_blocks, int32_t max_topk,
                       int32_t heads, int32_t head_dim, int32_t block_size, void* workspace,
                       size_t workspace_bytes, vsa_stream stream) {
    vsa_problem pr{};
    pr.layout = VSA_LAYOUT_PACKED;
    pr.heads = heads;
    pr.head_dim = head_dim;
    pr.block_size = block_size;
    pr.num_seqs = num_seqs;
    pr.total_q_blocks = total_q_blocks;
    pr.total_kv_blocks = total_kv_blocks;
    pr.max_q_blocks = max_q_blocks;
    pr.max_kv_blocks = max_kv_blocks;
    pr.max_topk = max_topk;
    pr.cu_blocks_q = cu_blocks_q;
    pr.cu_blocks_kv = cu_blocks_kv;
    pr.block_sizes_q = block_sizes_q;
    pr.block_sizes_kv = block_sizes_kv;
    pr.topk_per_seq = topk_per_seq;
    return forward_common(&pr, q, k, v, gate, gate_mode, gate_strides, out, q2k_idx, q2k_num, out_c, workspace,
                          workspace_bytes, stream);
}

int vsa_tile_partition(int32_t T, int32_t H, int32_t W, int32_t tile_t, int32_t tile_h, int32_t tile_w,
                       int32_t* num_tiles, int32_t* tile_sizes, int64_t* tile_partition_indices,
                       int64_t* reverse_tile_partition_indices, int64_t* non_pad_index) {
    if (!num_tiles) return fail(VSA_ERR_NULL, "num_tiles is NULL");
    *num_tiles = 0;
    vsa::TileGrid g;
    int rc = check_tiles(T, H, W, tile_t, tile_h, tile_w, &g);
    if (rc) return rc;
    *num_tiles = g.ntiles;
    int64_t p = 0;
    for (int b = 0; b < g.ntiles; ++b) {
        int et, eh, ew;
        const int n = vsa::tile_extents(g, b, et, eh, ew);
        if (tile_sizes) tile_sizes[b] = n;
        for (int u = 0; u < n; ++u, ++p) {
            const int64_t r = vsa::tile_token_raster(g, b, u, eh, ew);
            if (tile_partition_indices) tile_partition_indices[p] = r;
            if (reverse_tile_partition_indices) reverse_tile_partition_indices[r] = p;
            if (non_pad_index) non_pad_index[p] = (int64_t)g.blk * b + u;
        }
    }
    return ok();
}

int vsa_build_tile_metadata(int32_t num_videos, int32_t T, int32_t H, int32_t W, int32_t tile_t, int32_t tile_h,
                            int32_t tile_w, int32_t topk, vsa_meta_sizes* sizes, int32_t* cu_blocks_q,
                            int32_t* cu_blocks_kv, int32_t* block_sizes_q, int32_t* block_sizes_kv,
                            int32_t* topk_clamped) {
    if (!sizes) return fail(VSA_ERR_NULL, "sizes is NULL");
    *sizes = vsa_meta_sizes{};
    vsa::TileGrid g;
    int rc = check_tiles(T, H, W, tile_t, tile_h, tile_w, &g);
    if (rc) return rc;
    if (num_videos < 1) return fail(VSA_ERR_SHAPE, "empty batch (num_videos=%d)", num_videos);
    if (topk < 1) return fail(VSA_ERR_TOPK, "topk must be >= 1 (got %d)", topk);
    if (g.ntiles > vsa::kMaxKvBlocks)
        return fail(VSA_ERR_UNSUPPORTED, "%d tiles per video exceeds %d", g.ntiles, vsa::kMaxKvBlocks);
    const int nout = !!cu_blocks_q + !!cu_blocks_kv + !!block_sizes_q + !!block_sizes_kv + !!topk_clamped;
    if (nout != 0 && nout != 5) return fail(VSA_ERR_NULL, "pass all five output arrays or none");
    const int64_t total = (int64_t)num_videos * g.ntiles;
    if (total * g.blk > 0x7fffffffLL) return fail(VSA_ERR_SHAPE, "packed length exceeds 2^31 slots");
    const int32_t kk = std::min(topk, g.ntiles);
    sizes->num_seqs = num_videos;
    sizes->total_q_blocks = (int32_t)total;
    sizes->total_kv_blocks = (int32_t)total;
    sizes->max_q_blocks = g.ntiles;
    sizes->max_kv_blocks = g.ntiles;
    sizes->max_topk = kk;
    sizes->q_slots = total * g.blk;
    sizes->kv_slots = total * g.blk;
    if (nout == 0) return ok();
    for (int s = 0; s <= num_videos; ++s) cu_blocks_q[s] = cu_blocks_kv[s] = s * g.ntiles;
    for (int s = 0; s < num_videos; ++s) {
        topk_clamped[s] = kk;
        for (int b = 0; b < g.ntiles; ++b) {
            int et, eh, ew;
            block_sizes_q[s * g.ntiles + b] = block_sizes_kv[s * g.ntiles + b] = vsa::tile_extents(g, b, et, eh, ew);
        }
    }
    return ok();
}

int vsa_tile_gather(const vsa_bf16* x, vsa_bf16* y, int32_t batch, int32_t heads, int32_t T, int32_t H,
                    int32_t W, int32_t tile_t, int32_t tile_h, int32_t tile_w, int32_t elems, vsa_stream stream) {
    return tile_copy(x, y, batch, heads, T, H, W, tile_t, tile_h, tile_w, elems, false, stream);
}

int vsa_tile_scatter(const vsa_bf16* y, vsa_bf16* x, int32_t batch, int32_t heads, int32_t T, int32_t H,
                     int32_t W, int32_t tile_t, int32_t tile_h, int32_t tile_w, int32_t elems, vsa_stream stream) {
    return tile_copy(y, x, batch, heads, T, H, W, tile_t, tile_h, tile_w, elems, true, stream);
}

}  // extern "C"
