// C ABI of libflowcache: argument checks, workspace layout and the launch
// sequence of each entry point.  Declarations and the contract live in
// include/flowcache.h.
#include <math.h>

#include <atomic>

#include "../../include/flowcache.h"
#include "common.hpp"
#include "kernels.hpp"

namespace {

using namespace fc;

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// A usable workspace: present, large enough, and 256-byte aligned (every
// buffer carved from it sits at a 256-byte offset).
bool ws_ok(const void* ws, size_t bytes, size_t need) {
    return ws != nullptr && (reinterpret_cast<uintptr_t>(ws) & (kAlign - 1)) == 0 && bytes >= need;
}

// ---- KV compression -------------------------------------------------------------------
struct KvLayout {
    ImpPlan plan;
    int nbu, nbr;
    int nkb;  // importance pass-2 workgroups per head (redundancy softmax partials of the fused path)
    bool fits;  // every launch of the plan fits a dispatch
    size_t part, nlse2, imp, r, u_part, u, red_part, keys, queue, total;
};

fc_status check_kv(const fc_kv_params* p) {
    if (p == nullptr) return FC_ERR_INVALID_ARG;
    if (p->H < 1 || p->d < 1 || p->L_q < 1 || p->L_k < 1 || p->B_budget < 1) return FC_ERR_INVALID_ARG;
    if (!(p->lambda >= 0.0f && p->lambda <= 1.0f)) return FC_ERR_INVALID_ARG;
    if (p->pool_window < 1 || p->pool_window % 2 == 0 || p->pool_window > 129) return FC_ERR_INVALID_ARG;
    if (!(p->softmax_scale >= 0.0f) || isinf(p->softmax_scale)) return FC_ERR_INVALID_ARG;
    if (p->dtype != FC_F32 && p->dtype != FC_BF16) return FC_ERR_UNSUPPORTED;
    if (p->d != 64 && p->d != 128) return FC_ERR_UNSUPPORTED;
    if (p->H > 65535) return FC_ERR_UNSUPPORTED;
    // one head's Q or K rows are addressed with 32-bit byte offsets
    const long long esize = p->dtype == FC_BF16 ? 2 : 4;
    if ((long long)p->L_q * p->d * esize >= (1LL << 31) || (long long)p->L_k * p->d * esize >= (1LL << 31))
        return FC_ERR_UNSUPPORTED;
    return FC_OK;
}

KvLayout kv_layout(const fc_kv_params* p) {
    KvLayout L{};
    const int dt = p->dtype == FC_BF16 ? kBF16 : kF32;
    L.plan = imp_plan(p->H, p->L_q, p->L_k, dt, p->d);
    L.nbu = red_nbu(p->L_k);
    L.nbr = red_nbr(p->L_k);
    L.nkb = imp_colsum_blocks(p->L_k);
    L.fits = imp_grids_fit(p->H, p->L_q, p->L_k, L.plan, L.nbu) && sel_grid_fits(p->H, p->L_k);
    const size_t H = (size_t)p->H, Lk = (size_t)p->L_k;
    size_t o = 0;
    L.part = o;     o = align_up(o + H * L.plan.nsplit * (size_t)p->L_q * sizeof(float2));
    L.nlse2 = o;    o = align_up(o + H * (size_t)imp_lq_pad(p->L_q) * sizeof(float));
    L.imp = o;      o = align_up(o + (size_t)L.plan.nqs * H * Lk * sizeof(float));  // importance planes
    L.r = o;        o = align_up(o + H * Lk * sizeof(float));
    L.u_part = o;   o = align_up(o + H * L.nbu * (size_t)p->d * sizeof(float));
    L.u = o;        o = align_up(o + H * (size_t)p->d * sizeof(float));
    L.red_part = o; o = align_up(o + H * (size_t)(L.nbr > L.nkb ? L.nbr : L.nkb) * sizeof(float2));
    L.keys = o;     o = align_up(o + sel_ws_bytes(p->H, p->L_k));  // selection: keys, histograms, counts
    L.queue = o;    o = align_up(o + kImpQueueWords * sizeof(uint32_t));  // persistent passes' counters
    L.total = o;
    return L;
}

template <typename T>
T* at(void* ws, size_t off) { return reinterpret_cast<T*>(static_cast<char*>(ws) + off); }

float log2_scale(const fc_kv_params* p) {
    const float scale = p->softmax_scale > 0.0f ? p->softmax_scale : 1.0f / sqrtf((float)p->d);
    return scale * kLog2e;
}

fc_status hip_status(hipError_t e) { return e == hipSuccess ? FC_OK : FC_ERR_HIP; }

#define FC_TRY(expr)                                 \
    do {                                             \
        hipError_t e_ = (expr);                      \
        if (e_ != hipSuccess) return FC_ERR_HIP;     \
    } while (0)

// Importance (two passes) into the workspace's importance planes; with
// imp_out they are also added up into imp_out [H][Lk].  With `r` the pass-1
// launch also runs redundancy pass A (partials of u in the workspace), and
// the second pass produces the redundancy of the keys it holds and the
// softmax partials of r, one per key block.
fc_status run_importance(const fc_kv_params* p, const KvLayout& L, const void* Q, const void* K, float* imp_out,
                         void* ws, hipStream_t s, float* r = nullptr, int ldk = 0) {
    const int dt = p->dtype == FC_BF16 ? kBF16 : kF32;
    const float c = log2_scale(p);
    float2* part = at<float2>(ws, L.part);
    float* nlse2 = at<float>(ws, L.nlse2);
    // one plane goes straight to imp_out when the caller wants importance
    float* planes = (imp_out && L.plan.nqs == 1) ? imp_out : at<float>(ws, L.imp);
    float* u = r ? at<float>(ws, L.u) : nullptr;
    uint32_t* queue = at<uint32_t>(ws, L.queue);
    if (L.plan.persistent_lse || L.plan.persistent_colsum) FC_TRY(launch_imp_queue_zero(queue, s));
    // with r, redundancy pass A runs inside the pass-1 launch
    FC_TRY(launch_imp_lse(dt, p->d, Q, K, part, p->H, p->L_q, p->L_k, L.plan, c, s,
                          r ? at<float>(ws, L.u_part) : nullptr, L.nbu, queue, ldk));
    FC_TRY(launch_imp_lse_merge(part, nullptr, nlse2, p->H, p->L_q, L.plan.nsplit, s,
                                r ? at<float>(ws, L.u_part) : nullptr, L.nbu, u, p->d));
    FC_TRY(launch_imp_colsum(dt, p->d, Q, K, nlse2, planes, p->H, p->L_q, p->L_k, L.plan, c, s, u, r,
                             r ? at<float2>(ws, L.red_part) : nullptr, queue + 8, ldk));
    if (imp_out && planes != imp_out) FC_TRY(launch_imp_sum_planes(planes, imp_out, p->H, p->L_k, L.plan.nqs, s));
    return FC_OK;
}

// The whole compression of K, V [H][L_k][d] into K_out, V_out [H][B'][d]
// (arguments already checked).  With pos_out the positions pos [H][L_k]
// follow the kept rows.  Head strides in rows: ld_in for K, V and pos, ld_out
// for K_out, V_out and pos_out (0: dense, L_k and B').
fc_status kv_compress_run(const fc_kv_params* p, const KvLayout& L, const void* Q, const void* K, const void* V,
                          void* K_out, void* V_out, int32_t* idx_out, float* score_out, float* imp_pooled_out,
                          float* red_out, void* ws, hipStream_t s, const int32_t* pos = nullptr,
                          int32_t* pos_out = nullptr, int ld_in = 0, int ld_out = 0) {
    const int dt = p->dtype == FC_BF16 ? kBF16 : kF32;
    const int Bp = p->B_budget < p->L_k ? p->B_budget : p->L_k;
    if (Bp == p->L_k && !score_out && !imp_pooled_out && !red_out) {
        // every token is kept and no score is asked for: the rows are copied
        FC_TRY(launch_gather(dt, p->d, nullptr, p->H, p->L_k, Bp, K, V, K_out, V_out, s, pos, pos_out, idx_out, ld_in,
                             ld_out));
        return FC_OK;
    }
    float* imp = at<float>(ws, L.imp);
    float* r = at<float>(ws, L.r);
    float2* red_part = at<float2>(ws, L.red_part);
    // importance (planes in the workspace): its first launch also runs
    // redundancy pass A, its second pass forms r and the softmax partials of r
    const fc_status st = run_importance(p, L, Q, K, nullptr, ws, s, r, ld_in);
    if (st != FC_OK) return st;
    // pool + score + top-B + gather
    FC_TRY(launch_sel_head(imp, L.plan.nqs, r, red_part, L.nkb, p->lambda, p->pool_window, score_out, imp_pooled_out,
                           red_out, at<uint32_t>(ws, L.keys), p->H, p->L_k, Bp, idx_out, s));
    FC_TRY(launch_gather(dt, p->d, idx_out, p->H, p->L_k, Bp, K, V, K_out, V_out, s, pos, pos_out, nullptr, ld_in,
                         ld_out));
    return FC_OK;
}

// ---- KV cache manager ----------------------------------------------------------------------
fc_status check_cache(const fc_cache_params* c) {
    if (c == nullptr) return FC_ERR_INVALID_ARG;
    if (c->H < 1 || c->d < 1 || c->B_budget < 1 || c->B_active < 1) return FC_ERR_INVALID_ARG;
    if ((long long)c->B_budget + c->B_active > 0x7fffffffLL) return FC_ERR_UNSUPPORTED;
    return FC_OK;
}

// Compression parameters of a commit that merges L tokens.
fc_kv_params cache_kv_params(const fc_cache_params* c, int32_t L_q, int32_t L) {
    fc_kv_params p{};
    p.H = c->H;
    p.d = c->d;
    p.L_q = L_q;
    p.L_k = L;
    p.B_budget = c->B_budget;
    p.lambda = c->lambda;
    p.pool_window = c->pool_window;
    p.softmax_scale = c->softmax_scale;
    p.dtype = c->dtype;
    return p;
}

// Workspace of a compressing commit: the kept indices, then the
// compression's own workspace.
struct CacheLayout {
    size_t idx, comp;
};
CacheLayout cache_layout(const fc_cache_params* c) {
    CacheLayout L{};
    L.idx = 0;
    L.comp = align_up((size_t)c->H * (size_t)c->B_budget * sizeof(int32_t));
    return L;
}

// ---- chunk L1 ------------------------------------------------------------------------------
fc_status chunk_table(const fc_l1_params* p, const int64_t* off, ChunkTable* tab) {
    if (p == nullptr || off == nullptr) return FC_ERR_INVALID_ARG;
    if (p->n_chunks < 1) return FC_ERR_INVALID_ARG;
    if (p->n_chunks > FC_MAX_CHUNKS || p->n_chunks > kMaxChunks) return FC_ERR_UNSUPPORTED;
    if (p->dtype != FC_F32 && p->dtype != FC_BF16) return FC_ERR_UNSUPPORTED;
    if (p->m < 0 || !(p->eps >= 0.0f)) return FC_ERR_INVALID_ARG;
    if (off[0] < 0) return FC_ERR_INVALID_ARG;
    const int dt = p->dtype == FC_BF16 ? kBF16 : kF32;
    tab->n = p->n_chunks;
    long long blocks = 0;
    for (int i = 0; i < p->n_chunks; ++i) {
        if (off[i + 1] < off[i]) return FC_ERR_INVALID_ARG;
        tab->off[i] = off[i];
        tab->blk_start[i] = (int32_t)blocks;
        blocks += chunk_blocks_for(off[i + 1] - off[i], dt);
        if (blocks > 0xffffffffLL / 256) return FC_ERR_UNSUPPORTED;  // the slab grid's work-items fit 32 bits
    }
    tab->off[p->n_chunks] = off[p->n_chunks];
    tab->blk_start[p->n_chunks] = (int32_t)blocks;
    return FC_OK;
}

size_t chunk_ws_bytes(const ChunkTable& tab) { return align_up((size_t)tab.blk_start[tab.n] * sizeof(float2)); }

// ---- allocation-free chunk decision ---------------------------------------------------------
// The slab partials of fc_chunk_rel_l1_decide_noalloc live in this array, one
// copy per device, held until the process ends.  Host code never passes the
// array's name to a kernel (on the host it is only a stand-in for the
// symbol): the device address comes from hipGetSymbolAddress, looked up once
// per device with that device current.
constexpr size_t kNoAllocScratchBytes = FC_NOALLOC_SCRATCH_BYTES;
__device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

constexpr int kMaxScratchDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxScratchDevices];

// The device address of this device's scratch array (nullptr on failure).
void* scratch_ptr() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxScratchDevices) return nullptr;
    void* ptr = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (ptr == nullptr) {
        // two threads racing here look up the same address; either store wins
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) return nullptr;
        g_scratch_ptr[dev].store(ptr, std::memory_order_release);
    }
    return ptr;
}

}  // namespace

extern "C" {

const char* fc_status_string(fc_status s) {
    switch (s) {
        case FC_OK: return "ok";
        case FC_ERR_INVALID_ARG: return "invalid argument";
        case FC_ERR_UNSUPPORTED: return "unsupported configuration";
        case FC_ERR_WORKSPACE: return "workspace missing or too small";
        case FC_ERR_HIP: return "HIP launch failed";
        default: break;
    }
    return "unknown status";
}

size_t fc_kv_compress_workspace_bytes(const fc_kv_params* p) {
    if (check_kv(p) != FC_OK) return 0;
    const KvLayout L = kv_layout(p);
    return L.fits ? L.total : 0;
}

fc_status fc_kv_compress(const fc_kv_params* p, const void* Q, const void* K, const void* V, void* K_out,
                         void* V_out, int32_t* idx_out, float* score_out, float* imp_pooled_out, float* red_out,
                         void* workspace, size_t workspace_bytes, void* stream) {
    fc_status st = check_kv(p);
    if (st != FC_OK) return st;
    if (!Q || !K || !V || !K_out || !V_out || !idx_out) return FC_ERR_INVALID_ARG;
    if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(K_out) || !aligned16(V_out))
        return FC_ERR_INVALID_ARG;
    const KvLayout L = kv_layout(p);
    if (!L.fits) return FC_ERR_UNSUPPORTED;
    if (!ws_ok(workspace, workspace_bytes, L.total)) return FC_ERR_WORKSPACE;
    return kv_compress_run(p, L, Q, K, V, K_out, V_out, idx_out, score_out, imp_pooled_out, red_out, workspace,
                           static_cast<hipStream_t>(stream));
}

fc_status fc_kv_importance(const fc_kv_params* p, const void* Q, const void* K, float* imp_out, void* workspace,
                           size_t workspace_bytes, void* stream) {
    fc_status st = check_kv(p);
    if (st != FC_OK) return st;
    if (!Q || !K || !imp_out || !aligned16(Q) || !aligned16(K)) return FC_ERR_INVALID_ARG;
    const KvLayout L = kv_layout(p);
    if (!L.fits) return FC_ERR_UNSUPPORTED;
    if (!ws_ok(workspace, workspace_bytes, L.total)) return FC_ERR_WORKSPACE;
    return run_importance(p, L, Q, K, imp_out, workspace, static_cast<hipStream_t>(stream));
}

fc_status fc_kv_importance_redundancy(const fc_kv_params* p, const void* Q, const void* K, float* imp_out,
                                      float* r_out, void* workspace, size_t workspace_bytes, void* stream) {
    fc_status st = check_kv(p);
    if (st != FC_OK) return st;
    if (!Q || !K || !imp_out || !r_out || !aligned16(Q) || !aligned16(K)) return FC_ERR_INVALID_ARG;
    const KvLayout L = kv_layout(p);
    if (!L.fits) return FC_ERR_UNSUPPORTED;
    if (!ws_ok(workspace, workspace_bytes, L.total)) return FC_ERR_WORKSPACE;
    // the launches of fc_kv_compress's first half, into the caller's arrays
    return run_importance(p, L, Q, K, imp_out, workspace, static_cast<hipStream_t>(stream), r_out);
}

fc_status fc_kv_importance_lse(const fc_kv_params* p, const void* Q, const void* K, float* lse_out, void* workspace,
                               size_t workspace_bytes, void* stream) {
    fc_status st = check_kv(p);
    if (st != FC_OK) return st;
    if (!Q || !K || !lse_out || !aligned16(Q) || !aligned16(K)) return FC_ERR_INVALID_ARG;
    const KvLayout L = kv_layout(p);
    if (!L.fits) return FC_ERR_UNSUPPORTED;
    if (!ws_ok(workspace, workspace_bytes, L.total)) return FC_ERR_WORKSPACE;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int dt = p->dtype == FC_BF16 ? kBF16 : kF32;
    float2* part = at<float2>(workspace, L.part);
    uint32_t* queue = at<uint32_t>(workspace, L.queue);
    if (L.plan.persistent_lse) FC_TRY(launch_imp_queue_zero(queue, s));
    FC_TRY(launch_imp_lse(dt, p->d, Q, K, part, p->H, p->L_q, p->L_k, L.plan, log2_scale(p), s, nullptr, 0, queue));
    FC_TRY(launch_imp_lse_merge(part, lse_out, nullptr, p->H, p->L_q, L.plan.nsplit, s));
    return FC_OK;
}

fc_status fc_kv_importance_colsum(const fc_kv_params* p, const void* Q, const void* K, const float* lse,
                                  float* imp_out, void* workspace, size_t workspace_bytes, void* stream) {
    fc_status st = check_kv(p);
    if (st != FC_OK) return st;
    if (!Q || !K || !lse || !imp_out || !aligned16(Q) || !aligned16(K)) return FC_ERR_INVALID_ARG;
    const KvLayout L = kv_layout(p);
    if (!L.fits) return FC_ERR_UNSUPPORTED;
    if (!ws_ok(workspace, workspace_bytes, L.total)) return FC_ERR_WORKSPACE;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int dt = p->dtype == FC_BF16 ? kBF16 : kF32;
    float* nlse2 = at<float>(workspace, L.nlse2);
    float* planes = L.plan.nqs == 1 ? imp_out : at<float>(workspace, L.imp);
    uint32_t* queue = at<uint32_t>(workspace, L.queue);
    if (L.plan.persistent_colsum) FC_TRY(launch_imp_queue_zero(queue, s));
    FC_TRY(launch_imp_nlse2(lse, nlse2, p->H, p->L_q, s));
    FC_TRY(launch_imp_colsum(dt, p->d, Q, K, nlse2, planes, p->H, p->L_q, p->L_k, L.plan, log2_scale(p), s, nullptr,
                             nullptr, nullptr, queue + 8));
    if (planes != imp_out) FC_TRY(launch_imp_sum_planes(planes, imp_out, p->H, p->L_k, L.plan.nqs, s));
    return FC_OK;
}

fc_status fc_kv_redundancy(const fc_kv_params* p, const void* K, float* r_out, void* workspace,
                           size_t workspace_bytes, void* stream) {
    fc_status st = check_kv(p);
    if (st != FC_OK) return st;
    if (!K || !r_out || !aligned16(K)) return FC_ERR_INVALID_ARG;
    const KvLayout L = kv_layout(p);
    if (!L.fits) return FC_ERR_UNSUPPORTED;
    if (!ws_ok(workspace, workspace_bytes, L.total)) return FC_ERR_WORKSPACE;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int dt = p->dtype == FC_BF16 ? kBF16 : kF32;
    FC_TRY(launch_red_norm_sum(dt, p->d, K, at<float>(workspace, L.u_part), p->H, p->L_k, s));
    FC_TRY(launch_red_dot(dt, p->d, K, at<float>(workspace, L.u_part), r_out, at<float2>(workspace, L.red_part),
                          p->H, p->L_k, s));
    return FC_OK;
}

fc_status fc_kv_select(const fc_kv_params* p, const float* imp, const float* r, const void* K, const void* V,
                       void* K_out, void* V_out, int32_t* idx_out, float* score_out, float* imp_pooled_out,
                       float* red_out, void* workspace, size_t workspace_bytes, void* stream) {
    fc_status st = check_kv(p);
    if (st != FC_OK) return st;
    if (!imp || !r || !idx_out) return FC_ERR_INVALID_ARG;
    const bool gather = K || V || K_out || V_out;
    if (gather && !(K && V && K_out && V_out)) return FC_ERR_INVALID_ARG;
    if (gather && (!aligned16(K) || !aligned16(V) || !aligned16(K_out) || !aligned16(V_out)))
        return FC_ERR_INVALID_ARG;
    const KvLayout L = kv_layout(p);
    if (!L.fits) return FC_ERR_UNSUPPORTED;
    if (!ws_ok(workspace, workspace_bytes, L.total)) return FC_ERR_WORKSPACE;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int dt = p->dtype == FC_BF16 ? kBF16 : kF32;
    const int Bp = p->B_budget < p->L_k ? p->B_budget : p->L_k;
    float2* red_part = at<float2>(workspace, L.red_part);
    FC_TRY(launch_red_stats(r, red_part, p->H, p->L_k, s));
    FC_TRY(launch_sel_head(imp, 1, r, red_part, L.nbr, p->lambda, p->pool_window, score_out, imp_pooled_out, red_out,
                           at<uint32_t>(workspace, L.keys), p->H, p->L_k, Bp, idx_out, s));
    if (gather) FC_TRY(launch_gather(dt, p->d, idx_out, p->H, p->L_k, Bp, K, V, K_out, V_out, s));
    return FC_OK;
}

size_t fc_topb_select_workspace_bytes(int32_t H, int32_t L) {
    if (H < 1 || L < 1 || H > 65535 || !sel_grid_fits(H, L)) return 0;
    return align_up(sel_ws_bytes(H, L));  // keys, histograms, counts
}

fc_status fc_topb_select(int32_t H, int32_t L, int32_t B, const float* scores, int32_t* idx_out, void* workspace,
                         size_t workspace_bytes, void* stream) {
    if (H < 1 || L < 1 || B < 1 || !scores || !idx_out) return FC_ERR_INVALID_ARG;
    if (H > 65535 || !sel_grid_fits(H, L)) return FC_ERR_UNSUPPORTED;
    const size_t need = fc_topb_select_workspace_bytes(H, L);
    if (!ws_ok(workspace, workspace_bytes, need)) return FC_ERR_WORKSPACE;
    const int Bp = B < L ? B : L;
    FC_TRY(launch_sel_head(scores, 1, nullptr, nullptr, 0, 0.f, 1, nullptr, nullptr, nullptr,
                           static_cast<uint32_t*>(workspace), H, L, Bp, idx_out, static_cast<hipStream_t>(stream)));
    return FC_OK;
}

size_t fc_cache_commit_workspace_bytes(const fc_cache_params* c, int32_t L_q) {
    if (check_cache(c) != FC_OK || L_q < 1) return 0;
    // the compression's workspace for every merged length B_budget < L <= B_total;
    // it changes with L only through whole tiles of keys (32 or 64 rows), so one
    // length per 32 rows and the largest length cover every case
    const int32_t lo = c->B_budget + 1, hi = c->B_budget + c->B_active;
    size_t comp = 0;
    for (long long L = lo;; L = (L / 32 + 1) * 32) {
        const int32_t Lk = (int32_t)(L < hi ? L : hi);
        const fc_kv_params p = cache_kv_params(c, L_q, Lk);
        if (check_kv(&p) != FC_OK) return 0;
        const KvLayout KL = kv_layout(&p);
        if (!KL.fits) return 0;
        const size_t t = KL.total;
        comp = t > comp ? t : comp;
        if (Lk >= hi) break;
    }
    return cache_layout(c).comp + comp;
}

fc_status fc_cache_commit(const fc_cache_params* c, int32_t* L_clean, const void* K_chunk, const void* V_chunk,
                          int32_t L_c, int32_t pos0, const void* Q, int32_t L_q, void* K_cur, void* V_cur,
                          int32_t* pos_cur, void* K_spare, void* V_spare, int32_t* pos_spare, int32_t* swapped,
                          void* workspace, size_t workspace_bytes, void* stream) {
    fc_status st = check_cache(c);
    if (st != FC_OK) return st;
    if (L_clean == nullptr || *L_clean < 0 || *L_clean > c->B_budget) return FC_ERR_INVALID_ARG;
    if (L_c < 1 || L_c > c->B_active || pos0 < 0 || (long long)pos0 + L_c - 1 > 0x7fffffffLL) return FC_ERR_INVALID_ARG;
    if (!K_cur || !V_cur || !aligned16(K_cur) || !aligned16(V_cur)) return FC_ERR_INVALID_ARG;
    if ((K_chunk == nullptr) != (V_chunk == nullptr)) return FC_ERR_INVALID_ARG;
    if (K_chunk && (!aligned16(K_chunk) || !aligned16(V_chunk))) return FC_ERR_INVALID_ARG;
    const int32_t n_old = *L_clean, L = n_old + L_c;
    const int32_t ld = c->B_budget + c->B_active;  // rows per head of either region
    // the compression's checks (head dim, dtype, lambda, window, scale, sizes)
    // apply to every commit, so that an invalid cache fails on its first call
    const fc_kv_params kp = cache_kv_params(c, L_q > 0 ? L_q : 1, L);
    st = check_kv(&kp);
    if (st != FC_OK) return st;
    const bool full = L > c->B_budget;
    if (full) {
        if (Q == nullptr || L_q < 1 || !aligned16(Q)) return FC_ERR_INVALID_ARG;
        if (!K_spare || !V_spare || !aligned16(K_spare) || !aligned16(V_spare)) return FC_ERR_INVALID_ARG;
        if ((pos_cur == nullptr) != (pos_spare == nullptr)) return FC_ERR_INVALID_ARG;
        // the compression cannot gather into the region it reads
        if (K_spare == K_cur || V_spare == V_cur || K_spare == V_cur || V_spare == K_cur ||
            (pos_spare != nullptr && pos_spare == pos_cur))
            return FC_ERR_INVALID_ARG;
    }
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int dt = c->dtype == FC_BF16 ? kBF16 : kF32;
    if (!full) {
        // not full: the chunk is kept as it is, behind the clean tokens
        FC_TRY(launch_cache_append(dt, c->d, c->H, K_chunk, V_chunk, L_c, pos0, K_cur, V_cur, pos_cur, ld, n_old, s));
        *L_clean = L;
        if (swapped) *swapped = 0;
        return FC_OK;
    }
    // full: the clean rows and the chunk behind them are one row range of the
    // current region; its top-B_budget tokens per head go to the spare region
    const CacheLayout CL = cache_layout(c);
    const KvLayout KL = kv_layout(&kp);
    if (!KL.fits) return FC_ERR_UNSUPPORTED;
    if (!ws_ok(workspace, workspace_bytes, CL.comp + KL.total)) return FC_ERR_WORKSPACE;
    FC_TRY(launch_cache_append(dt, c->d, c->H, K_chunk, V_chunk, L_c, pos0, K_cur, V_cur, pos_cur, ld, n_old, s));
    st = kv_compress_run(&kp, KL, Q, K_cur, V_cur, K_spare, V_spare, at<int32_t>(workspace, CL.idx), nullptr, nullptr,
                         nullptr, at<char>(workspace, CL.comp), s, pos_cur, pos_spare, ld, ld);
    if (st != FC_OK) return st;
    *L_clean = c->B_budget;
    if (swapped) *swapped = 1;
    return FC_OK;
}

size_t fc_chunk_rel_l1_workspace_bytes(const fc_l1_params* p, const int64_t* chunk_offsets) {
    ChunkTable tab;
    if (chunk_table(p, chunk_offsets, &tab) != FC_OK) return 0;
    return chunk_ws_bytes(tab);
}

fc_status fc_chunk_rel_l1_decide(const fc_l1_params* p, const int64_t* chunk_offsets, const void* X_t,
                                 const void* X_tm1, int32_t* step, float* f, uint8_t* recompute, float* l1_rel_out,
                                 void* workspace, size_t workspace_bytes, void* stream) {
    ChunkTable tab;
    fc_status st = chunk_table(p, chunk_offsets, &tab);
    if (st != FC_OK) return st;
    if (!X_t || !X_tm1 || !step || !f || !recompute) return FC_ERR_INVALID_ARG;
    if (!aligned16(X_t) || !aligned16(X_tm1)) return FC_ERR_INVALID_ARG;
    if (!ws_ok(workspace, workspace_bytes, chunk_ws_bytes(tab))) return FC_ERR_WORKSPACE;
    const int dt = p->dtype == FC_BF16 ? kBF16 : kF32;
    return hip_status(launch_chunk_l1(dt, tab, X_t, X_tm1, step, f, recompute, l1_rel_out,
                                      static_cast<float2*>(workspace), p->m, p->eps,
                                      static_cast<hipStream_t>(stream)));
}

fc_status fc_chunk_rel_l1_decide_noalloc(const fc_l1_params* p, const int64_t* chunk_offsets, const void* X_t,
                                         const void* X_tm1, int32_t* step, float* f, uint8_t* recompute,
                                         float* l1_rel_out, void* stream) {
    ChunkTable tab;
    fc_status st = chunk_table(p, chunk_offsets, &tab);
    if (st != FC_OK) return st;
    if (!X_t || !X_tm1 || !step || !f || !recompute) return FC_ERR_INVALID_ARG;
    if (!aligned16(X_t) || !aligned16(X_tm1)) return FC_ERR_INVALID_ARG;
    if (chunk_ws_bytes(tab) > kNoAllocScratchBytes) return FC_ERR_UNSUPPORTED;  // states beyond the scratch's slabs
    void* ptr = scratch_ptr();
    if (ptr == nullptr) return FC_ERR_HIP;
    const int dt = p->dtype == FC_BF16 ? kBF16 : kF32;
    // every slab partial is written before it is read: nothing to clear
    return hip_status(launch_chunk_l1(dt, tab, X_t, X_tm1, step, f, recompute, l1_rel_out, static_cast<float2*>(ptr),
                                      p->m, p->eps, static_cast<hipStream_t>(stream)));
}

fc_status fc_euler_step_l1_decide(const fc_l1_params* p, const int64_t* chunk_offsets, const void* X_t,
                                  const void* v, const float* dt, void* X_next, int32_t* step, float* f,
                                  uint8_t* recompute, float* l1_rel_out, void* workspace, size_t workspace_bytes,
                                  void* stream) {
    ChunkTable tab;
    fc_status st = chunk_table(p, chunk_offsets, &tab);
    if (st != FC_OK) return st;
    if (!X_t || !v || !dt || !X_next || !step || !f || !recompute) return FC_ERR_INVALID_ARG;
    if (!aligned16(X_t) || !aligned16(v) || !aligned16(X_next)) return FC_ERR_INVALID_ARG;
    if (!ws_ok(workspace, workspace_bytes, chunk_ws_bytes(tab))) return FC_ERR_WORKSPACE;
    const int dtp = p->dtype == FC_BF16 ? kBF16 : kF32;
    return hip_status(launch_chunk_l1(dtp, tab, X_t, v, step, f, recompute, l1_rel_out,
                                      static_cast<float2*>(workspace), p->m, p->eps,
                                      static_cast<hipStream_t>(stream), dt, X_next));
}

fc_status fc_uniform_rel_l1_decide(const fc_l1_params* p, const int64_t* chunk_offsets, const void* X_t,
                                   const void* X_tm1, const int32_t* chunk_step, int32_t* step, float* f,
                                   uint8_t* recompute, float* l1_rel_out, void* workspace, size_t workspace_bytes,
                                   void* stream) {
    ChunkTable tab;
    fc_status st = chunk_table(p, chunk_offsets, &tab);
    if (st != FC_OK) return st;
    if (!X_t || !X_tm1 || !chunk_step || !step || !f || !recompute) return FC_ERR_INVALID_ARG;
    if (!aligned16(X_t) || !aligned16(X_tm1)) return FC_ERR_INVALID_ARG;
    if (!ws_ok(workspace, workspace_bytes, chunk_ws_bytes(tab))) return FC_ERR_WORKSPACE;
    const int dt = p->dtype == FC_BF16 ? kBF16 : kF32;
    return hip_status(launch_chunk_l1(dt, tab, X_t, X_tm1, const_cast<int32_t*>(chunk_step), f, recompute,
                                      l1_rel_out, static_cast<float2*>(workspace), p->m, p->eps,
                                      static_cast<hipStream_t>(stream), nullptr, nullptr, kRuleUniform, step));
}

fc_status fc_history_rel_l1_decide(const fc_l1_params* p, const int64_t* segment_offsets, const void* h_prev,
                                   const void* h_cur, int32_t* step, float* acc, uint8_t* refresh,
                                   float* dev_out, void* workspace, size_t workspace_bytes, void* stream) {
    ChunkTable tab;
    fc_status st = chunk_table(p, segment_offsets, &tab);
    if (st != FC_OK) return st;
    if (!h_prev || !h_cur || !step || !acc || !refresh) return FC_ERR_INVALID_ARG;
    if (!aligned16(h_prev) || !aligned16(h_cur)) return FC_ERR_INVALID_ARG;
    if (!ws_ok(workspace, workspace_bytes, chunk_ws_bytes(tab))) return FC_ERR_WORKSPACE;
    const int dt = p->dtype == FC_BF16 ? kBF16 : kF32;
    // ||h_t - h_{t+1}||_1 / ||h_{t+1}||_1: the previous state takes the
    // denominator's place, the first argument of the slab pass
    return hip_status(launch_chunk_l1(dt, tab, h_prev, h_cur, step, acc, refresh, dev_out,
                                      static_cast<float2*>(workspace), p->m, p->eps,
                                      static_cast<hipStream_t>(stream), nullptr, nullptr, kRuleHistory));
}

}  // extern "C"
