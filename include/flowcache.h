/*
 * flowcache.h -- C ABI of libflowcache.so: the FlowCache per-step hot path on
 * AMD Instinct MI355X (gfx950).
 *
 * The method is described on the page "Flow Caching for Autoregressive Video
 * Generation" (papernotes.org ICLR 2026 digest), section 方法详解 / 关键设计
 * ("Key designs"):
 *   item 1  chunk relative L1 distance  L1_rel = ||X_{t-1} - X_t||_1 / ||X_t||_1;
 *   item 2  chunkwise adaptive caching: accumulator f, forced recompute for the
 *           first m steps, recompute-and-reset when f + L1_rel > eps, else reuse;
 *   item 3  joint importance-redundancy KV-cache compression:
 *           Imp~ = max-pool_1d( mean_i softmax_j(scale q_i.k_j) ),
 *           Red_j = softmax_j( (1/L_k) sum_{i != j} khat_i.khat_j ),
 *           Score_j = lambda Imp~_j - (1 - lambda) Red_j, and each head keeps
 *           its top-B tokens (flowchart under 整体框架: cache full -> score ->
 *           top-B per head; not full -> keep as is).
 *
 * Conventions for every entry point
 *   - Pointers named as device pointers must point to memory of the current
 *     HIP device; host pointers are read before the call returns.
 *   - The caller owns all memory.  The library never allocates or frees; any
 *     temporary storage is the caller's workspace, sized by the *_bytes query
 *     and 256-byte aligned (as every hipMalloc or torch allocation is).
 *   - Work is queued on `stream` (a hipStream_t; NULL = the default stream)
 *     and runs asynchronously.  Argument checks happen on the host, before
 *     anything is queued, and return an error code synchronously.
 *   - Outputs must not alias inputs.  Tensors are dense and row-contiguous.
 *   - Alignment: the base pointers of the row tensors (Q, K, V, K_out,
 *     V_out, K_chunk, V_chunk, K_cur, V_cur, K_spare, V_spare) and of the
 *     chunk states (X_t, X_tm1, v, X_next, h_prev, h_cur) must be 16-byte
 *     aligned (every hipMalloc or torch allocation is; a view that starts
 *     inside a row may not be).  Any other base is FC_ERR_INVALID_ARG.  Float and int32
 *     arrays (imp, r, lse, scores, idx, step, f, ...) need only their
 *     natural alignment.
 *   - Errors: FC_ERR_INVALID_ARG (null required pointer, sizes < 1, lambda not
 *     in [0,1], even pool window or one above 129, a row tensor or state not
 *     16-byte aligned, ...), FC_ERR_UNSUPPORTED (head dim not 64 or
 *     128, unknown dtype, more than 65535 heads, one head's Q or K rows at
 *     2 GiB or more, launch grids beyond a dispatch's 32-bit work-item
 *     count, too many chunks), FC_ERR_WORKSPACE (workspace null,
 *     not 256-byte aligned or smaller than the query), FC_ERR_HIP (a launch
 *     failed).  No exception crosses the ABI.  NaN/Inf inputs are not
 *     supported.
 *   - The library keeps no state between calls (apart from a per-device
 *     cache of the importance kernels' occupancy, filled on first use, and
 *     the device scratch array of fc_chunk_rel_l1_decide_noalloc); calls on
 *     different streams with different workspaces may run concurrently.
 */
#ifndef FLOWCACHE_H
#define FLOWCACHE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Both enums carry a last enumerator of 0x7fffffff, so that any int value a
 * C caller passes is a valid value of the type on the C++ side as well
 * (such values are answered as unknown or unsupported). */
typedef enum {
    FC_OK = 0,
    FC_ERR_INVALID_ARG = 1,
    FC_ERR_UNSUPPORTED = 2,
    FC_ERR_WORKSPACE = 3,
    FC_ERR_HIP = 4,
    FC_STATUS_MAX_ENUM = 0x7fffffff
} fc_status;

/* Static, NUL-terminated description of a status code. */
const char* fc_status_string(fc_status s);

/* Element type of Q, K, V, K_out, V_out and of the chunk states. */
typedef enum { FC_F32 = 0, FC_BF16 = 1, FC_DTYPE_MAX_ENUM = 0x7fffffff } fc_dtype;

/* ------------------------------------------------------------------------ */
/* Joint importance-redundancy KV compression (Key designs, item 3)         */
/* ------------------------------------------------------------------------ */

/*
 * Parameters in the page's notation.
 *   H            heads (every head is compressed independently)
 *   d            head dimension, 64 or 128
 *   L_q          denoising queries (the active chunk's tokens)
 *   L_k          clean keys in the cache before compression
 *   B_budget     tokens each head keeps; B' = min(B_budget, L_k)
 *   lambda       importance weight in [0,1]
 *   pool_window  odd max-pool window, 1 <= w <= 129 (stride 1, same size,
 *                positions outside [0, L_k) ignored, along the token order)
 *   softmax_scale attention temperature; 0 means 1/sqrt(d)
 *   dtype        FC_BF16 or FC_F32 for Q, K, V and K_out, V_out
 */
typedef struct {
    int32_t H, d, L_q, L_k, B_budget;
    float lambda;
    int32_t pool_window;
    float softmax_scale;
    fc_dtype dtype;
} fc_kv_params;

/* Workspace bytes that fc_kv_compress, fc_kv_importance,
 * fc_kv_importance_redundancy, fc_kv_importance_lse, fc_kv_importance_colsum,
 * fc_kv_redundancy and fc_kv_select need for these parameters (0 if the
 * parameters are invalid). */
size_t fc_kv_compress_workspace_bytes(const fc_kv_params* p);

/*
 * fc_kv_compress -- the whole compression step for all heads.
 *   Q [H][L_q][d], K [H][L_k][d], V [H][L_k][d]       device, dtype
 *   K_out, V_out [H][B'][d]                           device, dtype; the rows
 *                                                     of the kept tokens, in
 *                                                     ascending token order
 *   idx_out [H][B']  int32                            device; kept token
 *                                                     indices, ascending
 *   score_out, imp_pooled_out, red_out [H][L_k] f32   device, nullable: the
 *                                                     joint score, the pooled
 *                                                     importance, the
 *                                                     redundancy softmax
 *   workspace                                         device, >= the query
 * Selection order: larger score first; equal scores keep the lower index.
 * L_k <= B_budget keeps every token (idx = 0..L_k-1); when no score output
 * is asked for, that call only copies the rows.  Zero-norm keys are
 * normalised with max(||k||, 1e-12) and so contribute no similarity.  A
 * key's squared norm is summed in float32: keys whose squared norm exceeds
 * the float32 range (elements beyond about 1e19) are outside the domain.
 * Deterministic on one device model: identical inputs give bit-identical
 * outputs.  The importance passes split their work from the device's compute
 * unit count and occupancy, which fixes the float32 summation order; a
 * device of another model may round differently (within the float32
 * accuracy of the sums).
 */
fc_status fc_kv_compress(const fc_kv_params* p, const void* Q, const void* K, const void* V,
                         void* K_out, void* V_out, int32_t* idx_out,
                         float* score_out, float* imp_pooled_out, float* red_out,
                         void* workspace, size_t workspace_bytes, void* stream);

/*
 * fc_kv_importance -- importance before the pool:
 *   imp_out[h][j] = (1/L_q) sum_i exp(s_ij - lse_i),  s_ij = scale q_i.k_j,
 *   lse_i = log sum_j exp(s_ij)  (softmax over the clean keys only).
 * Q, K device (dtype); imp_out [H][L_k] f32 device.  Uses p->H, d, L_q, L_k,
 * softmax_scale, dtype.
 */
fc_status fc_kv_importance(const fc_kv_params* p, const void* Q, const void* K, float* imp_out,
                           void* workspace, size_t workspace_bytes, void* stream);

/*
 * fc_kv_importance_redundancy -- the first half of fc_kv_compress, with the
 * same launches: importance pass 1 with the partial sums of the normalised
 * keys in extra workgroups, the merge, then pass 2, which also forms the
 * redundancy of the keys it holds:
 *   imp_out[h][j] as fc_kv_importance writes it (the same bits),
 *   r_out[h][j]   = (1/L_k) sum_{i != j} khat_i.khat_j  as fc_kv_redundancy
 *                   defines it (float32 sums in another order).
 * Q, K device (dtype); imp_out, r_out [H][L_k] f32 device.  Uses p->H, d,
 * L_q, L_k, softmax_scale, dtype.  Their outputs feed fc_kv_select.
 */
fc_status fc_kv_importance_redundancy(const fc_kv_params* p, const void* Q, const void* K, float* imp_out,
                                      float* r_out, void* workspace, size_t workspace_bytes, void* stream);

/*
 * fc_kv_importance_lse -- the first of the two passes alone:
 *   lse_out[h][i] = log sum_j exp(scale q_i.k_j)   (natural log, f32 [H][L_q])
 * over the clean keys.  Q, K device (dtype); lse_out device.
 */
fc_status fc_kv_importance_lse(const fc_kv_params* p, const void* Q, const void* K, float* lse_out,
                               void* workspace, size_t workspace_bytes, void* stream);

/*
 * fc_kv_importance_colsum -- the second pass alone, given the normalisers:
 *   imp_out[h][j] = (1/L_q) sum_i exp(scale q_i.k_j - lse[h][i]).
 * lse [H][L_q] f32 device (natural log, as written by fc_kv_importance_lse).
 * The workspace (same size query) receives the normalisers in the kernel's
 * own form before the pass.
 */
fc_status fc_kv_importance_colsum(const fc_kv_params* p, const void* Q, const void* K, const float* lse,
                                  float* imp_out, void* workspace, size_t workspace_bytes, void* stream);

/*
 * fc_kv_redundancy -- mean cosine similarity before its softmax:
 *   r_out[h][j] = (1/L_k) sum_{i != j} khat_i.khat_j,  khat = k / max(||k||, 1e-12),
 * computed as (u.khat_j - khat_j.khat_j)/L_k with u = sum_i khat_i (no L_k^2
 * matrix).  K device (dtype); r_out [H][L_k] f32 device.  Uses p->H, d, L_k,
 * dtype.
 */
fc_status fc_kv_redundancy(const fc_kv_params* p, const void* K, float* r_out,
                           void* workspace, size_t workspace_bytes, void* stream);

/*
 * fc_kv_select -- pool, score, top-B and gather from given importance and
 * redundancy means:
 *   imp [H][L_k] f32 device (before the pool), r [H][L_k] f32 device (before
 *   the softmax).  Red = softmax_j(r), Imp~ = max-pool(imp), Score as above.
 *   K, V, K_out, V_out may all be NULL (indices only); otherwise all four are
 *   required.  Other outputs as for fc_kv_compress.
 */
fc_status fc_kv_select(const fc_kv_params* p, const float* imp, const float* r,
                       const void* K, const void* V, void* K_out, void* V_out, int32_t* idx_out,
                       float* score_out, float* imp_pooled_out, float* red_out,
                       void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes for fc_topb_select. */
size_t fc_topb_select_workspace_bytes(int32_t H, int32_t L);

/*
 * fc_topb_select -- per row h of scores [H][L] (f32, device), the
 * B' = min(B, L) largest values, ties to the lower index, written to
 * idx_out [H][B'] (int32, device) in ascending index order.  -0.0 and +0.0
 * are equal.  Exact: the result is a function of the float32 values only.
 */
fc_status fc_topb_select(int32_t H, int32_t L, int32_t B, const float* scores, int32_t* idx_out,
                         void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------ */
/* KV cache manager (Key designs item 3; flowchart under 整体框架)          */
/* ------------------------------------------------------------------------ */

/*
 * The page splits a fixed KV buffer of B_total = B_budget + B_active tokens
 * per head into a compressed clean region of B_budget tokens and the region
 * of the chunk being denoised (B_active).  When a chunk completes it enters
 * the cache; if the clean tokens and the chunk together exceed B_budget
 * ("cache full"), the merged set is compressed back to B_budget tokens per
 * head with the joint score above; otherwise the chunk is kept as it is.
 *
 * The cache is two regions of that buffer's shape, K and V [H][B_total][d]
 * (dtype) and positions [H][B_total] (int32, optional), all device memory:
 * the current region and a spare.  In the current region, head h's clean
 * tokens are rows 0..L_clean-1 in ascending position order and the chunk
 * being denoised takes the rows right behind them.  A compressing commit
 * reads the current region and writes the kept tokens into the spare one,
 * which becomes the current region: the merged set is never copied.
 *
 *   H, d, lambda, pool_window, softmax_scale, dtype   as in fc_kv_params
 *   B_budget   clean tokens each head keeps
 *   B_active   most tokens one committed chunk may bring (per head)
 */
typedef struct {
    int32_t H, d, B_budget, B_active;
    float lambda;
    int32_t pool_window;
    float softmax_scale;
    fc_dtype dtype;
} fc_cache_params;

/* Workspace bytes that fc_cache_commit needs for any commit scored by L_q
 * queries (0 if the parameters are invalid): the kept indices [H][B_budget]
 * and the compression's workspace for the largest merged set.  A commit that
 * does not compress needs no workspace. */
size_t fc_cache_commit_workspace_bytes(const fc_cache_params* c, int32_t L_q);

/*
 * fc_cache_commit -- a completed chunk enters the cache.
 *   L_clean          host int32 in/out: clean tokens per head before the call
 *                    (0..B_budget); after it, min(L_clean + L_c, B_budget)
 *   K_chunk, V_chunk [H][L_c][d] device, dtype, or both NULL: the chunk's
 *                    keys and values, copied to rows L_clean..L_clean+L_c-1
 *                    of the current region; NULL when the producer already
 *                    wrote them there.  1 <= L_c <= B_active
 *   pos0             position of the chunk's first token (its tokens get
 *                    pos0, pos0 + 1, ...; pos0 >= 0, pos0 + L_c - 1 <= 2^31 - 1),
 *                    written to the chunk's rows of pos_cur
 *   Q [H][L_q][d]    device, dtype: the queries that score a compression;
 *                    may be NULL when the chunk fits (no compression)
 *   K_cur, V_cur, pos_cur        the current region (pos_cur nullable)
 *   K_spare, V_spare, pos_spare  the spare region: written only by a commit
 *                    that compresses, and then required (pos_spare NULL
 *                    exactly when pos_cur is)
 *   swapped          host int32 out, nullable: 1 when the commit compressed
 *                    and the clean tokens are now rows 0..B_budget-1 of the
 *                    spare region (the caller swaps the two regions' roles);
 *                    0 when they stay in the current region
 * Not full (L_clean + L_c <= B_budget): the chunk's rows stay (or are copied)
 * behind the clean rows.  Full: rows 0..L_clean+L_c-1 of the current region
 * are compressed as by fc_kv_compress with L_k = L_clean + L_c, into the
 * spare region, and the positions follow the kept rows.  The workspace
 * (device, >= the query for this L_q) may be NULL for a commit that does not
 * compress.  K_chunk, V_chunk and Q must not overlap either region, nor the
 * two regions each other.  *L_clean and *swapped are set when the work has
 * been queued.  Errors as for fc_kv_compress; an L_clean, L_c or pos0 out of
 * range, only one of K_chunk and V_chunk, or a NULL Q or spare region for a
 * commit that compresses, is FC_ERR_INVALID_ARG, and so is a spare tensor at
 * the address of a current one (the one overlap the library can see).
 */
fc_status fc_cache_commit(const fc_cache_params* c, int32_t* L_clean,
                          const void* K_chunk, const void* V_chunk, int32_t L_c, int32_t pos0,
                          const void* Q, int32_t L_q,
                          void* K_cur, void* V_cur, int32_t* pos_cur,
                          void* K_spare, void* V_spare, int32_t* pos_spare, int32_t* swapped,
                          void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------ */
/* Chunkwise relative L1 and reuse decision (Key designs, items 1 and 2)    */
/* ------------------------------------------------------------------------ */

/*
 *   n_chunks  chunks in the flat state arrays, 1..FC_MAX_CHUNKS
 *   m         forced-recompute steps counted from each chunk's first step
 *   eps       reuse threshold
 *   dtype     FC_BF16 or FC_F32 for the states
 */
#define FC_MAX_CHUNKS 128
typedef struct {
    int32_t n_chunks;
    int32_t m;
    float eps;
    fc_dtype dtype;
} fc_l1_params;

/* Workspace bytes for these chunk offsets (host array of n_chunks+1). */
size_t fc_chunk_rel_l1_workspace_bytes(const fc_l1_params* p, const int64_t* chunk_offsets);

/*
 * fc_chunk_rel_l1_decide -- one denoising step's decision for every chunk.
 *   chunk_offsets  host int64[n_chunks+1], element offsets into the states,
 *                  non-decreasing, chunk i = [off[i], off[i+1]), off[0] >= 0
 *   X_t, X_tm1     device, dtype: the current state X_t and the next state
 *                  X_{t-1}, chunks concatenated
 *   step           device int32[n_chunks] in/out: each chunk's local step n
 *                  (0 on its first step); < 0 marks an inactive chunk, whose
 *                  elements are not read and whose outputs are left untouched
 *   f              device f32[n_chunks] in/out: the accumulator
 *   recompute      device uint8[n_chunks] out: 1 = recompute, 0 = reuse
 *   l1_rel_out     device f32[n_chunks], nullable: L1_rel of this step
 *                  (+inf when ||X_t||_1 = 0)
 * For an active chunk with local step n:
 *   n < m:  recompute = 1, f = 0;
 *   else a = f + L1_rel;  a > eps: recompute = 1, f = 0;  else recompute = 0, f = a;
 *   then step = n + 1.
 * Sums are taken in float32 per thread and combined in a fixed order
 * (deterministic); the decision runs on the device, with no host round trip.
 * The workspace needs no initialisation; calls that share one workspace must
 * be ordered (same stream).
 */
fc_status fc_chunk_rel_l1_decide(const fc_l1_params* p, const int64_t* chunk_offsets,
                                 const void* X_t, const void* X_tm1,
                                 int32_t* step, float* f, uint8_t* recompute, float* l1_rel_out,
                                 void* workspace, size_t workspace_bytes, void* stream);

/*
 * fc_chunk_rel_l1_decide_noalloc -- fc_chunk_rel_l1_decide for callers that
 * cannot allocate (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): no workspace argument and no allocation
 * of any kind.  The slab partials live in a static device array of
 * FC_NOALLOC_SCRATCH_BYTES per device (one float2 per slab of 32768 bf16 or
 * 16384 float32 elements, each chunk rounded up to whole slabs: about 1.07e9
 * bf16 or 5.4e8 float32 elements in all), held until the process ends.
 * Arguments, results and errors as for fc_chunk_rel_l1_decide, the same
 * kernels and the same bits; states beyond the array's slabs are
 * FC_ERR_UNSUPPORTED (checked on the host, before anything touches the
 * device).  Every call on one device shares that device's array, so calls
 * that overlap in time on one device (different streams, or threads without
 * ordering) race and must not be made; calls ordered on one stream are safe.
 */
#define FC_NOALLOC_SCRATCH_BYTES ((size_t)256 * 1024)
fc_status fc_chunk_rel_l1_decide_noalloc(const fc_l1_params* p, const int64_t* chunk_offsets,
                                         const void* X_t, const void* X_tm1,
                                         int32_t* step, float* f, uint8_t* recompute, float* l1_rel_out,
                                         void* stream);

/*
 * fc_euler_step_l1_decide -- the sampler's Euler step with the decision fused.
 * Item 1 writes the L1 numerator as ||v dt||_1: the update X_{t-1} = X_t + v dt
 * itself.  For every active chunk i:
 *   X_next = X_t + v * dt[i]   per element, in float32 (the product and the sum
 *                              each rounded, no fused multiply-add), then
 *                              rounded to the storage type (bf16: to nearest,
 *                              ties to even);
 * then the decision exactly as fc_chunk_rel_l1_decide on (X_t, X_next): the
 * same sums in the same order, so the same bits.
 *   v       device, dtype: the velocity, laid out as the states
 *   dt      device f32[n_chunks]: each chunk's step of the schedule
 *   X_next  device, dtype: the next state; may be X_t itself (in-place
 *           update), otherwise it must not overlap X_t or v
 * Inactive chunks (step < 0) are neither read nor written.  Other arguments,
 * the workspace and errors as for fc_chunk_rel_l1_decide (same workspace
 * query).
 */
fc_status fc_euler_step_l1_decide(const fc_l1_params* p, const int64_t* chunk_offsets,
                                  const void* X_t, const void* v, const float* dt, void* X_next,
                                  int32_t* step, float* f, uint8_t* recompute, float* l1_rel_out,
                                  void* workspace, size_t workspace_bytes, void* stream);

/*
 * fc_uniform_rel_l1_decide -- the uniform policy the FlowCache page contrasts
 * with (背景与动机: TeaCache-style caches take one reuse/recompute decision
 * for all content at a timestep): one relative L1 over every active chunk,
 *   L1_rel = sum_i ||X^i_{t-1} - X^i_t||_1 / sum_i ||X^i_t||_1  (active i),
 * one accumulator f and one step counter, the rule of item 2, and the same
 * decision for every active chunk.
 *   chunk_step  device int32[n_chunks], read only: < 0 marks an inactive
 *               chunk (not read, its recompute flag untouched)
 *   step        device int32[1] in/out: the shared local step
 *   f           device f32[1] in/out
 *   recompute   device uint8[n_chunks] out (active chunks only)
 *   l1_rel_out  device f32[1], nullable
 * Other arguments, the workspace query and errors as for
 * fc_chunk_rel_l1_decide.
 */
fc_status fc_uniform_rel_l1_decide(const fc_l1_params* p, const int64_t* chunk_offsets,
                                   const void* X_t, const void* X_tm1, const int32_t* chunk_step,
                                   int32_t* step, float* f, uint8_t* recompute, float* l1_rel_out,
                                   void* workspace, size_t workspace_bytes, void* stream);

/*
 * fc_history_rel_l1_decide -- the History-Guided Cache rule of ARCache (page
 * "Accelerating Autoregressive Video Diffusion via History-Guided Cache and
 * Residual Correction", papernotes CVPR 2026 digest, 关键设计 item 1), per
 * segment i of the history tokens:
 *   Delta_i = ||h_t - h_{t+1}||_1 / ||h_{t+1}||_1
 * (h_prev = h_{t+1}, the previous step's history tokens; h_cur = h_t).  The
 * cache is reused while the deviations summed from the last refresh step
 * t_ref (that step included) through this one stay <= delta (p->eps);
 * otherwise it refreshes and t_ref becomes this step, so the sum restarts at
 * this step's Delta:
 *   n < m:  refresh = 1, acc = Delta;
 *   else a = acc + Delta;  a > delta: refresh = 1, acc = Delta;  else refresh = 0, acc = a;
 *   then step = n + 1.
 * Arguments as for fc_chunk_rel_l1_decide (segments in place of chunks;
 * dev_out, nullable, receives Delta; +inf when ||h_{t+1}||_1 = 0).
 */
fc_status fc_history_rel_l1_decide(const fc_l1_params* p, const int64_t* segment_offsets,
                                   const void* h_prev, const void* h_cur,
                                   int32_t* step, float* acc, uint8_t* refresh, float* dev_out,
                                   void* workspace, size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* FLOWCACHE_H */
