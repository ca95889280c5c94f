// Host-side launchers of the gfx950 kernels (internal to libflowcache).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace fc {

// ---- importance (two passes) ----------------------------------------------
// Pass 1 splits the keys of each head into `nsplit` ranges of
// `keys_per_split` keys (whole key tiles), chosen from the device's
// workgroup slots so that the last round of the grid is nearly full.  Pass 2
// splits the queries into `nqs` ranges of `qtiles_per_split` query tiles,
// one partial importance plane per range, only when its key blocks alone
// leave workgroup slots idle (few keys, many queries): measured on the
// MAGI-like shape, where the key blocks fill several rounds, any split costs
// more in per-workgroup set-up (each range re-loads its keys) than it saves
// in the grid's last round.
constexpr int kMaxQSplit = 64;
struct ImpPlan {
    int nsplit;
    int keys_per_split;
    int nqs;
    int qtiles_per_split;
    int slots_lse, slots_colsum;  // workgroups of each pass resident on the device at once
    // persistent passes: one workgroup per slot taking items from per-XCD
    // counters (queue words [0, 8) for pass 1, [8, 16) for pass 2)
    bool persistent_lse = false, persistent_colsum = false;
};
constexpr int kImpQueueWords = 16;
// Zeroes the persistent passes' counters (kImpQueueWords words).
hipError_t launch_imp_queue_zero(uint32_t* queue, hipStream_t s);
ImpPlan imp_plan(int H, int Lq, int Lk, int dt, int d);
// With u_part != nullptr the same launch also runs redundancy pass A as
// H * nbu extra workgroups: u_part[h][b] = sum of khat over key range b of
// head h (the ranges of launch_red_norm_sum).
// queue: the pass's 8 counters, zeroed beforehand, or nullptr (one item per
// workgroup); used only when the plan makes the pass persistent.
// ldk: rows per head in K (head h starts at row h * ldk); values below Lk
// mean dense (Lk).  The same for launch_imp_colsum.
hipError_t launch_imp_lse(int dt, int d, const void* Q, const void* K, float2* part, int H, int Lq,
                          int Lk, const ImpPlan& plan, float c, hipStream_t s, float* u_part = nullptr,
                          int nbu = 0, uint32_t* queue = nullptr, int ldk = 0);
// Queries padded to whole pass-2 tiles.
int imp_lq_pad(int Lq);
// Pass 2 from -lse2 [H][imp_lq_pad(Lq)] (base-2 log-sum-exp of the scaled
// logits, negated, padded with -inf) into imp_part [nqs][H][Lk] (the planes
// add up to the importance).  With u != nullptr ([H][d], the sum of the
// normalised keys) pass 2 also writes the redundancy r [H][Lk] of the keys
// it holds and one softmax partial (max, sum e^{r-max}, base 2) per key
// block into red_part [H][imp_colsum_blocks(Lk)].
int imp_colsum_blocks(int Lk);
// Whether both importance launches of this plan (pass 1 with nbu redundancy
// workgroups per head) fit a dispatch's 32-bit work-item count.
bool imp_grids_fit(int H, int Lq, int Lk, const ImpPlan& plan, int nbu);
hipError_t launch_imp_colsum(int dt, int d, const void* Q, const void* K, const float* nlse2, float* imp_part, int H,
                             int Lq, int Lk, const ImpPlan& plan, float c, hipStream_t s, const float* u = nullptr,
                             float* r = nullptr, float2* red_part = nullptr, uint32_t* queue = nullptr,
                             int ldk = 0);
// imp [H][Lk] = the sum of the nqs planes of imp_part.
hipError_t launch_imp_sum_planes(const float* imp_part, float* imp, int H, int Lk, int nqs, hipStream_t s);
// From the pass-1 partials: the natural-log lse [H][Lq] and/or -lse2 (either
// may be nullptr).  With u_part != nullptr it also sums the redundancy
// partials u_part [H][nbu][d] into u [H][d].
hipError_t launch_imp_lse_merge(const float2* part, float* lse, float* nlse2, int H, int Lq, int nsplit,
                                hipStream_t s, const float* u_part = nullptr, int nbu = 0, float* u = nullptr,
                                int d = 0);
// -lse2 from a natural-log lse.
hipError_t launch_imp_nlse2(const float* lse, float* nlse2, int H, int Lq, hipStream_t s);
// ---- redundancy -------------------------------------------------------------
// Blocks per head of the two redundancy passes (at most kRedMaxBlocks each).
constexpr int kRedMaxBlocks = 64;
int red_nbu(int Lk);
int red_nbr(int Lk);
// Pass A: per-block partial u = sum khat over the block's keys -> u_part[H][nbu][d].
hipError_t launch_red_norm_sum(int dt, int d, const void* K, float* u_part, int H, int Lk, hipStream_t s);
// Pass B: r = (u.khat - khat.khat)/Lk and per-block softmax partials (max, sum e^{r-max}).
hipError_t launch_red_dot(int dt, int d, const void* K, const float* u_part, float* r,
                          float2* red_part, int H, int Lk, hipStream_t s);
// Softmax partials of a given r (used when r comes from the caller).
hipError_t launch_red_stats(const float* r, float2* red_part, int H, int Lk, hipStream_t s);

// ---- selection ----------------------------------------------------------------
// Scores (from importance + redundancy when r != nullptr, else `src` holds
// them), order-preserving keys, radix select of the B' largest and the ordered
// compaction into idx_out [H][Bp].  Heads of one chunk take one workgroup per
// head; longer heads split over several workgroups per head (four launches).
// `keys` is the selection workspace of sel_ws_bytes(H, L) bytes.
// With r != nullptr, `src` holds nsrc planes [nsrc][H][L] of importance that
// add up to it.
size_t sel_ws_bytes(int H, int L);
// Whether the split selection's launch grids fit a dispatch's 32-bit work-item count.
bool sel_grid_fits(int H, int L);
hipError_t launch_sel_head(const float* src, int nsrc, const float* r, const float2* red_part, int nbr, float lam,
                           int w, float* score_out, float* imp_pooled_out, float* red_out, uint32_t* keys, int H,
                           int L, int Bp, int32_t* idx_out, hipStream_t s);
// K_out[h][b] = K[h][idx[h][b]], V likewise; with pos_out also
// pos_out[h][b] = pos[h][idx[h][b]] (pos [H][L], pos_out [H][Bp]).  With
// idx_keep_all (Bp == L) every row is kept: idx is not read, and
// idx_keep_all[h][b] = b is written.  Head strides in rows: ld_in for K, V
// and pos, ld_out for K_out, V_out and pos_out (values below L and Bp mean
// dense: L and Bp).
hipError_t launch_gather(int dt, int d, const int32_t* idx, int H, int L, int Bp, const void* K, const void* V,
                         void* K_out, void* V_out, hipStream_t s, const int32_t* pos = nullptr,
                         int32_t* pos_out = nullptr, int32_t* idx_keep_all = nullptr, int ld_in = 0,
                         int ld_out = 0);

// ---- KV cache manager -----------------------------------------------------------
// dst[h][row0 + j] = fresh[h][j] for K and V, 0 <= j < n_new (skipped when
// K_new is null), head strides n_new / ld_dst rows; with pos_dst also
// pos_dst[h][row0 + j] = pos0 + j.
hipError_t launch_cache_append(int dt, int d, int H, const void* K_new, const void* V_new, int n_new, int32_t pos0,
                               void* K_dst, void* V_dst, int32_t* pos_dst, int ld_dst, int row0, hipStream_t s);

// ---- chunk relative L1 ------------------------------------------------------
constexpr int kMaxChunks = 128;
struct ChunkTable {
    int n;
    int32_t blk_start[kMaxChunks + 1];
    long long off[kMaxChunks + 1];
};
int chunk_blocks_for(long long elems, int dt);
// Decision rules: per chunk (FlowCache), per segment with the refresh step
// kept in the sum (ARCache's history-guided cache), or one decision for all
// active chunks (uniform).
enum DecisionRule : int { kRuleChunkwise = 0, kRuleHistory = 1, kRuleUniform = 2 };
// With X_next != nullptr, X_tm1 is the velocity v instead: the slab kernel
// writes X_next = X_t + v * step_dt[chunk] (Euler update, rounded to the
// storage type) and measures the L1 against it.  Under kRuleUniform, `step`
// is the per-chunk activity (read only), gstep [1] and f [1] the shared
// counter and accumulator, l1_out [1].
hipError_t launch_chunk_l1(int dt, const ChunkTable& tab, const void* X_t, const void* X_tm1,
                           int32_t* step, float* f, uint8_t* recompute, float* l1_out, float2* partial,
                           int m, float eps, hipStream_t s, const float* step_dt = nullptr,
                           void* X_next = nullptr, int rule = kRuleChunkwise, int32_t* gstep = nullptr);

}  // namespace fc
