// Host-side launchers of the gfx950 kernels (internal to libflowcache).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace fc {

// ---- importance (two passes) ----------------------------------------------
// Pass 1 splits the keys of each head into `nsplit` ranges of
// `keys_per_split` keys (a multiple of the key tile) to fill the machine when
// H * ceil(L_q/128) is small; pass 2 merges the per-range (max, sum) pairs.
struct ImpPlan {
    int nsplit;
    int keys_per_split;
};
ImpPlan imp_plan(int H, int Lq, int Lk, int dt);
hipError_t launch_imp_lse(int dt, int d, const void* Q, const void* K, float2* part, int H, int Lq,
                          int Lk, const ImpPlan& plan, float c, hipStream_t s);
// Queries padded to whole pass-2 tiles.
int imp_lq_pad(int Lq);
// Pass 2 from -lse2 [H][imp_lq_pad(Lq)] (base-2 log-sum-exp of the scaled
// logits, negated, padded with -inf).
hipError_t launch_imp_colsum(int dt, int d, const void* Q, const void* K, const float* nlse2, float* imp, int H,
                             int Lq, int Lk, float c, hipStream_t s);
// From the pass-1 partials: the natural-log lse [H][Lq] and/or -lse2 (either
// may be nullptr).
hipError_t launch_imp_lse_merge(const float2* part, float* lse, float* nlse2, int H, int Lq, int nsplit,
                                hipStream_t s);
// -lse2 from a natural-log lse.
hipError_t launch_imp_nlse2(const float* lse, float* nlse2, int H, int Lq, hipStream_t s);

// ---- redundancy -------------------------------------------------------------
// Blocks per head of the two redundancy passes.
int red_nbu(int Lk);
int red_nbr(int Lk);
// Pass A: per-block partial u = sum khat over the block's keys -> u_part[H][nbu][d].
// Also zeroes hist0 (H * hist_words uint32) when hist != nullptr.
hipError_t launch_red_norm_sum(int dt, int d, const void* K, float* u_part, int H, int Lk,
                               uint32_t* hist, size_t hist_words, hipStream_t s);
// Pass B: r = (u.khat - khat.khat)/Lk and per-block softmax partials (max, sum e^{r-max}).
hipError_t launch_red_dot(int dt, int d, const void* K, const float* u_part, float* r,
                          float2* red_part, int H, int Lk, hipStream_t s);
// Softmax partials of a given r (used when r comes from the caller).
hipError_t launch_red_stats(const float* r, float2* red_part, int H, int Lk, uint32_t* hist,
                            size_t hist_words, hipStream_t s);

// ---- selection ----------------------------------------------------------------
constexpr int kSelTile = 2048;  // keys per selection block
constexpr int kHistBins = 4096;
constexpr int kHistWordsPerHead = 3 * kHistBins;
int sel_nblk(int L);
struct SelBuffers {
    uint32_t* keys;    // [H][L]
    uint32_t* hist;    // [H][3][4096]
    uint32_t* counts;  // [H][nblk][2]
    uint32_t* state;   // [H][2]: threshold key, tie quota
};
// Keys (and histogram round 0) from importance + redundancy, or from scores.
hipError_t launch_sel_keys_from_imp(const float* imp, const float* r, const float2* red_part, int nbr,
                                    float lam, int w, float* score_out, float* imp_pooled_out,
                                    float* red_out, const SelBuffers& b, int H, int L, hipStream_t s);
hipError_t launch_sel_keys_from_scores(const float* scores, const SelBuffers& b, int H, int L,
                                       hipStream_t s);
hipError_t launch_zero_u32(uint32_t* p, size_t n, hipStream_t s);
// Radix refinement, counting and compaction into idx_out [H][Bp].
hipError_t launch_sel_finish(const SelBuffers& b, int H, int L, int Bp, int32_t* idx_out, hipStream_t s);
// K_out[h][b] = K[h][idx[h][b]], V likewise.
hipError_t launch_gather(int dt, int d, const int32_t* idx, int H, int L, int Bp, const void* K, const void* V,
                         void* K_out, void* V_out, hipStream_t s);

// ---- chunk relative L1 ------------------------------------------------------
constexpr int kMaxChunks = 128;
struct ChunkTable {
    int n;
    int32_t blk_start[kMaxChunks + 1];
    long long off[kMaxChunks + 1];
};
int chunk_blocks_for(long long elems, int dt);
hipError_t launch_chunk_l1(int dt, const ChunkTable& tab, const void* X_t, const void* X_tm1,
                           int32_t* step, float* f, uint8_t* recompute, float* l1_out, float2* partial,
                           int m, float eps, hipStream_t s);

}  // namespace fc
