// Joint score, per-head top-B selection and K/V compaction, "Flow Caching for
// Autoregressive Video Generation" (papernotes digest), Key designs item 3:
//     Imp~_j  = max{Imp_k : |k - j| <= (w-1)/2, 0 <= k < L}      (1-D max-pool)
//     Red_j   = e^{r_j - max r} / sum_k e^{r_k - max r}           (softmax over tokens)
//     Score_j = lambda Imp~_j - (1 - lambda) Red_j,
// and each head keeps its B' = min(B, L) best tokens (flowchart under
// 整体框架: cache full -> joint score -> top-B per head).
//
// Selection is exact on the float32 scores: each score becomes an
// order-preserving uint32 key, a three-round radix select (12 + 12 + 8 bits,
// LDS histograms merged with integer atomics) finds the B'-th largest key T
// and the number q of keys equal to T that fit, and a compaction keeps every
// key > T plus the first q keys == T in token order (ties go to the lower
// index).  Kept tokens are written in ascending token order, and a gather
// kernel with one block per 64 kept rows copies their K and V rows.  Integer
// atomics only, so the result is deterministic.
#include "common.hpp"
#include "kernels.hpp"

namespace fc {

namespace {

constexpr int kThreads = 256;
constexpr int kPer = kSelTile / kThreads;  // consecutive keys per thread
static_assert(kPer * kThreads == kSelTile, "tile");

// Larger float -> larger key; -0.0 and +0.0 map to the same key.
__device__ __forceinline__ uint32_t order_key(float x) {
    uint32_t u = __float_as_uint(x + 0.0f);  // -0.0 + 0.0 = +0.0
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Block-level search of a histogram for the bin holding the k-th largest
// element (k >= 1).  Returns the bin; *k_in_bin receives k minus the count in
// higher bins.  All threads get the result.
template <int BINS>
__device__ __forceinline__ int find_bin_from_top(const uint32_t* __restrict__ hist, uint32_t k,
                                                 uint32_t* k_in_bin) {
    constexpr int kPerT = BINS / kThreads;
    __shared__ uint32_t scan_lds[4];
    __shared__ int found_bin;
    __shared__ uint32_t found_k;
    // thread t owns bins BINS-1-(t*kPerT + i), i.e. descending order
    uint32_t cnt[kPerT];
    uint32_t sum = 0;
#pragma unroll
    for (int i = 0; i < kPerT; ++i) {
        cnt[i] = hist[BINS - 1 - (threadIdx.x * kPerT + i)];
        sum += cnt[i];
    }
    uint32_t total;
    const uint32_t before = block256_exclusive_scan(sum, scan_lds, &total);
    if (before < k && k <= before + sum) {
        uint32_t acc = before;
        for (int i = 0; i < kPerT; ++i) {
            if (acc + cnt[i] >= k) {
                found_bin = BINS - 1 - (threadIdx.x * kPerT + i);
                found_k = k - acc;
                break;
            }
            acc += cnt[i];
        }
    }
    __syncthreads();
    *k_in_bin = found_k;
    const int b = found_bin;
    __syncthreads();
    return b;
}

// Prefix (bits above the current round) and remaining rank after `rounds`
// completed rounds.
struct RadixState {
    uint32_t prefix;  // key bits fixed so far (in place)
    uint32_t k;       // rank still to find within the keys matching prefix
};
__device__ __forceinline__ RadixState radix_state(const uint32_t* __restrict__ hist_h, uint32_t Bp, int rounds) {
    RadixState st{0u, Bp};
    if (rounds >= 1) {
        uint32_t k1;
        const int b0 = find_bin_from_top<kHistBins>(hist_h, st.k, &k1);
        st.prefix = (uint32_t)b0 << 20;
        st.k = k1;
    }
    if (rounds >= 2) {
        uint32_t k2;
        const int b1 = find_bin_from_top<kHistBins>(hist_h + kHistBins, st.k, &k2);
        st.prefix |= (uint32_t)b1 << 8;
        st.k = k2;
    }
    if (rounds >= 3) {
        uint32_t k3;
        const int b2 = find_bin_from_top<256>(hist_h + 2 * kHistBins, st.k, &k3);
        st.prefix |= (uint32_t)b2;
        st.k = k3;
    }
    return st;
}

// Adds a block's LDS histogram into the global one (non-zero bins only).
template <int BINS>
__device__ __forceinline__ void flush_hist(const uint32_t* lh, uint32_t* gh) {
    for (int b = threadIdx.x; b < BINS; b += kThreads) {
        const uint32_t c = lh[b];
        if (c) atomicAdd(gh + b, c);
    }
}

__device__ __forceinline__ void zero_rounds_1_2(uint32_t* hist_h, int blk, int nblk) {
    // rounds 1 and 2 of this head's histogram, split over the head's blocks
    const int words = 2 * kHistBins;
    const int per = (words + nblk - 1) / nblk;
    const int b = blk * per, e = min(words, b + per);
    for (int i = b + threadIdx.x; i < e; i += kThreads) hist_h[kHistBins + i] = 0u;
}

// Round 0: keys from pooled importance and redundancy softmax.
__global__ __launch_bounds__(kThreads) void sel_keys_from_imp_kernel(
    const float* __restrict__ imp, const float* __restrict__ r, const float2* __restrict__ red_part, int nbr,
    float lam, int hw, float* __restrict__ score_out, float* __restrict__ imp_pooled_out,
    float* __restrict__ red_out, uint32_t* __restrict__ keys, uint32_t* __restrict__ hist, int L) {
    __shared__ float tile[kSelTile + 2 * 64];
    __shared__ uint32_t lh[kHistBins];
    __shared__ float stat[2];
    const int h = blockIdx.y, blk = blockIdx.x, nblk = gridDim.x;
    const int j0 = blk * kSelTile;
    const float* imph = imp + (size_t)h * L;
    for (int b = threadIdx.x; b < kHistBins; b += kThreads) lh[b] = 0u;
    zero_rounds_1_2(hist + (size_t)h * kHistWordsPerHead, blk, nblk);
    // importance tile with a halo of hw on each side (hw <= 64)
    for (int i = threadIdx.x; i < kSelTile + 2 * hw; i += kThreads) {
        const int j = j0 - hw + i;
        tile[i] = (j >= 0 && j < L) ? imph[j] : -INFINITY;
    }
    if (threadIdx.x == 0) {
        float M = -1e30f, S = 0.f;
        for (int i = 0; i < nbr; ++i) {
            const float2 v = red_part[(size_t)h * nbr + i];
            lse2_merge(M, S, v.x, v.y);
        }
        stat[0] = M;            // max of r * log2e
        stat[1] = 1.0f / S;     // 1 / sum 2^{r*log2e - M}
    }
    __syncthreads();
    const float M = stat[0], invS = stat[1];
    const float lam_red = 1.0f - lam;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
        const int lj = threadIdx.x * kPer + i;
        const int j = j0 + lj;
        if (j >= L) break;
        float pooled = tile[lj + hw];
        for (int o = 1; o <= hw; ++o) pooled = fmaxf(pooled, fmaxf(tile[lj + hw - o], tile[lj + hw + o]));
        const float red = exp2_hw(fmaf(r[(size_t)h * L + j], kLog2e, -M)) * invS;
        const float sc = lam * pooled - lam_red * red;
        const size_t o = (size_t)h * L + j;
        if (score_out) score_out[o] = sc;
        if (imp_pooled_out) imp_pooled_out[o] = pooled;
        if (red_out) red_out[o] = red;
        const uint32_t key = order_key(sc);
        keys[o] = key;
        atomicAdd(&lh[key >> 20], 1u);
    }
    __syncthreads();
    flush_hist<kHistBins>(lh, hist + (size_t)h * kHistWordsPerHead);
}

// Round 0 from given scores.
__global__ __launch_bounds__(kThreads) void sel_keys_from_scores_kernel(const float* __restrict__ scores,
                                                                        uint32_t* __restrict__ keys,
                                                                        uint32_t* __restrict__ hist, int L) {
    __shared__ uint32_t lh[kHistBins];
    const int h = blockIdx.y, blk = blockIdx.x, nblk = gridDim.x;
    for (int b = threadIdx.x; b < kHistBins; b += kThreads) lh[b] = 0u;
    zero_rounds_1_2(hist + (size_t)h * kHistWordsPerHead, blk, nblk);
    __syncthreads();
    const int j0 = blk * kSelTile;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
        const int j = j0 + threadIdx.x + kThreads * i;
        if (j < L) {
            const uint32_t key = order_key(scores[(size_t)h * L + j]);
            keys[(size_t)h * L + j] = key;
            atomicAdd(&lh[key >> 20], 1u);
        }
    }
    __syncthreads();
    flush_hist<kHistBins>(lh, hist + (size_t)h * kHistWordsPerHead);
}

// Rounds 1 (bits 19..8) and 2 (bits 7..0) over the keys matching the prefix.
template <int ROUND>
__global__ __launch_bounds__(kThreads) void sel_refine_kernel(const uint32_t* __restrict__ keys,
                                                              uint32_t* __restrict__ hist, int L, int Bp) {
    constexpr int BINS = ROUND == 1 ? kHistBins : 256;
    __shared__ uint32_t lh[BINS];
    const int h = blockIdx.y, blk = blockIdx.x;
    uint32_t* hist_h = hist + (size_t)h * kHistWordsPerHead;
    for (int b = threadIdx.x; b < BINS; b += kThreads) lh[b] = 0u;
    const RadixState st = radix_state(hist_h, (uint32_t)Bp, ROUND);
    const uint32_t shift = ROUND == 1 ? 20u : 8u;
    const uint32_t want = st.prefix >> shift;
    const int j0 = blk * kSelTile;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
        const int j = j0 + threadIdx.x + kThreads * i;
        if (j < L) {
            const uint32_t key = keys[(size_t)h * L + j];
            if ((key >> shift) == want) {
                const uint32_t dig = ROUND == 1 ? ((key >> 8) & 0xfffu) : (key & 0xffu);
                atomicAdd(&lh[dig], 1u);
            }
        }
    }
    __syncthreads();
    flush_hist<BINS>(lh, hist_h + ROUND * kHistBins);
}

// Threshold T (the B'-th largest key), quota q of keys == T, and per-block counts.
__global__ __launch_bounds__(kThreads) void sel_count_kernel(const uint32_t* __restrict__ keys,
                                                             const uint32_t* __restrict__ hist,
                                                             uint32_t* __restrict__ counts,
                                                             uint32_t* __restrict__ state, int L, int Bp) {
    __shared__ uint32_t scan_lds[4];
    const int h = blockIdx.y, blk = blockIdx.x, nblk = gridDim.x;
    const RadixState st = radix_state(hist + (size_t)h * kHistWordsPerHead, (uint32_t)Bp, 3);
    const uint32_t T = st.prefix;
    const int j0 = blk * kSelTile;
    uint32_t gt = 0, eq = 0;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
        const int j = j0 + threadIdx.x + kThreads * i;
        if (j < L) {
            const uint32_t key = keys[(size_t)h * L + j];
            gt += key > T;
            eq += key == T;
        }
    }
    uint32_t tgt, teq;
    block256_exclusive_scan(gt, scan_lds, &tgt);
    block256_exclusive_scan(eq, scan_lds, &teq);
    if (threadIdx.x == 0) {
        counts[((size_t)h * nblk + blk) * 2 + 0] = tgt;
        counts[((size_t)h * nblk + blk) * 2 + 1] = teq;
        if (blk == 0) {
            state[2 * h + 0] = T;
            state[2 * h + 1] = st.k;
        }
    }
}

// Compaction in token order: every kept token's index at its output slot.
__global__ __launch_bounds__(kThreads) void sel_compact_kernel(const uint32_t* __restrict__ keys,
                                                               const uint32_t* __restrict__ counts,
                                                               const uint32_t* __restrict__ state, int L, int Bp,
                                                               int32_t* __restrict__ idx_out) {
    __shared__ uint32_t scan_lds[4];
    __shared__ uint32_t base_lds[2];
    const int h = blockIdx.y, blk = blockIdx.x, nblk = gridDim.x;
    const uint32_t T = state[2 * h + 0], q = state[2 * h + 1];
    if (threadIdx.x < kWave) {
        uint32_t gb = 0, eb = 0;
        for (int b = threadIdx.x; b < blk; b += kWave) {
            gb += counts[((size_t)h * nblk + b) * 2 + 0];
            eb += counts[((size_t)h * nblk + b) * 2 + 1];
        }
        gb = wave_sum(gb);
        eb = wave_sum(eb);
        if (threadIdx.x == 0) { base_lds[0] = gb; base_lds[1] = eb; }
    }
    __syncthreads();
    const uint32_t gt_before = base_lds[0], eq_before = base_lds[1];
    const uint32_t out_base = gt_before + min(eq_before, q);

    const int j0 = blk * kSelTile + threadIdx.x * kPer;  // this thread's consecutive keys
    uint32_t kv[kPer];
    uint32_t neq = 0;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
        const int j = j0 + i;
        kv[i] = j < L ? keys[(size_t)h * L + j] : 0u;
        neq += (j < L && kv[i] == T);
    }
    uint32_t teq;
    uint32_t eq_rank = eq_before + block256_exclusive_scan(neq, scan_lds, &teq);
    uint32_t sel_mask = 0, nsel = 0;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
        const int j = j0 + i;
        bool s = false;
        if (j < L) {
            if (kv[i] > T) s = true;
            else if (kv[i] == T) { s = eq_rank < q; ++eq_rank; }
        }
        if (s) { sel_mask |= 1u << i; ++nsel; }
    }
    uint32_t tsel;
    uint32_t pos = out_base + block256_exclusive_scan(nsel, scan_lds, &tsel);
    int32_t* idx_h = idx_out + (size_t)h * Bp;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
        if (sel_mask & (1u << i)) {
            if (pos < (uint32_t)Bp) idx_h[pos] = j0 + i;  // always true when the counts agree
            ++pos;
        }
    }
}

// K_out[h][b] = K[h][idx[h][b]], V likewise: 16 bytes per lane, one row per
// kRowBytes/16 lanes, kGatherRows output rows per block.
constexpr int kGatherRows = 64;

template <int DT, int D>
__global__ __launch_bounds__(kThreads) void gather_rows_kernel(const int32_t* __restrict__ idx, int L, int Bp,
                                                               const void* __restrict__ K, const void* __restrict__ V,
                                                               void* __restrict__ K_out, void* __restrict__ V_out) {
    constexpr int kRowBytes = D * Elem<DT>::kBytes;
    constexpr int kTpr = kRowBytes / 16;     // lanes per row
    constexpr int kRpi = kThreads / kTpr;    // rows per step
    constexpr int kSteps = kGatherRows / kRpi;
    const int h = blockIdx.y;
    const int b0 = blockIdx.x * kGatherRows + threadIdx.x / kTpr;
    const int e = threadIdx.x % kTpr;
    const char* Ks = static_cast<const char*>(K) + (size_t)h * L * kRowBytes + e * 16;
    const char* Vs = static_cast<const char*>(V) + (size_t)h * L * kRowBytes + e * 16;
    char* Kd = static_cast<char*>(K_out) + (size_t)h * Bp * kRowBytes + e * 16;
    char* Vd = static_cast<char*>(V_out) + (size_t)h * Bp * kRowBytes + e * 16;
    int j[kSteps];
#pragma unroll
    for (int i = 0; i < kSteps; ++i) {
        const int b = b0 + i * kRpi;
        j[i] = b < Bp ? idx[(size_t)h * Bp + b] : -1;
    }
    uint4 kv[kSteps], vv[kSteps];
#pragma unroll
    for (int i = 0; i < kSteps; ++i) {
        if ((unsigned)j[i] < (unsigned)L) {
            kv[i] = *reinterpret_cast<const uint4*>(Ks + (size_t)j[i] * kRowBytes);
            vv[i] = *reinterpret_cast<const uint4*>(Vs + (size_t)j[i] * kRowBytes);
        }
    }
#pragma unroll
    for (int i = 0; i < kSteps; ++i) {
        if ((unsigned)j[i] < (unsigned)L) {
            const size_t b = (size_t)(b0 + i * kRpi);
            *reinterpret_cast<uint4*>(Kd + b * kRowBytes) = kv[i];
            *reinterpret_cast<uint4*>(Vd + b * kRowBytes) = vv[i];
        }
    }
}

__global__ void zero_u32_kernel(uint32_t* p, size_t n) {
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
        p[i] = 0u;
}

template <int DT, int D>
hipError_t gather_launch(const int32_t* idx, int H, int L, int Bp, const void* K, const void* V, void* K_out,
                         void* V_out, hipStream_t s) {
    const dim3 grid((Bp + kGatherRows - 1) / kGatherRows, H);
    hipLaunchKernelGGL((gather_rows_kernel<DT, D>), grid, dim3(kThreads), 0, s, idx, L, Bp, K, V, K_out, V_out);
    return hipGetLastError();
}

}  // namespace

int sel_nblk(int L) { return (L + kSelTile - 1) / kSelTile; }

hipError_t launch_zero_u32(uint32_t* p, size_t n, hipStream_t s) {
    hipLaunchKernelGGL(zero_u32_kernel, dim3(64), dim3(kThreads), 0, s, p, n);
    return hipGetLastError();
}

hipError_t launch_sel_keys_from_imp(const float* imp, const float* r, const float2* red_part, int nbr, float lam,
                                    int w, float* score_out, float* imp_pooled_out, float* red_out,
                                    const SelBuffers& b, int H, int L, hipStream_t s) {
    hipLaunchKernelGGL(sel_keys_from_imp_kernel, dim3(sel_nblk(L), H), dim3(kThreads), 0, s, imp, r, red_part,
                       nbr, lam, (w - 1) / 2, score_out, imp_pooled_out, red_out, b.keys, b.hist, L);
    return hipGetLastError();
}

hipError_t launch_sel_keys_from_scores(const float* scores, const SelBuffers& b, int H, int L, hipStream_t s) {
    hipLaunchKernelGGL(sel_keys_from_scores_kernel, dim3(sel_nblk(L), H), dim3(kThreads), 0, s, scores, b.keys,
                       b.hist, L);
    return hipGetLastError();
}

hipError_t launch_sel_finish(const SelBuffers& b, int H, int L, int Bp, int32_t* idx_out, hipStream_t s) {
    const dim3 grid(sel_nblk(L), H);
    hipLaunchKernelGGL(sel_refine_kernel<1>, grid, dim3(kThreads), 0, s, b.keys, b.hist, L, Bp);
    hipLaunchKernelGGL(sel_refine_kernel<2>, grid, dim3(kThreads), 0, s, b.keys, b.hist, L, Bp);
    hipLaunchKernelGGL(sel_count_kernel, grid, dim3(kThreads), 0, s, b.keys, b.hist, b.counts, b.state, L, Bp);
    hipLaunchKernelGGL(sel_compact_kernel, grid, dim3(kThreads), 0, s, b.keys, b.counts, b.state, L, Bp, idx_out);
    return hipGetLastError();
}

hipError_t launch_gather(int dt, int d, const int32_t* idx, int H, int L, int Bp, const void* K, const void* V,
                         void* K_out, void* V_out, hipStream_t s) {
    if (dt == kBF16)
        return d == 128 ? gather_launch<kBF16, 128>(idx, H, L, Bp, K, V, K_out, V_out, s)
                        : gather_launch<kBF16, 64>(idx, H, L, Bp, K, V, K_out, V_out, s);
    return d == 128 ? gather_launch<kF32, 128>(idx, H, L, Bp, K, V, K_out, V_out, s)
                    : gather_launch<kF32, 64>(idx, H, L, Bp, K, V, K_out, V_out, s);
}

}  // namespace fc
