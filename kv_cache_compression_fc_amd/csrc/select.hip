// Joint score, per-head top-B selection and K/V compaction, "Flow Caching for
// Autoregressive Video Generation" (papernotes digest), Key designs item 3:
//     Imp~_j  = max{Imp_k : |k - j| <= (w-1)/2, 0 <= k < L}      (1-D max-pool)
//     Red_j   = e^{r_j - max r} / sum_k e^{r_k - max r}           (softmax over tokens)
//     Score_j = lambda Imp~_j - (1 - lambda) Red_j,
// and each head keeps its B' = min(B, L) best tokens (flowchart under
// 整体框架: cache full -> joint score -> top-B per head).
//
// Heads of up to one chunk of keys (sel_head_kernel): one 1024-thread
// workgroup per head does the whole selection, exactly, on the float32
// scores.  Each score becomes an order-preserving uint32 key;
// three radix rounds (8 + 12 + 12 bits) with LDS histograms find the B'-th
// largest key T and the number q of keys equal to T that fit.  The scores of
// one head sit in a narrow range, so the top key bits (sign and exponent) put
// most keys into a few bins: every bin is kept in several copies, picked by
// the lane, which bounds the lanes of one atomic instruction that meet at one
// address.  An ordered compaction keeps every key > T plus the first q keys
// == T in token order (ties go to the lower index) and writes the kept
// indices ascending.  Keys are processed in chunks of 18 consecutive keys per
// thread, staged through LDS so that every global access is coalesced; a head
// that fits one chunk keeps its keys in LDS between the passes, a longer one
// re-reads them from the workspace.  Longer heads take the split selection
// further down (several workgroups per head, four 8-bit radix rounds over
// per-workgroup histograms, one launch each).  No global atomics: the result
// is deterministic.  A gather kernel with one kept row per lane group then
// copies their K and V rows.
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace fc {

namespace {

constexpr int kSelThreads = 1024;
constexpr int kSelWaves = kSelThreads / kWave;
constexpr int kKpt = 18;                      // consecutive keys per thread per chunk
constexpr int kChunk = kSelThreads * kKpt;    // 18432 keys per chunk
constexpr int kMaxHalo = 64;                  // pool half-window limit ((w-1)/2 <= 64)
constexpr int kRegHalo = 4;                   // half-windows served from registers
constexpr int kAWords = kMaxHalo + kChunk + kMaxHalo;  // LDS area A: importance tile / histograms / staging
constexpr int kR4 = (kChunk / 4 + kSelThreads - 1) / kSelThreads;    // 4-key groups of a chunk per thread
constexpr int kA4 = (kAWords / 4 + kSelThreads - 1) / kSelThreads;   // 4-key groups of area A per thread
static_assert(kMaxHalo % 4 == 0 && kChunk % 4 == 0, "4-key groups align with the chunk and its halo");

// Larger float -> larger key; -0.0 and +0.0 map to the same key.
__device__ __forceinline__ uint32_t order_key(float x) {
    uint32_t u = __float_as_uint(x + 0.0f);  // -0.0 + 0.0 = +0.0
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Exclusive prefix sum over a workgroup of NT threads; *total receives the
// sum.  `lds` holds NT/64 words.
template <int NT = kSelThreads>
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t v, uint32_t* lds, uint32_t* total) {
    constexpr int kWaves = NT / kWave;
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    uint32_t inc = v;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
        const uint32_t t = __shfl_up(inc, o, kWave);
        if (lane >= o) inc += t;
    }
    if (lane == kWave - 1) lds[wave] = inc;
    __syncthreads();
    uint32_t before = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
        const uint32_t x = lds[w];
        before += w < wave ? x : 0u;
        tot += x;
    }
    *total = tot;
    __syncthreads();
    return before + inc - v;
}

// The bin of an LDS histogram of BINS bins, each kept in COPIES copies
// (word bin*COPIES + copy), that holds the k-th largest element (k >= 1), and
// k minus the count of the higher bins; every thread gets both.
template <int BINS, int COPIES, int NT = kSelThreads>
__device__ __forceinline__ uint32_t find_bin_from_top(const uint32_t* hist, uint32_t k, uint32_t* k_in_bin,
                                                      uint32_t* scan_lds, uint32_t* s_res) {
    constexpr int kPerT = BINS >= NT ? BINS / NT : 1;
    constexpr int kActive = BINS / kPerT;
    // thread t owns bins BINS-1-(t*kPerT + i): descending order
    uint32_t cnt[kPerT];
    uint32_t sum = 0;
#pragma unroll
    for (int i = 0; i < kPerT; ++i) {
        uint32_t c = 0;
        if (threadIdx.x < kActive) {
            const uint32_t* hb = hist + (BINS - 1 - (threadIdx.x * kPerT + i)) * COPIES;
#pragma unroll
            for (int cp = 0; cp < COPIES; ++cp) c += hb[cp];
        }
        cnt[i] = c;
        sum += c;
    }
    uint32_t total;
    const uint32_t before = block_exclusive_scan<NT>(sum, scan_lds, &total);
    if (sum > 0 && before < k && k <= before + sum) {
        uint32_t acc = before;
        for (int i = 0; i < kPerT; ++i) {
            if (acc + cnt[i] >= k) {
                s_res[0] = BINS - 1 - (threadIdx.x * kPerT + i);
                s_res[1] = k - acc;
                break;
            }
            acc += cnt[i];
        }
    }
    __syncthreads();
    *k_in_bin = s_res[1];
    const uint32_t b = s_res[0];
    __syncthreads();
    return b;
}

// kFromImp: scores from importance (nsrc planes [nsrc][H][L] that add up to
// it; pooled here) and redundancy r with its softmax partials red_part
// [H][nbr]; otherwise `src` holds the scores.
template <bool kFromImp, bool kVec>
__global__ __launch_bounds__(kSelThreads) void sel_head_kernel(
    const float* __restrict__ src, int nsrc, const float* __restrict__ r, const float2* __restrict__ red_part, int nbr,
    float lam, int hw, float* __restrict__ score_out, float* __restrict__ imp_pooled_out,
    float* __restrict__ red_out, uint32_t* __restrict__ keys, int L, int Bp, int32_t* __restrict__ idx_out) {
    // Area A: the chunk's importance with its halo (tile_a[kMaxHalo + x] =
    // Imp[c0 + x]) while the keys are formed, then the radix histograms, then
    // the staging of the kept indices.  tile_b: the chunk's r (or scores),
    // then its keys.
    __shared__ __align__(16) uint32_t area_a[kAWords];
    __shared__ __align__(16) uint32_t tile_b[kChunk];
    __shared__ uint32_t scan_lds[kSelWaves];
    float* const tile_a = reinterpret_cast<float*>(area_a);
    uint32_t* const hist = area_a;
    __shared__ uint32_t s_res[2];
    __shared__ float stat[2];

    const int h = blockIdx.x, tid = threadIdx.x;
    const size_t hL = (size_t)h * L;
    const int nch = (L + kChunk - 1) / kChunk;
    const bool cached = nch == 1;  // the keys stay in tile_b between the passes
    const int x0 = tid * kKpt;     // this thread's first key in a chunk

    // softmax statistics of r, (max of r*log2e, 1 / sum 2^{r*log2e - max}),
    // by wave 0 while the first chunk's loads are in flight
    auto red_stats = [&]() {
        if (tid < kWave) {
            float M = -1e30f, S = 0.f;
            for (int i = tid; i < nbr; i += kWave) {
                const float2 v = red_part[(size_t)h * nbr + i];
                lse2_merge(M, S, v.x, v.y);
            }
#pragma unroll
            for (int o = kWave / 2; o > 0; o >>= 1) {
                const float m2 = __shfl_xor(M, o, kWave), s2 = __shfl_xor(S, o, kWave);
                lse2_merge(M, S, m2, s2);
            }
            if (tid == 0) {
                stat[0] = M;
                stat[1] = 1.0f / S;
            }
        }
    };

    // ---- keys --------------------------------------------------------------------------
    for (int c = 0; c < nch; ++c) {
        const int c0 = c * kChunk;
        const int n = min(kChunk, L - c0);
        // Every load of the chunk is issued before any is waited for: r (or
        // the scores), then the importance with a halo of hw <= kMaxHalo on
        // each side (the planes added in a fixed order).
        constexpr int kQa = (kChunk + 2 * kMaxHalo + kSelThreads - 1) / kSelThreads;
        const float* rs = (kFromImp ? r : src) + hL + c0;
        const size_t plane = (size_t)gridDim.x * L;
        if constexpr (kVec) {
            // 16-byte loads: r (or the scores) as 4-key groups of the chunk,
            // the importance as 4-key groups of [c0 - kMaxHalo, c0 + kChunk +
            // kMaxHalo) (keys outside [0, L) read as -inf), each group
            // stored at its own place in LDS
            float4 vr4[kR4], vi4[kA4];
#pragma unroll
            for (int q = 0; q < kR4; ++q) {
                const int g = tid + q * kSelThreads, e = 4 * g;
                if (e + 3 < n) {
                    vr4[q] = *reinterpret_cast<const float4*>(rs + e);
                } else {
                    vr4[q].x = e < n ? rs[e] : 0.f;
                    vr4[q].y = e + 1 < n ? rs[e + 1] : 0.f;
                    vr4[q].z = e + 2 < n ? rs[e + 2] : 0.f;
                    vr4[q].w = e + 3 < n ? rs[e + 3] : 0.f;
                }
            }
            if constexpr (kFromImp) {
                for (int pl = 0; pl < nsrc; ++pl) {
                    const float* ps = src + pl * plane + hL;
#pragma unroll
                    for (int q = 0; q < kA4; ++q) {
                        const int g = tid + q * kSelThreads, j = c0 - kMaxHalo + 4 * g;
                        float4 x;
                        if (j >= 0 && j + 3 < L) {
                            x = *reinterpret_cast<const float4*>(ps + j);
                        } else {
                            x.x = (j >= 0 && j < L) ? ps[j] : -INFINITY;
                            x.y = (j + 1 >= 0 && j + 1 < L) ? ps[j + 1] : -INFINITY;
                            x.z = (j + 2 >= 0 && j + 2 < L) ? ps[j + 2] : -INFINITY;
                            x.w = (j + 3 >= 0 && j + 3 < L) ? ps[j + 3] : -INFINITY;
                        }
                        if (pl == 0) vi4[q] = x;
                        else { vi4[q].x += x.x; vi4[q].y += x.y; vi4[q].z += x.z; vi4[q].w += x.w; }
                    }
                }
            }
            if (c == 0 && kFromImp) red_stats();
#pragma unroll
            for (int q = 0; q < kR4; ++q) {
                const int g = tid + q * kSelThreads;
                if (4 * g < kChunk)
                    reinterpret_cast<uint4*>(tile_b)[g] = make_uint4(__float_as_uint(vr4[q].x), __float_as_uint(vr4[q].y),
                                                                     __float_as_uint(vr4[q].z), __float_as_uint(vr4[q].w));
            }
            if constexpr (kFromImp) {
#pragma unroll
                for (int q = 0; q < kA4; ++q) {
                    const int g = tid + q * kSelThreads;
                    if (4 * g < kAWords) reinterpret_cast<float4*>(tile_a)[g] = vi4[q];
                }
            }
            __syncthreads();
        } else {
        float vr[kKpt], vi[kQa];
#pragma unroll
        for (int q = 0; q < kKpt; ++q) {
            const int i = tid + q * kSelThreads;
            vr[q] = i < n ? rs[i] : 0.f;
        }
        if constexpr (kFromImp) {
#pragma unroll
            for (int q = 0; q < kQa; ++q) {
                const int i = tid + q * kSelThreads, j = c0 - hw + i;
                vi[q] = (i < kChunk + 2 * hw && j >= 0 && j < L) ? src[hL + j] : -INFINITY;
            }
            for (int pl = 1; pl < nsrc; ++pl) {
#pragma unroll
                for (int q = 0; q < kQa; ++q) {
                    const int i = tid + q * kSelThreads, j = c0 - hw + i;
                    if (i < kChunk + 2 * hw && j >= 0 && j < L) vi[q] += src[pl * plane + hL + j];
                }
            }
            if (c == 0) red_stats();
        }
#pragma unroll
        for (int q = 0; q < kKpt; ++q) tile_b[tid + q * kSelThreads] = __float_as_uint(vr[q]);
        if constexpr (kFromImp) {
#pragma unroll
            for (int q = 0; q < kQa; ++q) {
                const int i = tid + q * kSelThreads;
                if (i < kChunk + 2 * hw) tile_a[kMaxHalo - hw + i] = vi[q];
            }
        }
        __syncthreads();
        }
        const float M = kFromImp ? stat[0] : 0.f, invS = kFromImp ? stat[1] : 0.f;
        float pooled[kKpt];
        if constexpr (kFromImp) {
            if (hw <= kRegHalo) {
                float v[kKpt + 2 * kRegHalo];
                const float2* t2 = reinterpret_cast<const float2*>(tile_a + kMaxHalo - kRegHalo + x0);
#pragma unroll
                for (int q = 0; q < (kKpt + 2 * kRegHalo) / 2; ++q) {
                    const float2 f = t2[q];
                    v[2 * q] = f.x;
                    v[2 * q + 1] = f.y;
                }
#pragma unroll
                for (int i = 0; i < kKpt; ++i) {
                    float p = v[kRegHalo + i];
#pragma unroll
                    for (int o = 1; o <= kRegHalo; ++o)
                        if (o <= hw) p = fmaxf(p, fmaxf(v[kRegHalo + i - o], v[kRegHalo + i + o]));
                    pooled[i] = p;
                }
            } else {
#pragma unroll
                for (int i = 0; i < kKpt; ++i) {
                    const float* t = tile_a + kMaxHalo + x0 + i;
                    float p = t[0];
                    for (int o = 1; o <= hw; ++o) p = fmaxf(p, fmaxf(t[-o], t[o]));
                    pooled[i] = p;
                }
            }
        }
        uint2* tb2 = reinterpret_cast<uint2*>(tile_b + x0);
#pragma unroll
        for (int q = 0; q < kKpt / 2; ++q) {
            const uint2 in = tb2[q];
            uint32_t out[2];
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const int i = 2 * q + e;
                const int j = c0 + x0 + i;
                const float x = __uint_as_float(e == 0 ? in.x : in.y);
                float sc = x;
                if constexpr (kFromImp) {
                    const float red = exp2_hw(fmaf(x, kLog2e, -M)) * invS;
                    sc = lam * pooled[i] - (1.0f - lam) * red;
                    if (j < L) {
                        if (score_out) score_out[hL + j] = sc;
                        if (imp_pooled_out) imp_pooled_out[hL + j] = pooled[i];
                        if (red_out) red_out[hL + j] = red;
                    }
                }
                out[e] = order_key(sc);
            }
            tb2[q] = make_uint2(out[0], out[1]);  // this thread's own slots
        }
        if (!cached) {
            __syncthreads();
#pragma unroll
            for (int q = 0; q < kKpt; ++q) {
                const int i = tid + q * kSelThreads;
                if (i < n) keys[hL + c0 + i] = tile_b[i];
            }
            __syncthreads();  // the tiles are refilled by the next chunk
        }
    }
    __syncthreads();  // area A (the importance tile) becomes the histograms
    // this thread's keys of chunk c (from tile_b; staged there when not cached)
    auto load_keys = [&](int c, uint32_t (&kv)[kKpt]) {
        if (!cached) {
            const int c0 = c * kChunk, n = min(kChunk, L - c0);
            uint32_t v[kKpt];
#pragma unroll
            for (int q = 0; q < kKpt; ++q) {
                const int i = tid + q * kSelThreads;
                v[q] = i < n ? keys[hL + c0 + i] : 0u;
            }
            __syncthreads();  // everybody is done with the previous contents
#pragma unroll
            for (int q = 0; q < kKpt; ++q) tile_b[tid + q * kSelThreads] = v[q];
            __syncthreads();
        }
        const uint2* tb2 = reinterpret_cast<const uint2*>(tile_b + x0);
#pragma unroll
        for (int q = 0; q < kKpt / 2; ++q) {
            const uint2 v = tb2[q];
            kv[2 * q] = v.x;
            kv[2 * q + 1] = v.y;
        }
    };

    // ---- radix rounds: bits 31..24, 23..12, 11..0 ---------------------------------
    // (a round's histogram counts the keys that match the bits fixed so far)
    const uint32_t copy16 = tid & 15u, copy4 = tid & 3u;
    auto round = [&](auto bits_c, auto copies_c, int sh, uint32_t pre, int pre_sh, uint32_t copy) {
        constexpr int kBitsR = decltype(bits_c)::value, kCopies = decltype(copies_c)::value;
        for (int b = tid; b < (1 << kBitsR) * kCopies; b += kSelThreads) hist[b] = 0u;
        __syncthreads();
        for (int c = 0; c < nch; ++c) {
            uint32_t kv[kKpt];
            load_keys(c, kv);
            const int j0 = c * kChunk + x0;
#pragma unroll
            for (int i = 0; i < kKpt; ++i) {
                const bool match = j0 + i < L && (pre_sh >= 32 || (kv[i] >> pre_sh) == pre);
                if (match) atomicAdd(&hist[((kv[i] >> sh) & ((1u << kBitsR) - 1u)) * kCopies + copy], 1u);
            }
        }
        __syncthreads();
    };
    uint32_t k1, k2, q;
    round(std::integral_constant<int, 8>{}, std::integral_constant<int, 16>{}, 24, 0u, 32, copy16);
    const uint32_t b0 = find_bin_from_top<256, 16>(hist, (uint32_t)Bp, &k1, scan_lds, s_res);
    round(std::integral_constant<int, 12>{}, std::integral_constant<int, 4>{}, 12, b0, 24, copy4);
    const uint32_t b1 = find_bin_from_top<4096, 4>(hist, k1, &k2, scan_lds, s_res);
    const uint32_t pre2 = (b0 << 12) | b1;  // bits 31..12
    round(std::integral_constant<int, 12>{}, std::integral_constant<int, 4>{}, 0, pre2, 12, copy4);
    const uint32_t b2 = find_bin_from_top<4096, 4>(hist, k2, &q, scan_lds, s_res);
    const uint32_t T = (pre2 << 12) | b2;  // the B'-th largest key; q of the keys equal to T fit

    // ---- ordered compaction -------------------------------------------------------
    int32_t* idx_h = idx_out + (size_t)h * Bp;
    uint32_t out_pos = 0, eq_seen = 0;
    for (int c = 0; c < nch; ++c) {
        uint32_t kv[kKpt];
        load_keys(c, kv);
        const int j0 = c * kChunk + x0;
        // One scan of both counts (keys > T, keys == T), 16 bits each: a
        // chunk holds fewer than 2^16 keys.  The equal keys are kept in
        // token order, the first q of the head, so the keys this thread
        // keeps land after the greater keys before it and after the kept
        // equal keys before it.
        uint32_t ngt = 0, neq = 0;
#pragma unroll
        for (int i = 0; i < kKpt; ++i) {
            ngt += (j0 + i < L && kv[i] > T);
            neq += (j0 + i < L && kv[i] == T);
        }
        uint32_t tot;
        const uint32_t before = block_exclusive_scan(ngt | (neq << 16), scan_lds, &tot);
        const uint32_t gt_before = before & 0xffffu, eq_before = before >> 16;
        const uint32_t tot_gt = tot & 0xffffu, tot_eq = tot >> 16;
        const uint32_t eq_kept_before = min(eq_seen + eq_before, q) - min(eq_seen, q);
        const uint32_t tot_sel = tot_gt + min(eq_seen + tot_eq, q) - min(eq_seen, q);
        uint32_t eq_rank = eq_seen + eq_before;
        // kept indices go to their slots of this chunk's output in area A,
        // then out with coalesced stores
        uint32_t pos = gt_before + eq_kept_before;
#pragma unroll
        for (int i = 0; i < kKpt; ++i) {
            if (j0 + i < L) {
                bool s = kv[i] > T;
                if (kv[i] == T) { s = eq_rank < q; ++eq_rank; }
                if (s) area_a[pos++] = (uint32_t)(j0 + i);
            }
        }
        __syncthreads();
        for (uint32_t i = tid; i < tot_sel; i += kSelThreads)
            if (out_pos + i < (uint32_t)Bp) idx_h[out_pos + i] = (int32_t)area_a[i];  // always true when the counts agree
        __syncthreads();
        out_pos += tot_sel;
        eq_seen += tot_eq;
    }
}

// ---- selection split over several workgroups per head ----------------------------------
// For heads longer than one chunk the same exact selection runs as five
// launches of G workgroups per head, each workgroup owning S <= 4096
// consecutive keys [g S, g S + S):
//   keys:    pool + score + order-preserving key of its keys, written to the
//            workspace, and the workgroup's 256-bin histogram of key bits
//            31..24;
//   round R (R = 1, 2, 3): the head's histogram of the previous round (the
//            sum of the G partial ones, in workgroup order) gives the bin of
//            the B'-th largest key among those matching the prefix found so
//            far, so the prefix grows by 8 bits; the workgroup writes its
//            256-bin histogram of the next 8 bits of its keys that match it.
//            Round 3 also writes, per workgroup, how many of its keys lie
//            above the 24-bit prefix and its suffix counts per low-8-bit bin,
//            so the compaction counts the keys of earlier workgroups above
//            and at the threshold with two reads each;
//   compact: the threshold key T and the number q of keys equal to T that
//            fit come from the head's round-3 histogram; the workgroup's
//            output offset is the kept keys of the earlier workgroups, and its
//            kept indices (every key > T, the equal keys while fewer than q
//            lie before them in token order) go out ascending.
// Integer counts only, no atomics outside LDS: deterministic.  Separate
// launches order the phases (no grid barrier, no spin-wait); every small
// global read of a phase is issued before any is waited for.
constexpr int kMT = 512;                  // threads per workgroup
constexpr int kMWaves = kMT / kWave;
constexpr int kMKpt = 8;                  // consecutive keys per thread
constexpr int kMMaxKeys = kMT * kMKpt;    // 4096: most keys one workgroup owns
constexpr int kR0Copies = 16;             // LDS copies of each round-0 bin (scores share their top bits)
constexpr int kRCopies = 4;               // LDS copies of each later bin
constexpr int kCum = 260;                 // per-workgroup suffix counts (257 used)
static_assert(kMMaxKeys < 65536, "packed 16-bit counts of one workgroup");

// Workspace of the split selection, per head h and workgroup g.
struct MselWs {
    uint32_t* keys;     // [H][L] order-preserving keys
    uint32_t* hist[4];  // [H][G][256] per-workgroup histograms of rounds 0..3
    uint32_t* above;    // [H][G] keys above the 24-bit prefix per workgroup
    uint32_t* cum3;     // [H][G][kCum] suffix counts of the prefix-matching keys per low-8-bit bin
    uint32_t* state;    // [H][4][2] (prefix, rank in its bin) after rounds 1..3
};

// Work item of a split-selection workgroup: (head, workgroup of the head).
__device__ __forceinline__ bool msel_item(int H, int G, int& h, int& g) {
    const int item = xcd_item((int)(gridDim.x / 8u));
    if (item >= H * G) return false;
    h = item / G;
    g = item % G;
    return true;
}

// tot[256] = the head's histogram of a round: the sum of its G per-workgroup
// rows, in workgroup order per bin.  Thread t adds 4 bins (column t % 64) of
// the rows w = t/64, t/64 + 8, ... (loads issued four at a time), then the
// eight partial sums per bin are added.
__device__ __forceinline__ void msel_sum_rows(const uint32_t* __restrict__ rows, int G, uint32_t* part,
                                              uint32_t* tot) {
    const int tid = threadIdx.x, col = tid & 63, w0 = tid >> 6;
    const uint4* r4 = reinterpret_cast<const uint4*>(rows);
    uint4 acc = make_uint4(0, 0, 0, 0);
    int w = w0;
    for (; w + 24 < G; w += 32) {
        const uint4 a = r4[(size_t)w * 64 + col], b = r4[(size_t)(w + 8) * 64 + col];
        const uint4 c = r4[(size_t)(w + 16) * 64 + col], d = r4[(size_t)(w + 24) * 64 + col];
        acc.x += a.x + b.x + c.x + d.x; acc.y += a.y + b.y + c.y + d.y;
        acc.z += a.z + b.z + c.z + d.z; acc.w += a.w + b.w + c.w + d.w;
    }
    for (; w < G; w += 8) {
        const uint4 a = r4[(size_t)w * 64 + col];
        acc.x += a.x; acc.y += a.y; acc.z += a.z; acc.w += a.w;
    }
    reinterpret_cast<uint4*>(part)[w0 * 64 + col] = acc;
    __syncthreads();
    if (tid < 256) {
        uint32_t c = 0;
#pragma unroll
        for (int k = 0; k < 8; ++k) c += part[k * 256 + tid];
        tot[tid] = c;
    }
    __syncthreads();
}

template <bool kFromImp>
__global__ __launch_bounds__(kMT) void msel_keys_kernel(const float* __restrict__ src, int nsrc,
                                                        const float* __restrict__ r,
                                                        const float2* __restrict__ red_part, int nbr, float lam,
                                                        int hw, float* __restrict__ score_out,
                                                        float* __restrict__ imp_pooled_out,
                                                        float* __restrict__ red_out, int H, int L, int G, int S,
                                                        MselWs ws) {
    // it[kMaxHalo + x] = importance of key j0 + x (x in [-kMaxHalo, S + kMaxHalo),
    // -inf outside [0, L)); kt[x]: r (or the score) of key j0 + x, then its key
    __shared__ __align__(16) float it[kMMaxKeys + 2 * kMaxHalo];
    __shared__ __align__(16) uint32_t kt[kMMaxKeys];
    __shared__ uint32_t hist[256 * kR0Copies];
    __shared__ float2 wstat[kMWaves];
    int h, g;
    if (!msel_item(H, G, h, g)) return;
    const int tid = threadIdx.x;
    const int j0 = g * S, n = min(S, L - j0);
    const size_t hL = (size_t)h * L;
    const size_t plane = (size_t)H * L;

    // every global read of the phase first: r (or the scores), the
    // importance with its halo, the redundancy softmax partials
    const float* rs = (kFromImp ? r : src) + hL + j0;
    float vr[kMKpt];
#pragma unroll
    for (int q = 0; q < kMKpt; ++q) {
        const int i = tid + q * kMT;
        vr[q] = i < n ? rs[i] : 0.f;
    }
    constexpr int kQa = (kMMaxKeys + 2 * kMaxHalo + kMT - 1) / kMT;
    float vi[kQa];
    float M = -1e30f, Sm = 0.f;
    if constexpr (kFromImp) {
#pragma unroll
        for (int q = 0; q < kQa; ++q) {
            const int i = tid + q * kMT, j = j0 - kMaxHalo + i;
            vi[q] = (i < n + 2 * kMaxHalo && j >= 0 && j < L) ? src[hL + j] : -INFINITY;
        }
        for (int pl = 1; pl < nsrc; ++pl) {
#pragma unroll
            for (int q = 0; q < kQa; ++q) {
                const int i = tid + q * kMT, j = j0 - kMaxHalo + i;
                if (i < n + 2 * kMaxHalo && j >= 0 && j < L) vi[q] += src[pl * plane + hL + j];
            }
        }
        // softmax statistics of r: (max of r log2 e, sum 2^{r log2 e - max}) over
        // the head's partials, four loads in flight per thread
        const float2* rp = red_part + (size_t)h * nbr;
        int i = tid;
        for (; i + 3 * kMT < nbr; i += 4 * kMT) {
            const float2 a = rp[i], b = rp[i + kMT], c = rp[i + 2 * kMT], d = rp[i + 3 * kMT];
            lse2_merge(M, Sm, a.x, a.y);
            lse2_merge(M, Sm, b.x, b.y);
            lse2_merge(M, Sm, c.x, c.y);
            lse2_merge(M, Sm, d.x, d.y);
        }
        for (; i < nbr; i += kMT) {
            const float2 a = rp[i];
            lse2_merge(M, Sm, a.x, a.y);
        }
    }
    for (int b = tid; b < 256 * kR0Copies; b += kMT) hist[b] = 0u;
#pragma unroll
    for (int q = 0; q < kMKpt; ++q) {
        const int i = tid + q * kMT;
        if (i < n) kt[i] = __float_as_uint(vr[q]);
    }
    if constexpr (kFromImp) {
#pragma unroll
        for (int q = 0; q < kQa; ++q) {
            const int i = tid + q * kMT;
            if (i < n + 2 * kMaxHalo) it[i] = vi[q];
        }
#pragma unroll
        for (int o = kWave / 2; o > 0; o >>= 1) {
            const float m2 = __shfl_xor(M, o, kWave), s2 = __shfl_xor(Sm, o, kWave);
            lse2_merge(M, Sm, m2, s2);
        }
        if ((tid & (kWave - 1)) == 0) wstat[tid / kWave] = make_float2(M, Sm);
    }
    __syncthreads();
    float invS = 0.f;
    if constexpr (kFromImp) {
        M = wstat[0].x;
        Sm = wstat[0].y;
#pragma unroll
        for (int w = 1; w < kMWaves; ++w) lse2_merge(M, Sm, wstat[w].x, wstat[w].y);
        invS = 1.0f / Sm;
    }

    const int x0 = tid * kMKpt;
    const uint32_t copy = tid & (kR0Copies - 1);
    float pooled[kMKpt];
    if constexpr (kFromImp) {
        if (hw <= kRegHalo) {
            // the window of this thread's 8 keys, 16 values, as four 16-byte
            // LDS reads (kMaxHalo - kRegHalo + x0 is a multiple of 4)
            float v[kMKpt + 2 * kRegHalo];
            const float4* w4 = reinterpret_cast<const float4*>(it + kMaxHalo - kRegHalo + x0);
#pragma unroll
            for (int q = 0; q < (kMKpt + 2 * kRegHalo) / 4; ++q) {
                const float4 f = w4[q];
                v[4 * q] = f.x; v[4 * q + 1] = f.y; v[4 * q + 2] = f.z; v[4 * q + 3] = f.w;
            }
#pragma unroll
            for (int i = 0; i < kMKpt; ++i) {
                float p = v[kRegHalo + i];
#pragma unroll
                for (int o = 1; o <= kRegHalo; ++o)
                    if (o <= hw) p = fmaxf(p, fmaxf(v[kRegHalo + i - o], v[kRegHalo + i + o]));
                pooled[i] = p;
            }
        } else {
#pragma unroll
            for (int i = 0; i < kMKpt; ++i) {
                const float* t = it + kMaxHalo + x0 + i;
                float p = t[0];
                for (int o = 1; o <= hw; ++o) p = fmaxf(p, fmaxf(t[-o], t[o]));
                pooled[i] = p;
            }
        }
    }
    uint32_t raw[kMKpt], kout[kMKpt];
#pragma unroll
    for (int q = 0; q < kMKpt / 4; ++q) {  // this thread's 8 values, two 16-byte LDS reads
        const uint4 u = reinterpret_cast<const uint4*>(kt + x0)[q];
        raw[4 * q] = u.x; raw[4 * q + 1] = u.y; raw[4 * q + 2] = u.z; raw[4 * q + 3] = u.w;
    }
#pragma unroll
    for (int i = 0; i < kMKpt; ++i) {
        const int x = x0 + i;
        kout[i] = 0u;
        if (x < n) {
            const float v = __uint_as_float(raw[i]);
            float sc = v;
            if constexpr (kFromImp) {
                const float red = exp2_hw(fmaf(v, kLog2e, -M)) * invS;
                sc = lam * pooled[i] - (1.0f - lam) * red;
                const size_t j = hL + j0 + x;
                if (score_out) score_out[j] = sc;
                if (imp_pooled_out) imp_pooled_out[j] = pooled[i];
                if (red_out) red_out[j] = red;
            }
            const uint32_t key = order_key(sc);
            kout[i] = key;
            atomicAdd(&hist[(key >> 24) * kR0Copies + copy], 1u);
        }
    }
#pragma unroll
    for (int q = 0; q < kMKpt / 4; ++q)  // this thread's own slots
        reinterpret_cast<uint4*>(kt + x0)[q] = make_uint4(kout[4 * q], kout[4 * q + 1], kout[4 * q + 2], kout[4 * q + 3]);
    __syncthreads();
    uint32_t* kg = ws.keys + hL + j0;
#pragma unroll
    for (int q = 0; q < kMKpt; ++q) {
        const int i = tid + q * kMT;
        if (i < n) kg[i] = kt[i];
    }
    if (tid < 256) {
        uint32_t c = 0;
#pragma unroll
        for (int cp = 0; cp < kR0Copies; ++cp) c += hist[tid * kR0Copies + cp];
        ws.hist[0][((size_t)h * G + g) * 256 + tid] = c;
    }
}

// Round R = 1, 2, 3: the bin of the previous round's head histogram that
// holds the B'-th largest key extends the prefix by 8 bits; the workgroup's
// histogram of the next 8 bits of its keys that match the new prefix.
template <int R>
__global__ __launch_bounds__(kMT) void msel_round_kernel(int H, int L, int G, int S, int Bp, MselWs ws) {
    constexpr int kShift = 24 - 8 * R;   // the bits this round counts: (key >> kShift) & 0xff
    __shared__ uint32_t hist[256 * kRCopies];
    __shared__ __align__(16) uint32_t part[8 * 256];
    __shared__ uint32_t tot[256];
    __shared__ uint32_t scan_lds[kMWaves];
    __shared__ uint32_t s_res[2];
    int h, g;
    if (!msel_item(H, G, h, g)) return;
    const int tid = threadIdx.x;
    const int j0 = g * S, n = min(S, L - j0);
    const uint32_t* kg = ws.keys + (size_t)h * L + j0;
    uint32_t kv[kMKpt];
#pragma unroll
    for (int q = 0; q < kMKpt; ++q) {
        const int i = tid + q * kMT;
        kv[q] = i < n ? kg[i] : 0u;
    }
    // prefix and rank so far (round 1: none, rank B')
    const uint32_t P0 = R == 1 ? 0u : ws.state[(h * 4 + R - 1) * 2 + 0];
    const uint32_t k0 = R == 1 ? (uint32_t)Bp : ws.state[(h * 4 + R - 1) * 2 + 1];
    for (int b = tid; b < 256 * kRCopies; b += kMT) hist[b] = 0u;
    msel_sum_rows(ws.hist[R - 1] + (size_t)h * G * 256, G, part, tot);
    uint32_t k1;
    const uint32_t bin = find_bin_from_top<256, 1, kMT>(tot, k0, &k1, scan_lds, s_res);
    const uint32_t P = (P0 << 8) | bin;  // the top 8 R bits of the threshold
    const uint32_t copy = tid & (kRCopies - 1);
    uint32_t above = 0;
#pragma unroll
    for (int q = 0; q < kMKpt; ++q) {
        const int i = tid + q * kMT;
        if (i < n) {
            const uint32_t p = kv[q] >> (kShift + 8);
            if (p == P) atomicAdd(&hist[((kv[q] >> kShift) & 0xffu) * kRCopies + copy], 1u);
            if (R == 3) above += p > P;
        }
    }
    __syncthreads();
    if constexpr (R < 3) {
        if (tid < 256) {
            uint32_t c = 0;
#pragma unroll
            for (int cp = 0; cp < kRCopies; ++cp) c += hist[tid * kRCopies + cp];
            ws.hist[R][((size_t)h * G + g) * 256 + tid] = c;
        }
    } else {
        // thread t < 256 owns bin 255 - t: suffix counts by a scan in
        // descending bin order
        uint32_t c = 0;
        if (tid < 256) {
#pragma unroll
            for (int cp = 0; cp < kRCopies; ++cp) c += hist[(255 - tid) * kRCopies + cp];
            ws.hist[3][((size_t)h * G + g) * 256 + 255 - tid] = c;
        }
        uint32_t t1;
        const uint32_t before = block_exclusive_scan<kMT>(c, scan_lds, &t1);
        uint32_t* cum = ws.cum3 + ((size_t)h * G + g) * kCum;
        if (tid < 256) cum[255 - tid] = before + c;  // prefix-matching keys with low 8 bits >= the bin
        if (tid == 0) cum[256] = 0u;
        uint32_t t2;
        (void)block_exclusive_scan<kMT>(above, scan_lds, &t2);
        if (tid == 0) ws.above[(size_t)h * G + g] = t2;
    }
    if (g == 0 && tid == 0) {
        ws.state[(h * 4 + R) * 2 + 0] = P;
        ws.state[(h * 4 + R) * 2 + 1] = k1;
    }
}

__global__ __launch_bounds__(kMT) void msel_compact_kernel(int H, int L, int G, int S, int Bp, MselWs ws,
                                                           int32_t* __restrict__ idx_out) {
    __shared__ __align__(16) uint32_t part[8 * 256];
    __shared__ uint32_t tot[256];
    __shared__ __align__(16) uint32_t kt[kMMaxKeys];
    __shared__ uint32_t scan_lds[kMWaves];
    __shared__ uint32_t s_res[2];
    int h, g;
    if (!msel_item(H, G, h, g)) return;
    const int tid = threadIdx.x;
    const int j0 = g * S, n = min(S, L - j0);
    const uint32_t* kg = ws.keys + (size_t)h * L + j0;
    uint32_t kq[kMKpt];
#pragma unroll
    for (int q = 0; q < kMKpt; ++q) {
        const int i = tid + q * kMT;
        kq[q] = i < n ? kg[i] : 0u;
    }
    const uint32_t P3 = ws.state[(h * 4 + 3) * 2 + 0], k3 = ws.state[(h * 4 + 3) * 2 + 1];
    // keys above the 24-bit prefix and suffix counts of the earlier workgroups
    // (read before the bin is known: both candidate entries come later)
    msel_sum_rows(ws.hist[3] + (size_t)h * G * 256, G, part, tot);
    uint32_t q;
    const uint32_t b3 = find_bin_from_top<256, 1, kMT>(tot, k3, &q, scan_lds, s_res);
    const uint32_t T = (P3 << 8) | b3;  // the B'-th largest key; q of the keys equal to T fit
    uint32_t gt_p = 0, eq_p = 0;
    for (int w = tid; w < g; w += kMT) {
        const uint32_t* cum = ws.cum3 + ((size_t)h * G + w) * kCum;
        const uint32_t hi = cum[b3 + 1];
        gt_p += ws.above[(size_t)h * G + w] + hi;
        eq_p += cum[b3] - hi;
    }
#pragma unroll
    for (int qq = 0; qq < kMKpt; ++qq) {
        const int i = tid + qq * kMT;
        if (i < n) kt[i] = kq[qq];
    }
    uint32_t gt_before, eq_before;
    (void)block_exclusive_scan<kMT>(gt_p, scan_lds, &gt_before);  // (its barriers also publish kt)
    (void)block_exclusive_scan<kMT>(eq_p, scan_lds, &eq_before);
    // this thread's consecutive keys, in token order
    const int x0 = tid * kMKpt;
    uint32_t kv[kMKpt];
    uint32_t ngt = 0, neq = 0;
#pragma unroll
    for (int q = 0; q < kMKpt / 4; ++q) {  // two 16-byte LDS reads
        const uint4 u = reinterpret_cast<const uint4*>(kt + x0)[q];
        kv[4 * q] = u.x; kv[4 * q + 1] = u.y; kv[4 * q + 2] = u.z; kv[4 * q + 3] = u.w;
    }
#pragma unroll
    for (int i = 0; i < kMKpt; ++i) {
        ngt += (x0 + i < n && kv[i] > T);
        neq += (x0 + i < n && kv[i] == T);
    }
    uint32_t totc;
    const uint32_t before = block_exclusive_scan<kMT>(ngt | (neq << 16), scan_lds, &totc);  // also orders kt's reuse
    const uint32_t gt_b = before & 0xffffu, eq_b = before >> 16;
    const uint32_t tot_gt = totc & 0xffffu, tot_eq = totc >> 16;
    const uint32_t eq_kept_b = min(eq_before + eq_b, q) - min(eq_before, q);
    const uint32_t tot_sel = tot_gt + min(eq_before + tot_eq, q) - min(eq_before, q);
    uint32_t eq_rank = eq_before + eq_b;
    uint32_t pos = gt_b + eq_kept_b;
#pragma unroll
    for (int i = 0; i < kMKpt; ++i) {
        if (x0 + i < n) {
            bool keep = kv[i] > T;
            if (kv[i] == T) { keep = eq_rank < q; ++eq_rank; }
            if (keep) kt[pos++] = (uint32_t)(j0 + x0 + i);
        }
    }
    __syncthreads();
    const uint32_t base = gt_before + min(eq_before, q);
    int32_t* idx_h = idx_out + (size_t)h * Bp;
    for (uint32_t i = tid; i < tot_sel; i += kMT)
        if (base + i < (uint32_t)Bp) idx_h[base + i] = (int32_t)kt[i];  // always true when the counts agree
}

// K_out[h][b] = K[h][idx[h][b]], V likewise: 16 bytes per lane, one row per
// kRowBytes/16 lanes, one kept row per lane group (16 rows per 256-thread
// block for bf16 rows of 128).  Rows are read and written once, with
// non-temporal accesses.  One 16-byte load of K and one of V per lane, in many
// small blocks, measured faster than more loads in flight per lane (long
// video: 182.4 -> 179.7 us for select + gather against two rows per lane
// group; a plain streaming copy of the same bytes: 6.50 TB/s with one load per
// lane, 6.13 with two or four).  With pos_out, the tokens' positions follow
// them: pos_out[h][b] = pos[h][idx[h][b]].  Head strides: ld_in rows for K, V
// and pos, ld_out rows for K_out, V_out and pos_out (L and Bp when the
// tensors are dense).
constexpr int kThreads = 256;
template <int DT, int D> constexpr int gather_rows() { return kThreads / (D * Elem<DT>::kBytes / 16); }

// kKeepAll: every row is kept (B' = L): the kernel writes idx[h][b] = b
// itself instead of reading it.
template <int DT, int D, bool kKeepAll>
__global__ __launch_bounds__(kThreads) void gather_rows_kernel(int32_t* __restrict__ idx, int L, int Bp,
                                                               const void* __restrict__ K, const void* __restrict__ V,
                                                               void* __restrict__ K_out, void* __restrict__ V_out,
                                                               const int32_t* __restrict__ pos,
                                                               int32_t* __restrict__ pos_out, int ld_in, int ld_out) {
    constexpr int kRowBytes = D * Elem<DT>::kBytes;
    constexpr int kTpr = kRowBytes / 16;     // lanes per row
    const int h = blockIdx.y;
    const int b = blockIdx.x * gather_rows<DT, D>() + threadIdx.x / kTpr;
    const int e = threadIdx.x % kTpr;
    if (b >= Bp) return;
    int j;
    if constexpr (kKeepAll) {
        j = b;
        if (e == 0) idx[(size_t)h * Bp + b] = b;
    } else {
        j = idx[(size_t)h * Bp + b];
    }
    if ((unsigned)j >= (unsigned)L) return;  // never, for indices the selection wrote
    const size_t src = (size_t)h * ld_in + j, dst = (size_t)h * ld_out + b;
    const uint4 kv = load_stream16(static_cast<const char*>(K) + src * kRowBytes + e * 16);
    const uint4 vv = load_stream16(static_cast<const char*>(V) + src * kRowBytes + e * 16);
    store_stream16(static_cast<char*>(K_out) + dst * kRowBytes + e * 16, kv);
    store_stream16(static_cast<char*>(V_out) + dst * kRowBytes + e * 16, vv);
    if (pos_out != nullptr && e == 0) pos_out[dst] = pos[src];
}

template <int DT, int D>
hipError_t gather_launch(const int32_t* idx, int H, int L, int Bp, const void* K, const void* V, void* K_out,
                         void* V_out, const int32_t* pos, int32_t* pos_out, hipStream_t s, int32_t* idx_keep_all,
                         int ld_in, int ld_out) {
    constexpr int kRows = gather_rows<DT, D>();
    const dim3 grid((Bp + kRows - 1) / kRows, H);
    if (idx_keep_all != nullptr)
        hipLaunchKernelGGL((gather_rows_kernel<DT, D, true>), grid, dim3(kThreads), 0, s, idx_keep_all, L, Bp, K, V,
                           K_out, V_out, pos, pos_out, ld_in, ld_out);
    else
        hipLaunchKernelGGL((gather_rows_kernel<DT, D, false>), grid, dim3(kThreads), 0, s, const_cast<int32_t*>(idx),
                           L, Bp, K, V, K_out, V_out, pos, pos_out, ld_in, ld_out);
    return hipGetLastError();
}

struct MselPlan {
    int G, S;  // workgroups per head and keys per workgroup; G == 0: one workgroup per head
};

// Heads of one chunk keep the one-workgroup kernel (its keys stay in LDS
// between the passes).  Longer heads split into G workgroups of S <= 4096
// consecutive keys: at least 1024 keys each, and enough workgroups for about
// three per compute unit of a 256-CU device (one round of the grid) when the
// heads are few.
MselPlan msel_plan(int H, int L) {
    if (L <= kChunk) return MselPlan{0, 0};
    long long G = (L + kMMaxKeys - 1) / kMMaxKeys;
    const long long g_fill = 768 / H, g_max = (L + 1023) / 1024;
    const long long g_want = g_fill < g_max ? g_fill : g_max;
    if (g_want > G) G = g_want;
    const int S = (int)((L + G - 1) / G);
    return MselPlan{(int)((L + S - 1) / S), S};  // every workgroup non-empty
}

constexpr size_t kWsAlign = 256;
size_t ws_up(size_t x) { return (x + kWsAlign - 1) / kWsAlign * kWsAlign; }

// Layout of the selection workspace: keys, then (split plans only) the four
// histogram arrays, the counts and the per-head state.  Offsets in bytes;
// [9] = total.
void msel_offsets(int H, int L, const MselPlan& mp, size_t (&o)[10]) {
    const size_t h = (size_t)H, G = (size_t)mp.G;
    size_t x = 0;
    o[0] = x; x = ws_up(x + h * (size_t)L * 4);  // keys
    if (mp.G > 0) {
        for (int r = 0; r < 4; ++r) { o[1 + r] = x; x = ws_up(x + h * G * 256 * 4); }
        o[5] = x; x = ws_up(x + h * G * 4);
        o[6] = x; x = ws_up(x + h * G * kCum * 4);
        o[7] = x; x = ws_up(x + h * 4 * 2 * 4);
    } else {
        for (int i = 1; i < 8; ++i) o[i] = x;
    }
    o[8] = x;
    o[9] = x;
}

MselWs msel_carve(void* base, int H, int L, const MselPlan& mp) {
    size_t o[10];
    msel_offsets(H, L, mp, o);
    auto at = [&](int i) { return reinterpret_cast<uint32_t*>(static_cast<char*>(base) + o[i]); };
    return MselWs{at(0), {at(1), at(2), at(3), at(4)}, at(5), at(6), at(7)};
}

}  // namespace

size_t sel_ws_bytes(int H, int L) {
    const MselPlan mp = msel_plan(H, L);
    size_t o[10];
    msel_offsets(H, L, mp, o);
    return o[9];
}

bool sel_grid_fits(int H, int L) {
    const MselPlan mp = msel_plan(H, L);
    const long long wgs = ((long long)H * mp.G + 7) / 8 * 8;
    return wgs * kMT < (1LL << 32);
}

hipError_t launch_sel_head(const float* src, int nsrc, const float* r, const float2* red_part, int nbr, float lam,
                           int w, float* score_out, float* imp_pooled_out, float* red_out, uint32_t* keys, int H,
                           int L, int Bp, int32_t* idx_out, hipStream_t s) {
    // 16-byte loads when a head fits one chunk and every head's rows of
    // every input start 16-byte aligned (L a multiple of 4, aligned bases).
    // Heads of several chunks keep the 4-byte loads: measured on the
    // long-video shape, the 16-byte form was slower there (171.0 against
    // 166.5 us), against 27.0 -> 26.0 us on the MAGI-like shape.
    const MselPlan mp = msel_plan(H, L);
    if (mp.G > 0) {
        const MselWs ws = msel_carve(keys, H, L, mp);
        const dim3 grid((unsigned)(((long long)H * mp.G + 7) / 8 * 8));
        if (r != nullptr)
            hipLaunchKernelGGL(msel_keys_kernel<true>, grid, dim3(kMT), 0, s, src, nsrc, r, red_part, nbr, lam,
                               (w - 1) / 2, score_out, imp_pooled_out, red_out, H, L, mp.G, mp.S, ws);
        else
            hipLaunchKernelGGL(msel_keys_kernel<false>, grid, dim3(kMT), 0, s, src, 1, nullptr, nullptr, 0, 0.f, 0,
                               nullptr, nullptr, nullptr, H, L, mp.G, mp.S, ws);
        hipLaunchKernelGGL(msel_round_kernel<1>, grid, dim3(kMT), 0, s, H, L, mp.G, mp.S, Bp, ws);
        hipLaunchKernelGGL(msel_round_kernel<2>, grid, dim3(kMT), 0, s, H, L, mp.G, mp.S, Bp, ws);
        hipLaunchKernelGGL(msel_round_kernel<3>, grid, dim3(kMT), 0, s, H, L, mp.G, mp.S, Bp, ws);
        hipLaunchKernelGGL(msel_compact_kernel, grid, dim3(kMT), 0, s, H, L, mp.G, mp.S, Bp, ws, idx_out);
        return hipGetLastError();
    }
    const bool vec = L <= kChunk && L % 4 == 0 && (reinterpret_cast<uintptr_t>(src) & 15) == 0 &&
                     (r == nullptr || (reinterpret_cast<uintptr_t>(r) & 15) == 0);
    if (r != nullptr) {
        auto kern = vec ? sel_head_kernel<true, true> : sel_head_kernel<true, false>;
        hipLaunchKernelGGL(kern, dim3(H), dim3(kSelThreads), 0, s, src, nsrc, r, red_part, nbr, lam, (w - 1) / 2,
                           score_out, imp_pooled_out, red_out, keys, L, Bp, idx_out);
    } else {
        auto kern = vec ? sel_head_kernel<false, true> : sel_head_kernel<false, false>;
        hipLaunchKernelGGL(kern, dim3(H), dim3(kSelThreads), 0, s, src, 1, nullptr, nullptr, 0, 0.f, 0, nullptr,
                           nullptr, nullptr, keys, L, Bp, idx_out);
    }
    return hipGetLastError();
}

hipError_t launch_gather(int dt, int d, const int32_t* idx, int H, int L, int Bp, const void* K, const void* V,
                         void* K_out, void* V_out, hipStream_t s, const int32_t* pos, int32_t* pos_out,
                         int32_t* idx_keep_all, int ld_in, int ld_out) {
    if (ld_in < L) ld_in = L;
    if (ld_out < Bp) ld_out = Bp;
#define FC_GATHER(DT_, D_) \
    gather_launch<DT_, D_>(idx, H, L, Bp, K, V, K_out, V_out, pos, pos_out, s, idx_keep_all, ld_in, ld_out)
    if (dt == kBF16) return d == 128 ? FC_GATHER(kBF16, 128) : FC_GATHER(kBF16, 64);
    return d == 128 ? FC_GATHER(kF32, 128) : FC_GATHER(kF32, 64);
#undef FC_GATHER
}

}  // namespace fc
