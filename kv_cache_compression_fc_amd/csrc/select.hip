// Joint score, per-head top-B selection and K/V compaction, "Flow Caching for
// Autoregressive Video Generation" (papernotes digest), Key designs item 3:
//     Imp~_j  = max{Imp_k : |k - j| <= (w-1)/2, 0 <= k < L}      (1-D max-pool)
//     Red_j   = e^{r_j - max r} / sum_k e^{r_k - max r}           (softmax over tokens)
//     Score_j = lambda Imp~_j - (1 - lambda) Red_j,
// and each head keeps its B' = min(B, L) best tokens (flowchart under
// 整体框架: cache full -> joint score -> top-B per head).
//
// One 1024-thread workgroup per head does the whole selection, exactly, on
// the float32 scores.  Each score becomes an order-preserving uint32 key;
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
// re-reads them from the workspace.  No global atomics: the result is
// deterministic.  A gather kernel with one block per 32 kept rows then copies
// their K and V rows.
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

// Exclusive prefix sum over the workgroup; *total receives the sum.
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t v, uint32_t* lds, uint32_t* total) {
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
    for (int w = 0; w < kSelWaves; ++w) {
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
template <int BINS, int COPIES>
__device__ __forceinline__ uint32_t find_bin_from_top(const uint32_t* hist, uint32_t k, uint32_t* k_in_bin,
                                                      uint32_t* scan_lds, uint32_t* s_res) {
    constexpr int kPerT = BINS >= kSelThreads ? BINS / kSelThreads : 1;
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
    const uint32_t before = block_exclusive_scan(sum, scan_lds, &total);
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

// K_out[h][b] = K[h][idx[h][b]], V likewise: 16 bytes per lane, one row per
// kRowBytes/16 lanes, kGatherRows output rows per block.  Rows are read and
// written once, with non-temporal accesses.  With pos_out, the tokens'
// positions follow them: pos_out[h][b] = pos[h][idx[h][b]].
constexpr int kThreads = 256;
constexpr int kGatherRows = 32;  // measured 62.6 -> 60.0 us for select + gather (MAGI-like) against 64

// kKeepAll: every row is kept (B' = L): the kernel writes idx[h][b] = b
// itself instead of reading it.
template <int DT, int D, bool kKeepAll>
__global__ __launch_bounds__(kThreads) void gather_rows_kernel(int32_t* __restrict__ idx, int L, int Bp,
                                                               const void* __restrict__ K, const void* __restrict__ V,
                                                               void* __restrict__ K_out, void* __restrict__ V_out,
                                                               const int32_t* __restrict__ pos,
                                                               int32_t* __restrict__ pos_out) {
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
        if constexpr (kKeepAll) {
            j[i] = b < Bp ? b : -1;
            if (b < Bp && e == 0) idx[(size_t)h * Bp + b] = b;
        } else {
            j[i] = b < Bp ? idx[(size_t)h * Bp + b] : -1;
        }
    }
    uint4 kv[kSteps], vv[kSteps];
#pragma unroll
    for (int i = 0; i < kSteps; ++i) {
        if ((unsigned)j[i] < (unsigned)L) {
            kv[i] = load_stream16(Ks + (size_t)j[i] * kRowBytes);
            vv[i] = load_stream16(Vs + (size_t)j[i] * kRowBytes);
        }
    }
#pragma unroll
    for (int i = 0; i < kSteps; ++i) {
        if ((unsigned)j[i] < (unsigned)L) {
            const size_t b = (size_t)(b0 + i * kRpi);
            store_stream16(Kd + b * kRowBytes, kv[i]);
            store_stream16(Vd + b * kRowBytes, vv[i]);
            if (pos_out != nullptr && e == 0) pos_out[(size_t)h * Bp + b] = pos[(size_t)h * L + j[i]];
        }
    }
}

template <int DT, int D>
hipError_t gather_launch(const int32_t* idx, int H, int L, int Bp, const void* K, const void* V, void* K_out,
                         void* V_out, const int32_t* pos, int32_t* pos_out, hipStream_t s, int32_t* idx_keep_all) {
    const dim3 grid((Bp + kGatherRows - 1) / kGatherRows, H);
    if (idx_keep_all != nullptr)
        hipLaunchKernelGGL((gather_rows_kernel<DT, D, true>), grid, dim3(kThreads), 0, s, idx_keep_all, L, Bp, K, V,
                           K_out, V_out, pos, pos_out);
    else
        hipLaunchKernelGGL((gather_rows_kernel<DT, D, false>), grid, dim3(kThreads), 0, s, const_cast<int32_t*>(idx),
                           L, Bp, K, V, K_out, V_out, pos, pos_out);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_sel_head(const float* src, int nsrc, const float* r, const float2* red_part, int nbr, float lam,
                           int w, float* score_out, float* imp_pooled_out, float* red_out, uint32_t* keys, int H,
                           int L, int Bp, int32_t* idx_out, hipStream_t s) {
    // 16-byte loads when a head fits one chunk and every head's rows of
    // every input start 16-byte aligned (L a multiple of 4, aligned bases).
    // Heads of several chunks keep the 4-byte loads: measured on the
    // long-video shape, the 16-byte form was slower there (171.0 against
    // 166.5 us), against 27.0 -> 26.0 us on the MAGI-like shape.
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
                         int32_t* idx_keep_all) {
    if (dt == kBF16)
        return d == 128 ? gather_launch<kBF16, 128>(idx, H, L, Bp, K, V, K_out, V_out, pos, pos_out, s, idx_keep_all)
                        : gather_launch<kBF16, 64>(idx, H, L, Bp, K, V, K_out, V_out, pos, pos_out, s, idx_keep_all);
    return d == 128 ? gather_launch<kF32, 128>(idx, H, L, Bp, K, V, K_out, V_out, pos, pos_out, s, idx_keep_all)
                    : gather_launch<kF32, 64>(idx, H, L, Bp, K, V, K_out, V_out, pos, pos_out, s, idx_keep_all);
}

}  // namespace fc
