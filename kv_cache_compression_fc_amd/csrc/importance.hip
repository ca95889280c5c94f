// Importance of the clean keys, "Flow Caching for Autoregressive Video
// Generation" (papernotes digest), Key designs item 3: the attention softmax
// of the current denoising queries over the clean keys, averaged across the
// queries.  Per head h:
//     Imp_j = (1/L_q) sum_i exp(s_ij - lse_i),   s_ij = scale * q_i . k_j,
//     lse_i = log sum_j exp(s_ij).
// Two passes over Q K^T, both on bf16 MFMA (v_mfma_f32_32x32x16_bf16, fp32
// accumulate), neither materialising the L_q x L_k matrix:
//   pass 1 (imp_lse_kernel)    a workgroup owns 128 queries, streams K tiles
//                              through LDS and keeps a per-lane online
//                              (max, sum of 2^x) in base 2;
//   pass 2 (imp_colsum_kernel) a workgroup owns 128 keys, streams Q tiles and
//                              their -lse through LDS, recomputes the logits
//                              and accumulates column sums of 2^(x - lse2)
//                              in registers.  No atomics: deterministic.
// The scale is folded with log2(e) into one FMA before v_exp_f32.
#include "common.hpp"
#include "kernels.hpp"

namespace fc {

namespace {

constexpr int kThreads = 256;
constexpr int kNB = 2;                           // register-resident 32-row blocks per wave
constexpr int kRowsPerWave = 32 * kNB;
constexpr int kRowsPerBlock = 4 * kRowsPerWave;  // 256 queries (pass 1) or keys (pass 2)

// Global -> registers -> LDS staging of a ROWS x D tile of row-major data,
// 16 bytes per thread per step.  LDS rows are padded by 16 bytes so that the
// 16-byte fragment reads of 16 consecutive rows hit distinct banks.
template <int DT, int D, int ROWS>
struct TileStager {
    static constexpr int kE = Elem<DT>::kBytes;
    static constexpr int kRowBytes = D * kE;
    static constexpr int kChunksPerRow = kRowBytes / 16;
    static constexpr int kPerThread = ROWS * kChunksPerRow / kThreads;
    static constexpr int kRowStride = kRowBytes + 16;
    static constexpr int kBytes = ROWS * kRowStride;
    static_assert(ROWS * kChunksPerRow % kThreads == 0, "tile must split evenly over the block");
    uint4 regs[kPerThread];

    // rows_valid may be <= 0 or > ROWS; rows beyond it are zero-filled.
    __device__ __forceinline__ void load(const char* gtile, int rows_valid) {
#pragma unroll
        for (int i = 0; i < kPerThread; ++i) {
            const int c = threadIdx.x + kThreads * i;
            const int row = c / kChunksPerRow, col = c % kChunksPerRow;
            regs[i] = row < rows_valid
                          ? *reinterpret_cast<const uint4*>(gtile + (size_t)row * kRowBytes + col * 16)
                          : make_uint4(0, 0, 0, 0);
        }
    }
    __device__ __forceinline__ void store(char* lds) const {
#pragma unroll
        for (int i = 0; i < kPerThread; ++i) {
            const int c = threadIdx.x + kThreads * i;
            const int row = c / kChunksPerRow, col = c % kChunksPerRow;
            *reinterpret_cast<uint4*>(lds + row * kRowStride + col * 16) = regs[i];
        }
    }
};

template <int DT> constexpr int tile_rows() { return DT == kBF16 ? 64 : 32; }

// The hardware hands linear block b to XCD b % 8.  Give every XCD a
// contiguous range of logical work items, so that the blocks running together
// on one XCD share a head and a key (or query) range in that XCD's L2.
__device__ __forceinline__ int xcd_item(int per_xcd) {
    return (int)(blockIdx.x % 8u) * per_xcd + (int)(blockIdx.x / 8u);
}

template <int DT, int D>
__global__ __launch_bounds__(kThreads) void imp_lse_kernel(const void* __restrict__ Q,
                                                           const void* __restrict__ K,
                                                           float2* __restrict__ part, int Lq, int Lk,
                                                           int keys_per_split, int nsplit, int nqb,
                                                           int n_items, float c) {
    constexpr int kE = Elem<DT>::kBytes;
    constexpr int KT = tile_rows<DT>();
    constexpr int NKK = D / 16;
    using Stager = TileStager<DT, D, KT>;
    __shared__ __align__(16) char lds[2][Stager::kBytes];

    const int item = xcd_item((n_items + 7) / 8);
    if (item >= n_items) return;
    const int qblk = item % nqb, hs = item / nqb;
    const int split = hs % nsplit, h = hs / nsplit;

    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    const int half = lane >> 5;
    const int q0 = qblk * kRowsPerBlock + wave * kRowsPerWave + (lane & 31);
    const char* Qh = static_cast<const char*>(Q) + (size_t)h * Lq * D * kE;
    const char* Kh = static_cast<const char*>(K) + (size_t)h * Lk * D * kE;

    // Q^T fragments (B operand) of this wave's kNB query blocks.
    Frag8<DT> qf[kNB][NKK];
#pragma unroll
    for (int nb = 0; nb < kNB; ++nb) {
        const int q = q0 + 32 * nb;
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk) {
            if (q < Lq) qf[nb][kk].load(Qh + ((size_t)q * D + 16 * kk + 8 * half) * kE);
            else qf[nb][kk].zero();
        }
    }

    const int k_begin = split * keys_per_split;
    const int k_end = min(Lk, k_begin + keys_per_split);
    const int ntiles = (k_end - k_begin + KT - 1) / KT;

    // Per query block: this lane's keys so far, sum 2^(x - m) with x = c q.k.
    float m[kNB], s[kNB];
#pragma unroll
    for (int nb = 0; nb < kNB; ++nb) { m[nb] = -1e30f; s[nb] = 0.f; }
    Stager st;
    st.load(Kh + (size_t)k_begin * D * kE, k_end - k_begin);
    st.store(lds[0]);
    __syncthreads();
    for (int t = 0; t < ntiles; ++t) {
        const int kt0 = k_begin + t * KT;
        if (t + 1 < ntiles) st.load(Kh + (size_t)(kt0 + KT) * D * kE, k_end - (kt0 + KT));
        const char* L = lds[t & 1];
#pragma unroll
        for (int kb = 0; kb < KT / 32; ++kb) {
            if (kt0 + kb * 32 >= k_end) break;  // uniform over the block
            f32x16_t acc[kNB];
#pragma unroll
            for (int nb = 0; nb < kNB; ++nb) acc[nb] = f32x16_t{};
#pragma unroll
            for (int kk = 0; kk < NKK; ++kk) {
                Frag8<DT> a;
                a.load(L + (kb * 32 + (lane & 31)) * Stager::kRowStride + (16 * kk + 8 * half) * kE);
#pragma unroll
                for (int nb = 0; nb < kNB; ++nb) mfma16(acc[nb], a, qf[nb][kk]);
            }
            // acc[nb][r] = k_j . q with j = kt0 + 32*kb + 8*(r/4) + 4*half + r%4.
            if (kt0 + kb * 32 + 32 > k_end) {
                const int j0 = kt0 + kb * 32 + 4 * half;
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    if (j0 + 8 * (r >> 2) + (r & 3) >= k_end) {
#pragma unroll
                        for (int nb = 0; nb < kNB; ++nb) acc[nb][r] = -INFINITY;
                    }
            }
#pragma unroll
            for (int nb = 0; nb < kNB; ++nb) {
                float tmax = fmaxf(fmaxf(acc[nb][0], acc[nb][1]), acc[nb][2]);
#pragma unroll
                for (int r = 3; r < 15; r += 2) tmax = fmaxf(fmaxf(tmax, acc[nb][r]), acc[nb][r + 1]);
                tmax = fmaxf(tmax, acc[nb][15]);
                const float mn = fmaxf(m[nb], tmax * c);
                float p0 = 0.f, p1 = 0.f, p2 = 0.f, p3 = 0.f;
#pragma unroll
                for (int r = 0; r < 16; r += 4) {
                    p0 += exp2_hw(fmaf(acc[nb][r + 0], c, -mn));
                    p1 += exp2_hw(fmaf(acc[nb][r + 1], c, -mn));
                    p2 += exp2_hw(fmaf(acc[nb][r + 2], c, -mn));
                    p3 += exp2_hw(fmaf(acc[nb][r + 3], c, -mn));
                }
                s[nb] = fmaf(s[nb], exp2_hw(m[nb] - mn), (p0 + p1) + (p2 + p3));
                m[nb] = mn;
            }
        }
        if (t + 1 < ntiles) st.store(lds[(t + 1) & 1]);
        __syncthreads();
    }
#pragma unroll
    for (int nb = 0; nb < kNB; ++nb) {
        // Lanes l and l^32 hold disjoint key subsets of the same query.
        float mm = m[nb], ss = s[nb];
        const float m2 = __shfl_xor(mm, 32, kWave), s2 = __shfl_xor(ss, 32, kWave);
        lse2_merge(mm, ss, m2, s2);
        const int q = q0 + 32 * nb;
        if (lane < 32 && q < Lq) part[((size_t)h * nsplit + split) * Lq + q] = make_float2(mm, ss);
    }
}

// lse of query q in base 2 (log2 sum_j 2^(c s_ij)), merged over the key splits.
__device__ __forceinline__ float merged_lse2(const float2* __restrict__ ph, int Lq, int nsplit, int q) {
    float m = -1e30f, s = 0.f;
    for (int i = 0; i < nsplit; ++i) {
        const float2 v = ph[(size_t)i * Lq + q];
        lse2_merge(m, s, v.x, v.y);
    }
    return m + log2_hw(s);
}

// Natural-log lse of each query from the pass-1 partials.
__global__ __launch_bounds__(kThreads) void imp_lse_merge_kernel(const float2* __restrict__ part,
                                                                 float* __restrict__ lse, int Lq, int nsplit) {
    const int h = blockIdx.y;
    const int q = blockIdx.x * kThreads + threadIdx.x;
    if (q < Lq) lse[(size_t)h * Lq + q] = merged_lse2(part + (size_t)h * nsplit * Lq, Lq, nsplit, q) / kLog2e;
}

template <int DT, int D>
__global__ __launch_bounds__(kThreads) void imp_colsum_kernel(const void* __restrict__ Q,
                                                              const void* __restrict__ K,
                                                              const float* __restrict__ lse,
                                                              float* __restrict__ imp, int Lq, int Lk, int nkb,
                                                              int n_items, float c, float inv_lq) {
    constexpr int kE = Elem<DT>::kBytes;
    constexpr int QT = tile_rows<DT>();
    constexpr int NKK = D / 16;
    using Stager = TileStager<DT, D, QT>;
    __shared__ __align__(16) char lds[2][Stager::kBytes];
    __shared__ __align__(16) float nlse[2][QT];  // -lse2 of the tile's queries (-inf past L_q)

    const int item = xcd_item((n_items + 7) / 8);
    if (item >= n_items) return;
    const int kblk = item % nkb, h = item / nkb;

    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    const int half = lane >> 5;
    const int key0 = kblk * kRowsPerBlock + wave * kRowsPerWave + (lane & 31);
    const char* Qh = static_cast<const char*>(Q) + (size_t)h * Lq * D * kE;
    const char* Kh = static_cast<const char*>(K) + (size_t)h * Lk * D * kE;
    const float* lse_h = lse + (size_t)h * Lq;

    // K^T fragments (B operand) of this wave's kNB key blocks.
    Frag8<DT> kf[kNB][NKK];
#pragma unroll
    for (int nb = 0; nb < kNB; ++nb) {
        const int key = key0 + 32 * nb;
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk) {
            if (key < Lk) kf[nb][kk].load(Kh + ((size_t)key * D + 16 * kk + 8 * half) * kE);
            else kf[nb][kk].zero();
        }
    }

    const int ntiles = (Lq + QT - 1) / QT;
    float cs[kNB][4];
#pragma unroll
    for (int nb = 0; nb < kNB; ++nb) cs[nb][0] = cs[nb][1] = cs[nb][2] = cs[nb][3] = 0.f;
    Stager st;
    st.load(Qh, Lq);
    st.store(lds[0]);
    if (threadIdx.x < QT) nlse[0][threadIdx.x] = (int)threadIdx.x < Lq ? -lse_h[threadIdx.x] * kLog2e : -INFINITY;
    __syncthreads();
    for (int t = 0; t < ntiles; ++t) {
        const int qt0 = t * QT;
        float lse_next = INFINITY;
        if (t + 1 < ntiles) {
            st.load(Qh + (size_t)(qt0 + QT) * D * kE, Lq - (qt0 + QT));
            const int qn = qt0 + QT + threadIdx.x;
            if (threadIdx.x < QT && qn < Lq) lse_next = lse_h[qn];
        }
        const char* L = lds[t & 1];
        const float* NL = nlse[t & 1];
#pragma unroll
        for (int qb = 0; qb < QT / 32; ++qb) {
            f32x16_t acc[kNB];
#pragma unroll
            for (int nb = 0; nb < kNB; ++nb) acc[nb] = f32x16_t{};
#pragma unroll
            for (int kk = 0; kk < NKK; ++kk) {
                Frag8<DT> a;
                a.load(L + (qb * 32 + (lane & 31)) * Stager::kRowStride + (16 * kk + 8 * half) * kE);
#pragma unroll
                for (int nb = 0; nb < kNB; ++nb) mfma16(acc[nb], a, kf[nb][kk]);
            }
            // acc[nb][r] = q_i . k with i = qt0 + 32*qb + 8*(r/4) + 4*half + r%4.
            const float* nl = NL + qb * 32 + 4 * half;
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const float4 n = *reinterpret_cast<const float4*>(nl + 8 * g);
#pragma unroll
                for (int nb = 0; nb < kNB; ++nb) {
                    cs[nb][0] += exp2_hw(fmaf(acc[nb][4 * g + 0], c, n.x));
                    cs[nb][1] += exp2_hw(fmaf(acc[nb][4 * g + 1], c, n.y));
                    cs[nb][2] += exp2_hw(fmaf(acc[nb][4 * g + 2], c, n.z));
                    cs[nb][3] += exp2_hw(fmaf(acc[nb][4 * g + 3], c, n.w));
                }
            }
        }
        if (t + 1 < ntiles) {
            st.store(lds[(t + 1) & 1]);
            if (threadIdx.x < QT) nlse[(t + 1) & 1][threadIdx.x] = -lse_next * kLog2e;
        }
        __syncthreads();
    }
#pragma unroll
    for (int nb = 0; nb < kNB; ++nb) {
        float v = (cs[nb][0] + cs[nb][1]) + (cs[nb][2] + cs[nb][3]);
        v += __shfl_xor(v, 32, kWave);  // the other half of the queries of this key
        const int key = key0 + 32 * nb;
        if (lane < 32 && key < Lk) imp[(size_t)h * Lk + key] = v * inv_lq;
    }
}

template <int DT, int D>
hipError_t lse_launch(const void* Q, const void* K, float2* part, int H, int Lq, int Lk, const ImpPlan& p,
                      float c, hipStream_t s) {
    const int nqb = (Lq + kRowsPerBlock - 1) / kRowsPerBlock;
    const long long n_items = (long long)H * p.nsplit * nqb;
    const int blocks = (int)((n_items + 7) / 8 * 8);
    hipLaunchKernelGGL((imp_lse_kernel<DT, D>), dim3(blocks), dim3(kThreads), 0, s, Q, K, part, Lq, Lk,
                       p.keys_per_split, p.nsplit, nqb, (int)n_items, c);
    return hipGetLastError();
}

template <int DT, int D>
hipError_t colsum_launch(const void* Q, const void* K, const float* lse, float* imp, int H, int Lq, int Lk, float c,
                         hipStream_t s) {
    const int nkb = (Lk + kRowsPerBlock - 1) / kRowsPerBlock;
    const long long n_items = (long long)H * nkb;
    const int blocks = (int)((n_items + 7) / 8 * 8);
    hipLaunchKernelGGL((imp_colsum_kernel<DT, D>), dim3(blocks), dim3(kThreads), 0, s, Q, K, lse, imp, Lq, Lk, nkb,
                       (int)n_items, c, 1.0f / (float)Lq);
    return hipGetLastError();
}

}  // namespace

ImpPlan imp_plan(int H, int Lq, int Lk, int dt) {
    const int kt = dt == kBF16 ? tile_rows<kBF16>() : tile_rows<kF32>();
    const long long blocks = (long long)H * ((Lq + kRowsPerBlock - 1) / kRowsPerBlock);
    const int max_split = (Lk + 4 * kt - 1) / (4 * kt);  // keep >= 4 tiles per split
    int ns = (int)((2048 + blocks - 1) / blocks);         // ~8 blocks per CU: a short tail
    if (ns > max_split) ns = max_split;
    if (ns < 1) ns = 1;
    int tiles = (Lk + kt - 1) / kt;
    int kps = ((tiles + ns - 1) / ns) * kt;
    ns = (Lk + kps - 1) / kps;  // every split non-empty
    return ImpPlan{ns, kps};
}

hipError_t launch_imp_lse(int dt, int d, const void* Q, const void* K, float2* part, int H, int Lq, int Lk,
                          const ImpPlan& plan, float c, hipStream_t s) {
    if (dt == kBF16) return d == 128 ? lse_launch<kBF16, 128>(Q, K, part, H, Lq, Lk, plan, c, s)
                                     : lse_launch<kBF16, 64>(Q, K, part, H, Lq, Lk, plan, c, s);
    return d == 128 ? lse_launch<kF32, 128>(Q, K, part, H, Lq, Lk, plan, c, s)
                    : lse_launch<kF32, 64>(Q, K, part, H, Lq, Lk, plan, c, s);
}

hipError_t launch_imp_colsum(int dt, int d, const void* Q, const void* K, const float* lse, float* imp, int H,
                             int Lq, int Lk, float c, hipStream_t s) {
    if (dt == kBF16) return d == 128 ? colsum_launch<kBF16, 128>(Q, K, lse, imp, H, Lq, Lk, c, s)
                                     : colsum_launch<kBF16, 64>(Q, K, lse, imp, H, Lq, Lk, c, s);
    return d == 128 ? colsum_launch<kF32, 128>(Q, K, lse, imp, H, Lq, Lk, c, s)
                    : colsum_launch<kF32, 64>(Q, K, lse, imp, H, Lq, Lk, c, s);
}

hipError_t launch_imp_lse_merge(const float2* part, float* lse, int H, int Lq, int nsplit, hipStream_t s) {
    hipLaunchKernelGGL(imp_lse_merge_kernel, dim3((Lq + kThreads - 1) / kThreads, H), dim3(kThreads), 0, s, part,
                       lse, Lq, nsplit);
    return hipGetLastError();
}

}  // namespace fc
