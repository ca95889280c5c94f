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
constexpr int kRowsPerWave = 32;
constexpr int kRowsPerBlock = 4 * kRowsPerWave;  // 128 queries (pass 1) or keys (pass 2)

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

template <int DT, int D>
__global__ __launch_bounds__(kThreads) void imp_lse_kernel(const void* __restrict__ Q,
                                                           const void* __restrict__ K,
                                                           float2* __restrict__ part, int Lq, int Lk,
                                                           int keys_per_split, float c) {
    constexpr int kE = Elem<DT>::kBytes;
    constexpr int KT = tile_rows<DT>();
    constexpr int NKK = D / 16;
    using Stager = TileStager<DT, D, KT>;
    __shared__ __align__(16) char lds[2][Stager::kBytes];

    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    const int h = blockIdx.z, split = blockIdx.y, nsplit = gridDim.y;
    const int q = blockIdx.x * kRowsPerBlock + wave * kRowsPerWave + (lane & 31);
    const char* Qh = static_cast<const char*>(Q) + (size_t)h * Lq * D * kE;
    const char* Kh = static_cast<const char*>(K) + (size_t)h * Lk * D * kE;
    const int half = lane >> 5;

    // Q^T fragments (B operand): query q, depth 16*kk + 8*half .. +8.
    Frag8<DT> qf[NKK];
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
        if (q < Lq) qf[kk].load(Qh + ((size_t)q * D + 16 * kk + 8 * half) * kE);
        else qf[kk].zero();
    }

    const int k_begin = split * keys_per_split;
    const int k_end = min(Lk, k_begin + keys_per_split);
    const int ntiles = (k_end - k_begin + KT - 1) / KT;

    float m = -1e30f, s = 0.f;  // this lane's keys so far: sum 2^(x - m), x = c * q.k
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
            f32x16_t acc = {};
#pragma unroll
            for (int kk = 0; kk < NKK; ++kk) {
                Frag8<DT> a;
                a.load(L + (kb * 32 + (lane & 31)) * Stager::kRowStride + (16 * kk + 8 * half) * kE);
                mfma16(acc, a, qf[kk]);
            }
            // acc[r] = k_j . q_i with j = kt0 + 32*kb + 8*(r/4) + 4*half + r%4, i = q.
            if (kt0 + kb * 32 + 32 > k_end) {
                const int j0 = kt0 + kb * 32 + 4 * half;
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    if (j0 + 8 * (r >> 2) + (r & 3) >= k_end) acc[r] = -INFINITY;
            }
            float tmax = acc[0];
#pragma unroll
            for (int r = 1; r < 16; ++r) tmax = fmaxf(tmax, acc[r]);
            const float mn = fmaxf(m, tmax * c);
            float p0 = 0.f, p1 = 0.f, p2 = 0.f, p3 = 0.f;
#pragma unroll
            for (int r = 0; r < 16; r += 4) {
                p0 += exp2_hw(fmaf(acc[r + 0], c, -mn));
                p1 += exp2_hw(fmaf(acc[r + 1], c, -mn));
                p2 += exp2_hw(fmaf(acc[r + 2], c, -mn));
                p3 += exp2_hw(fmaf(acc[r + 3], c, -mn));
            }
            s = s * exp2_hw(m - mn) + ((p0 + p1) + (p2 + p3));
            m = mn;
        }
        if (t + 1 < ntiles) st.store(lds[(t + 1) & 1]);
        __syncthreads();
    }
    // Lanes l and l^32 hold disjoint key subsets of the same query.
    const float m2 = __shfl_xor(m, 32, kWave), s2 = __shfl_xor(s, 32, kWave);
    lse2_merge(m, s, m2, s2);
    if (lane < 32 && q < Lq) part[((size_t)h * nsplit + split) * Lq + q] = make_float2(m, s);
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

template <int DT, int D>
__global__ __launch_bounds__(kThreads) void imp_colsum_kernel(const void* __restrict__ Q,
                                                              const void* __restrict__ K,
                                                              const float2* __restrict__ part,
                                                              float* __restrict__ imp, int Lq, int Lk,
                                                              int nsplit, float c, float inv_lq) {
    constexpr int kE = Elem<DT>::kBytes;
    constexpr int QT = tile_rows<DT>();
    constexpr int NKK = D / 16;
    using Stager = TileStager<DT, D, QT>;
    __shared__ __align__(16) char lds[2][Stager::kBytes];
    __shared__ __align__(16) float nlse[2][QT];  // -lse2 of the tile's queries (-inf past L_q)

    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    const int h = blockIdx.y;
    const int key = blockIdx.x * kRowsPerBlock + wave * kRowsPerWave + (lane & 31);
    const char* Qh = static_cast<const char*>(Q) + (size_t)h * Lq * D * kE;
    const char* Kh = static_cast<const char*>(K) + (size_t)h * Lk * D * kE;
    const float2* ph = part + (size_t)h * nsplit * Lq;
    const int half = lane >> 5;

    // K^T fragments (B operand): key, depth 16*kk + 8*half .. +8.
    Frag8<DT> kf[NKK];
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
        if (key < Lk) kf[kk].load(Kh + ((size_t)key * D + 16 * kk + 8 * half) * kE);
        else kf[kk].zero();
    }

    const int ntiles = (Lq + QT - 1) / QT;
    float cs0 = 0.f, cs1 = 0.f, cs2 = 0.f, cs3 = 0.f;
    Stager st;
    st.load(Qh, Lq);
    st.store(lds[0]);
    if (threadIdx.x < QT)
        nlse[0][threadIdx.x] = threadIdx.x < Lq ? -merged_lse2(ph, Lq, nsplit, threadIdx.x) : -INFINITY;
    __syncthreads();
    for (int t = 0; t < ntiles; ++t) {
        const int qt0 = t * QT;
        float nl_next = -INFINITY;
        if (t + 1 < ntiles) {
            st.load(Qh + (size_t)(qt0 + QT) * D * kE, Lq - (qt0 + QT));
            const int qn = qt0 + QT + threadIdx.x;
            if (threadIdx.x < QT && qn < Lq) nl_next = -merged_lse2(ph, Lq, nsplit, qn);
        }
        const char* L = lds[t & 1];
        const float* NL = nlse[t & 1];
#pragma unroll
        for (int qb = 0; qb < QT / 32; ++qb) {
            f32x16_t acc = {};
#pragma unroll
            for (int kk = 0; kk < NKK; ++kk) {
                Frag8<DT> a;
                a.load(L + (qb * 32 + (lane & 31)) * Stager::kRowStride + (16 * kk + 8 * half) * kE);
                mfma16(acc, a, kf[kk]);
            }
            // acc[r] = q_i . k_key with i = qt0 + 32*qb + 8*(r/4) + 4*half + r%4.
            const float* nl = NL + qb * 32 + 4 * half;
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const float4 n = *reinterpret_cast<const float4*>(nl + 8 * g);
                cs0 += exp2_hw(fmaf(acc[4 * g + 0], c, n.x));
                cs1 += exp2_hw(fmaf(acc[4 * g + 1], c, n.y));
                cs2 += exp2_hw(fmaf(acc[4 * g + 2], c, n.z));
                cs3 += exp2_hw(fmaf(acc[4 * g + 3], c, n.w));
            }
        }
        if (t + 1 < ntiles) {
            st.store(lds[(t + 1) & 1]);
            if (threadIdx.x < QT) nlse[(t + 1) & 1][threadIdx.x] = nl_next;
        }
        __syncthreads();
    }
    float cs = (cs0 + cs1) + (cs2 + cs3);
    cs += __shfl_xor(cs, 32, kWave);  // the other half of the queries of this key
    if (lane < 32 && key < Lk) imp[(size_t)h * Lk + key] = cs * inv_lq;
}

template <int DT, int D>
hipError_t lse_launch(const void* Q, const void* K, float2* part, int H, int Lq, int Lk, const ImpPlan& p,
                      float c, hipStream_t s) {
    dim3 grid((Lq + kRowsPerBlock - 1) / kRowsPerBlock, p.nsplit, H);
    hipLaunchKernelGGL((imp_lse_kernel<DT, D>), grid, dim3(kThreads), 0, s, Q, K, part, Lq, Lk,
                       p.keys_per_split, c);
    return hipGetLastError();
}

template <int DT, int D>
hipError_t colsum_launch(const void* Q, const void* K, const float2* part, float* imp, int H, int Lq,
                         int Lk, int nsplit, float c, hipStream_t s) {
    dim3 grid((Lk + kRowsPerBlock - 1) / kRowsPerBlock, H);
    hipLaunchKernelGGL((imp_colsum_kernel<DT, D>), grid, dim3(kThreads), 0, s, Q, K, part, imp, Lq, Lk,
                       nsplit, c, 1.0f / (float)Lq);
    return hipGetLastError();
}

}  // namespace

ImpPlan imp_plan(int H, int Lq, int Lk, int dt) {
    const int kt = dt == kBF16 ? tile_rows<kBF16>() : tile_rows<kF32>();
    const long long blocks = (long long)H * ((Lq + kRowsPerBlock - 1) / kRowsPerBlock);
    const int max_split = (Lk + 4 * kt - 1) / (4 * kt);  // keep >= 4 tiles per split
    int ns = (int)((1024 + blocks - 1) / blocks);
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

hipError_t launch_imp_colsum(int dt, int d, const void* Q, const void* K, const float2* part, float* imp,
                             int H, int Lq, int Lk, int nsplit, float c, hipStream_t s) {
    if (dt == kBF16) return d == 128 ? colsum_launch<kBF16, 128>(Q, K, part, imp, H, Lq, Lk, nsplit, c, s)
                                     : colsum_launch<kBF16, 64>(Q, K, part, imp, H, Lq, Lk, nsplit, c, s);
    return d == 128 ? colsum_launch<kF32, 128>(Q, K, part, imp, H, Lq, Lk, nsplit, c, s)
                    : colsum_launch<kF32, 64>(Q, K, part, imp, H, Lq, Lk, nsplit, c, s);
}

}  // namespace fc
