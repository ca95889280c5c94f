// Redundancy of the clean keys, "Flow Caching for Autoregressive Video
// Generation" (papernotes digest), Key designs item 3: the cosine similarity
// of l2-normalised keys with the diagonal zeroed, averaged over tokens, then
// softmaxed.  With khat_j = k_j / max(||k_j||, 1e-12) and u = sum_i khat_i,
//     r_j = (1/L_k) sum_{i != j} khat_i . khat_j = (u . khat_j - khat_j . khat_j) / L_k,
// so no L_k x L_k matrix is formed.  Two streaming passes over K, both
// HBM-bound (16-byte non-temporal loads, one row per TPR lanes, two rows per
// lane group in flight, wave reductions):
//   pass A: per-block partial u (fixed-order reduction, no float atomics;
//           inside fc_kv_compress it runs as extra workgroups of importance
//           pass 1 instead);
//   pass B: u from the partials, r_j, and per-block (max, sum e^{r-max}) for
//           the softmax over j.
#include "common.hpp"
#include "kernels.hpp"
#include "red_rows.hpp"

namespace fc {

namespace {

constexpr int kThreads = 256;
// Rows each lane group loads before reducing them.  Measured on the
// long-video keys (24 x 129600 rows of 256 B, MALL flushed): 2 rows with
// non-temporal loads 122 + 149 us for the two passes, against 135 + 170 us
// with 4 rows and cached loads; 1, 3 and 4 rows, and 96 or 128 workgroups
// per head, were slower.
constexpr int kRowsInFlight = 2;
template <int DT, int D> using RL256 = RowLayout<DT, D, kThreads>;

template <int DT, int D>
__global__ __launch_bounds__(kThreads) void red_norm_sum_kernel(const void* __restrict__ K,
                                                                float* __restrict__ u_part, int Lk) {
    constexpr int kE = Elem<DT>::kBytes;
    __shared__ float scratch[kThreads / kWave * D];
    const int h = blockIdx.y, blk = blockIdx.x, nblk = gridDim.x;
    const int rows = (Lk + nblk - 1) / nblk;
    const int r0 = blk * rows, r1 = min(Lk, r0 + rows);
    red_norm_sum_rows<DT, D, kThreads, kRowsInFlight, true>(static_cast<const char*>(K) + (size_t)h * Lk * D * kE,
                                                            r0, r1, scratch, u_part + ((size_t)h * nblk + blk) * D);
}

// Online softmax statistics of a block's values, merged over the block.
// Each thread passes its running (m, s) with s = sum e^{x - m}; the result is
// written by thread 0.
__device__ __forceinline__ void block_softmax_stats(float m, float s, float2* out) {
    __shared__ float sm[kThreads / kWave], ss[kThreads / kWave];
    // natural-log statistics are kept in base 2 inside: x*log2e
#pragma unroll
    for (int o = kWave / 2; o > 0; o >>= 1) {
        const float m2 = __shfl_xor(m, o, kWave), s2 = __shfl_xor(s, o, kWave);
        lse2_merge(m, s, m2, s2);
    }
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    if (lane == 0) { sm[wave] = m; ss[wave] = s; }
    __syncthreads();
    if (threadIdx.x == 0) {
        float M = sm[0], S = ss[0];
        for (int w = 1; w < kThreads / kWave; ++w) lse2_merge(M, S, sm[w], ss[w]);
        *out = make_float2(M, S);
    }
}

template <int DT, int D>
__global__ __launch_bounds__(kThreads) void red_dot_kernel(const void* __restrict__ K,
                                                           const float* __restrict__ u_part, int nbu,
                                                           float* __restrict__ r, float2* __restrict__ red_part,
                                                           int Lk) {
    using RL = RL256<DT, D>;
    constexpr int kE = Elem<DT>::kBytes;
    constexpr int kParts = kThreads / D;  // threads per column of u
    __shared__ float upart[kParts][D];
    __shared__ float ush[D];
    const int h = blockIdx.y, blk = blockIdx.x, nblk = gridDim.x;
    const int rows = (Lk + nblk - 1) / nblk;
    const int r0 = blk * rows, r1 = min(Lk, r0 + rows);
    const char* Kh = static_cast<const char*>(K) + (size_t)h * Lk * D * kE;
    const int g = threadIdx.x / RL::kTpr, e = threadIdx.x % RL::kTpr;
    auto load_rows = [&](int row, float (&x)[kRowsInFlight][RL::kVec]) {
#pragma unroll
        for (int i = 0; i < kRowsInFlight; ++i) {
            const int rr = row + i * RL::kRpi;
            if (rr < r1) {
                load_vec_stream<DT>(Kh + ((size_t)rr * D + e * RL::kVec) * kE, x[i]);
            } else {
#pragma unroll
                for (int v = 0; v < RL::kVec; ++v) x[i][v] = 0.f;
            }
        }
    };
    // the workgroup's first rows are in flight while u is formed
    float x[kRowsInFlight][RL::kVec];
    load_rows(r0 + g, x);
    // u = sum of the nbu partials: every thread takes every kParts-th partial
    // of one column (two interleaved sums, all loads issued at once), then
    // the parts are added in order
    {
        const int c = threadIdx.x % D, part = threadIdx.x / D;
        const float* pc = u_part + (size_t)h * nbu * D + c;
        constexpr int kMaxJ = (kRedMaxBlocks / kParts + 1) / 2 * 2;
        float t[kMaxJ];
#pragma unroll
        for (int j = 0; j < kMaxJ; ++j) {
            const int i = part + j * kParts;
            t[j] = i < nbu ? pc[(size_t)i * D] : 0.f;
        }
        float a0 = 0.f, a1 = 0.f;
#pragma unroll
        for (int j = 0; j < kMaxJ; j += 2) {
            a0 += t[j];
            a1 += t[j + 1];
        }
        upart[part][c] = a0 + a1;
    }
    __syncthreads();
    if (threadIdx.x < D) {
        float acc = 0.f;
#pragma unroll
        for (int q = 0; q < kParts; ++q) acc += upart[q][threadIdx.x];
        ush[threadIdx.x] = acc;
    }
    __syncthreads();
    float u[RL::kVec];
#pragma unroll
    for (int v = 0; v < RL::kVec; ++v) u[v] = ush[e * RL::kVec + v];
    const float inv_lk = 1.0f / (float)Lk;
    // r_j is a mean of cosines, |r_j| < 1, so sum 2^(r_j log2e - log2e) needs
    // no running maximum: the block's softmax partial is (log2e, s)
    float s = 0.f;
    for (int row = r0 + g; row < r1; row += kRowsInFlight * RL::kRpi) {
        if (row != r0 + g) load_rows(row, x);
#pragma unroll
        for (int i = 0; i < kRowsInFlight; ++i) {
            const int rr = row + i * RL::kRpi;
            float dot = 0.f, n2 = 0.f;
#pragma unroll
            for (int v = 0; v < RL::kVec; ++v) {
                dot = fmaf(x[i][v], u[v], dot);
                n2 = fmaf(x[i][v], x[i][v], n2);
            }
            dot = group_sum<RL::kTpr>(dot);
            n2 = group_sum<RL::kTpr>(n2);
            const float inv = 1.0f / fmaxf(sqrtf(n2), 1e-12f);
            const float rj = (dot * inv - n2 * inv * inv) * inv_lk;
            if (e == 0 && rr < r1) {
                r[(size_t)h * Lk + rr] = rj;
                s += exp2_hw(fmaf(rj, kLog2e, -kLog2e));
            }
        }
    }
    block_softmax_stats(kLog2e, s, red_part + (size_t)h * nblk + blk);
}

__global__ __launch_bounds__(kThreads) void red_stats_kernel(const float* __restrict__ r,
                                                             float2* __restrict__ red_part, int Lk) {
    const int h = blockIdx.y, blk = blockIdx.x, nblk = gridDim.x;
    const int rows = (Lk + nblk - 1) / nblk;
    const int r0 = blk * rows, r1 = min(Lk, r0 + rows);
    float m = -1e30f, s = 0.f;
    for (int j = r0 + threadIdx.x; j < r1; j += kThreads) lse2_merge(m, s, r[(size_t)h * Lk + j] * kLog2e, 1.0f);
    block_softmax_stats(m, s, red_part + (size_t)h * nblk + blk);
}

template <int DT, int D>
hipError_t norm_sum_launch(const void* K, float* u_part, int H, int Lk, hipStream_t s) {
    hipLaunchKernelGGL((red_norm_sum_kernel<DT, D>), dim3(red_nbu(Lk), H), dim3(kThreads), 0, s, K, u_part, Lk);
    return hipGetLastError();
}
template <int DT, int D>
hipError_t dot_launch(const void* K, const float* u_part, float* r, float2* red_part, int H, int Lk,
                      hipStream_t s) {
    hipLaunchKernelGGL((red_dot_kernel<DT, D>), dim3(red_nbr(Lk), H), dim3(kThreads), 0, s, K, u_part,
                       red_nbu(Lk), r, red_part, Lk);
    return hipGetLastError();
}

}  // namespace

int red_nbu(int Lk) {
    int n = (Lk + 511) / 512;
    return n < 1 ? 1 : (n > kRedMaxBlocks ? kRedMaxBlocks : n);
}
int red_nbr(int Lk) {
    int n = (Lk + 255) / 256;
    return n < 1 ? 1 : (n > kRedMaxBlocks ? kRedMaxBlocks : n);
}

hipError_t launch_red_norm_sum(int dt, int d, const void* K, float* u_part, int H, int Lk, hipStream_t s) {
    if (dt == kBF16) return d == 128 ? norm_sum_launch<kBF16, 128>(K, u_part, H, Lk, s)
                                     : norm_sum_launch<kBF16, 64>(K, u_part, H, Lk, s);
    return d == 128 ? norm_sum_launch<kF32, 128>(K, u_part, H, Lk, s)
                    : norm_sum_launch<kF32, 64>(K, u_part, H, Lk, s);
}

hipError_t launch_red_dot(int dt, int d, const void* K, const float* u_part, float* r, float2* red_part,
                          int H, int Lk, hipStream_t s) {
    if (dt == kBF16) return d == 128 ? dot_launch<kBF16, 128>(K, u_part, r, red_part, H, Lk, s)
                                     : dot_launch<kBF16, 64>(K, u_part, r, red_part, H, Lk, s);
    return d == 128 ? dot_launch<kF32, 128>(K, u_part, r, red_part, H, Lk, s)
                    : dot_launch<kF32, 64>(K, u_part, r, red_part, H, Lk, s);
}

hipError_t launch_red_stats(const float* r, float2* red_part, int H, int Lk, hipStream_t s) {
    hipLaunchKernelGGL(red_stats_kernel, dim3(red_nbr(Lk), H), dim3(kThreads), 0, s, r, red_part, Lk);
    return hipGetLastError();
}

}  // namespace fc
