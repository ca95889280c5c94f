// Redundancy pass A over a range of one head's keys, shared by the
// stand-alone kernel (redundancy.hip) and by the extra workgroups that run it
// inside importance pass 1 (importance.hip).
//
// Key designs item 3 of "Flow Caching for Autoregressive Video Generation"
// (papernotes digest) averages the cosine similarity of l2-normalised keys;
// with khat_j = k_j / max(||k_j||, 1e-12) the mean goes through
// u = sum_j khat_j, and this pass sums khat_j over rows [r0, r1).
#pragma once

#include "common.hpp"

namespace fc {

// Thread layout for one row of D elements of type DT: 16 bytes per lane.
template <int DT, int D, int THREADS>
struct RowLayout {
    static constexpr int kVec = 16 / Elem<DT>::kBytes;  // elements per lane
    static constexpr int kTpr = D / kVec;                // lanes per row
    static constexpr int kRpi = THREADS / kTpr;          // rows per block step
    static constexpr int kGroups = kWave / kTpr;         // rows per wave step
    static_assert(kTpr <= kWave && kWave % kTpr == 0, "a row must fit in one wave");
};

template <int DT>
__device__ __forceinline__ void load_vec(const void* p, float* x);
template <>
__device__ __forceinline__ void load_vec<kBF16>(const void* p, float* x) {
    const uint4 u = *reinterpret_cast<const uint4*>(p);
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        x[2 * i] = __uint_as_float(w[i] << 16);
        x[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
}
template <>
__device__ __forceinline__ void load_vec<kF32>(const void* p, float* x) {
    const float4 v = *reinterpret_cast<const float4*>(p);
    x[0] = v.x; x[1] = v.y; x[2] = v.z; x[3] = v.w;
}

// load_vec with a non-temporal load (rows read once by a streaming pass).
template <int DT>
__device__ __forceinline__ void load_vec_stream(const void* p, float* x) {
    const uint4 u = load_stream16(p);
    if constexpr (DT == kBF16) {
        const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            x[2 * i] = __uint_as_float(w[i] << 16);
            x[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
        }
    } else {
        x[0] = __uint_as_float(u.x); x[1] = __uint_as_float(u.y);
        x[2] = __uint_as_float(u.z); x[3] = __uint_as_float(u.w);
    }
}

constexpr int kRedRowsInFlight = 4;  // rows each lane group loads before reducing

// u_out[c] = sum over rows r0 <= j < r1 of khat_j[c] (Kh: the head's rows).
// Lane groups of kTpr lanes take one row each; the per-lane partials are
// added across the groups of a wave with shuffles, then across waves in
// `scratch` (THREADS / 64 * D floats of LDS), in a fixed order.  RIF rows per
// lane group are loaded before they are reduced; STREAM: non-temporal loads.
template <int DT, int D, int THREADS, int RIF = kRedRowsInFlight, bool STREAM = false>
__device__ __forceinline__ void red_norm_sum_rows(const char* __restrict__ Kh, int r0, int r1,
                                                  float* __restrict__ scratch, float* __restrict__ u_out) {
    using RL = RowLayout<DT, D, THREADS>;
    constexpr int kE = Elem<DT>::kBytes;
    const int g = threadIdx.x / RL::kTpr, e = threadIdx.x % RL::kTpr;
    float u[RL::kVec];
#pragma unroll
    for (int v = 0; v < RL::kVec; ++v) u[v] = 0.f;
    for (int row = r0 + g; row < r1; row += RIF * RL::kRpi) {
        float x[RIF][RL::kVec];
#pragma unroll
        for (int i = 0; i < RIF; ++i) {
            const int rr = row + i * RL::kRpi;
            if (rr < r1) {
                const char* src = Kh + ((size_t)rr * D + e * RL::kVec) * kE;
                if constexpr (STREAM) load_vec_stream<DT>(src, x[i]);
                else load_vec<DT>(src, x[i]);
            } else {
#pragma unroll
                for (int v = 0; v < RL::kVec; ++v) x[i][v] = 0.f;  // contributes nothing to u
            }
        }
#pragma unroll
        for (int i = 0; i < RIF; ++i) {
            float n2 = 0.f;
#pragma unroll
            for (int v = 0; v < RL::kVec; ++v) n2 = fmaf(x[i][v], x[i][v], n2);
            n2 = group_sum<RL::kTpr>(n2);
            const float inv = 1.0f / fmaxf(sqrtf(n2), 1e-12f);
#pragma unroll
            for (int v = 0; v < RL::kVec; ++v) u[v] = fmaf(x[i][v], inv, u[v]);
        }
    }
    // the row groups of a wave hold the same columns: add them pairwise
#pragma unroll
    for (int o = RL::kTpr; o < kWave; o <<= 1)
#pragma unroll
        for (int v = 0; v < RL::kVec; ++v) u[v] += __shfl_xor(u[v], o, kWave);
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    if (lane < RL::kTpr) {
#pragma unroll
        for (int v = 0; v < RL::kVec; ++v) scratch[wave * D + e * RL::kVec + v] = u[v];
    }
    __syncthreads();
    for (int c = threadIdx.x; c < D; c += THREADS) {
        float acc = 0.f;
        for (int w = 0; w < THREADS / kWave; ++w) acc += scratch[w * D + c];
        u_out[c] = acc;
    }
}

}  // namespace fc
