// Chunkwise relative L1 and reuse decision, "Flow Caching for Autoregressive
// Video Generation" (papernotes digest), Key designs item 1
//     L1_rel(X, t, i) = ||X^i_{t-1} - X^i_t||_1 / ||X^i_t||_1
// and item 2: the first m steps of a chunk recompute with f = 0; afterwards
// recompute and reset f when f + L1_rel > eps, else accumulate f and reuse.
//
// Two launches per denoising step.  Each chunk is cut into slabs of a fixed
// element count; a workgroup streams one slab of X_t and X_{t-1} with 16-byte
// loads, reduces sum|X_{t-1} - X_t| and sum|X_t| (float32 per lane,
// fixed-order wave and block reductions) and writes the pair.  A second,
// one-workgroup-per-chunk kernel adds the chunk's pairs in slab order (fp64),
// forms L1_rel and updates f, the recompute flag and the step counter on the
// device.  The kernel boundary orders the two (no cross-XCD fences or
// atomics), and the result is deterministic.  HBM-bound: every state byte is
// read once, with non-temporal loads.
#include "common.hpp"
#include "kernels.hpp"

namespace fc {

namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 4;     // 16-byte loads in flight per input per lane
constexpr int kSteps = 4;      // unrolled groups per slab
template <int DT> constexpr int vec_elems() { return 16 / Elem<DT>::kBytes; }
template <int DT> constexpr long long slab_elems() { return (long long)kThreads * vec_elems<DT>() * kUnroll * kSteps; }

template <int DT>
__device__ __forceinline__ void accum16(const uint4& a, const uint4& b, float& sa, float& sn);
template <>
__device__ __forceinline__ void accum16<kBF16>(const uint4& a, const uint4& b, float& sa, float& sn) {
    const uint32_t wa[4] = {a.x, a.y, a.z, a.w}, wb[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float a0 = __uint_as_float(wa[i] << 16), a1 = __uint_as_float(wa[i] & 0xffff0000u);
        const float b0 = __uint_as_float(wb[i] << 16), b1 = __uint_as_float(wb[i] & 0xffff0000u);
        sa += fabsf(b0 - a0) + fabsf(b1 - a1);
        sn += fabsf(a0) + fabsf(a1);
    }
}
template <>
__device__ __forceinline__ void accum16<kF32>(const uint4& a, const uint4& b, float& sa, float& sn) {
    const float fa[4] = {__uint_as_float(a.x), __uint_as_float(a.y), __uint_as_float(a.z), __uint_as_float(a.w)};
    const float fb[4] = {__uint_as_float(b.x), __uint_as_float(b.y), __uint_as_float(b.z), __uint_as_float(b.w)};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        sa += fabsf(fb[i] - fa[i]);
        sn += fabsf(fa[i]);
    }
}

template <int DT>
__device__ __forceinline__ float load_scalar(const void* p, long long i) {
    if constexpr (DT == kBF16) return bf16_to_f32(static_cast<const uint16_t*>(p)[i]);
    else return static_cast<const float*>(p)[i];
}

template <int DT>
__global__ __launch_bounds__(kThreads) void chunk_l1_partial_kernel(ChunkTable tab, const void* __restrict__ X_t,
                                                                    const void* __restrict__ X_tm1,
                                                                    const int32_t* __restrict__ step,
                                                                    float2* __restrict__ partial) {
    constexpr int V = vec_elems<DT>();
    constexpr long long EPB = slab_elems<DT>();
    __shared__ float red_a[kThreads / kWave], red_n[kThreads / kWave];

    const int bid = blockIdx.x;
    int lo = 0, hi = tab.n - 1;  // largest chunk c with blk_start[c] <= bid
    while (lo < hi) {
        const int mid = (lo + hi + 1) / 2;
        if (tab.blk_start[mid] <= bid) lo = mid; else hi = mid - 1;
    }
    const int c = lo;
    if (step[c] < 0) return;  // inactive chunk: nothing is read or written

    const long long s0 = tab.off[c] + (long long)(bid - tab.blk_start[c]) * EPB;
    const long long e0 = min(s0 + EPB, tab.off[c + 1]);
    const long long a0 = min(e0, (s0 + V - 1) / V * V);
    const long long a1 = max(a0, e0 / V * V);
    float sa = 0.f, sn = 0.f;
    // unaligned head and tail (fewer than V elements each)
    if (threadIdx.x < a0 - s0) {
        const float x = load_scalar<DT>(X_t, s0 + threadIdx.x), y = load_scalar<DT>(X_tm1, s0 + threadIdx.x);
        sa += fabsf(y - x); sn += fabsf(x);
    }
    if (threadIdx.x < e0 - a1) {
        const float x = load_scalar<DT>(X_t, a1 + threadIdx.x), y = load_scalar<DT>(X_tm1, a1 + threadIdx.x);
        sa += fabsf(y - x); sn += fabsf(x);
    }
    const uint4* va = reinterpret_cast<const uint4*>(X_t) + a0 / V;
    const uint4* vb = reinterpret_cast<const uint4*>(X_tm1) + a0 / V;
    const int nvec = (int)((a1 - a0) / V);
    int v = threadIdx.x;
    for (; v + (kUnroll - 1) * kThreads < nvec; v += kUnroll * kThreads) {
        uint4 xa[kUnroll], xb[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            xa[u] = load_stream16(va + v + u * kThreads);
            xb[u] = load_stream16(vb + v + u * kThreads);
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) accum16<DT>(xa[u], xb[u], sa, sn);
    }
    for (; v < nvec; v += kThreads) accum16<DT>(va[v], vb[v], sa, sn);

    sa = wave_sum(sa);
    sn = wave_sum(sn);
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    if (lane == 0) { red_a[wave] = sa; red_n[wave] = sn; }
    __syncthreads();
    if (threadIdx.x == 0) {
        float ta = 0.f, tn = 0.f;
        for (int w = 0; w < kThreads / kWave; ++w) { ta += red_a[w]; tn += red_n[w]; }
        partial[bid] = make_float2(ta, tn);
    }
}

// One workgroup per chunk: L1_rel from the chunk's slab pairs, then the
// reuse decision.
__global__ __launch_bounds__(kThreads) void chunk_decide_kernel(ChunkTable tab, const float2* __restrict__ partial,
                                                                int32_t* __restrict__ step, float* __restrict__ f,
                                                                uint8_t* __restrict__ recompute,
                                                                float* __restrict__ l1_out, int m, float eps) {
    __shared__ double fin_a[kThreads / kWave], fin_n[kThreads / kWave];
    const int c = blockIdx.x;
    const int n_step = step[c];
    if (n_step < 0) return;
    double A = 0.0, N = 0.0;
    for (int b = tab.blk_start[c] + threadIdx.x; b < tab.blk_start[c + 1]; b += kThreads) {
        const float2 p = partial[b];
        A += (double)p.x;
        N += (double)p.y;
    }
    A = wave_sum(A);
    N = wave_sum(N);
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    if (lane == 0) { fin_a[wave] = A; fin_n[wave] = N; }
    __syncthreads();
    if (threadIdx.x == 0) {
        double TA = 0.0, TN = 0.0;
        for (int w = 0; w < kThreads / kWave; ++w) { TA += fin_a[w]; TN += fin_n[w]; }
        const float l1 = TN > 0.0 ? (float)(TA / TN) : INFINITY;
        float f_new;
        uint8_t rec;
        if (n_step < m) {
            rec = 1; f_new = 0.f;                   // forced recompute, f = 0
        } else {
            const float a = f[c] + l1;
            if (a > eps) { rec = 1; f_new = 0.f; }  // recompute and reset
            else { rec = 0; f_new = a; }            // reuse and accumulate
        }
        f[c] = f_new;
        recompute[c] = rec;
        step[c] = n_step + 1;
        if (l1_out) l1_out[c] = l1;
    }
}

template <int DT>
hipError_t l1_launch(const ChunkTable& tab, const void* X_t, const void* X_tm1, int32_t* step, float* f,
                     uint8_t* recompute, float* l1_out, float2* partial, int m, float eps, hipStream_t s) {
    const int blocks = tab.blk_start[tab.n];
    hipLaunchKernelGGL(chunk_l1_partial_kernel<DT>, dim3(blocks), dim3(kThreads), 0, s, tab, X_t, X_tm1, step,
                       partial);
    hipLaunchKernelGGL(chunk_decide_kernel, dim3(tab.n), dim3(kThreads), 0, s, tab, partial, step, f, recompute,
                       l1_out, m, eps);
    return hipGetLastError();
}

}  // namespace

int chunk_blocks_for(long long elems, int dt) {
    const long long epb = dt == kBF16 ? slab_elems<kBF16>() : slab_elems<kF32>();
    const long long nb = (elems + epb - 1) / epb;
    return nb < 1 ? 1 : (int)nb;
}

hipError_t launch_chunk_l1(int dt, const ChunkTable& tab, const void* X_t, const void* X_tm1, int32_t* step,
                           float* f, uint8_t* recompute, float* l1_out, float2* partial, int m, float eps,
                           hipStream_t s) {
    if (dt == kBF16) return l1_launch<kBF16>(tab, X_t, X_tm1, step, f, recompute, l1_out, partial, m, eps, s);
    return l1_launch<kF32>(tab, X_t, X_tm1, step, f, recompute, l1_out, partial, m, eps, s);
}

}  // namespace fc
