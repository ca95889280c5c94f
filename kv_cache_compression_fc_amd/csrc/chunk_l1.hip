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
//
// Fused variant: item 1 writes the numerator as ||v dt||_1, the sampler's own
// update, so the slab kernel can take X_t and the velocity v instead of two
// states, write the Euler update X_{t-1} = X_t + v dt_i itself and sum
// |X_{t-1} - X_t| from the value it stores: three streams instead of the five
// of an update kernel followed by the L1 pass.  The slabs and the order of
// every sum are those of the unfused kernel, so the decision is the one
// fc_chunk_rel_l1_decide takes on (X_t, the stored X_{t-1}), bit for bit.
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

// Storage rounding of a float32 value: bf16 to nearest, ties to even
// (finite inputs); float32 unchanged.
__device__ __forceinline__ uint32_t bf16_rne_bits(float y) {
    const uint32_t u = __float_as_uint(y);
    return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// Euler update of one element in float32: the product and the sum are each
// rounded (no fused multiply-add), then the result is rounded to storage.
__device__ __forceinline__ float euler_f32(float x, float v, float dt) {
#pragma clang fp contract(off)
    const float p = v * dt;
    return x + p;
}

template <int DT>
__device__ __forceinline__ void euler16(const uint4& a, const uint4& b, float dt, uint4& out, float& sa, float& sn);
template <>
__device__ __forceinline__ void euler16<kBF16>(const uint4& a, const uint4& b, float dt, uint4& out, float& sa,
                                               float& sn) {
    const uint32_t wa[4] = {a.x, a.y, a.z, a.w}, wb[4] = {b.x, b.y, b.z, b.w};
    uint32_t wy[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float a0 = __uint_as_float(wa[i] << 16), a1 = __uint_as_float(wa[i] & 0xffff0000u);
        const float v0 = __uint_as_float(wb[i] << 16), v1 = __uint_as_float(wb[i] & 0xffff0000u);
        const uint32_t y0 = bf16_rne_bits(euler_f32(a0, v0, dt)), y1 = bf16_rne_bits(euler_f32(a1, v1, dt));
        wy[i] = y0 | (y1 << 16);
        const float b0 = __uint_as_float(y0 << 16), b1 = __uint_as_float(y1 << 16);
        sa += fabsf(b0 - a0) + fabsf(b1 - a1);
        sn += fabsf(a0) + fabsf(a1);
    }
    out = make_uint4(wy[0], wy[1], wy[2], wy[3]);
}
template <>
__device__ __forceinline__ void euler16<kF32>(const uint4& a, const uint4& b, float dt, uint4& out, float& sa,
                                              float& sn) {
    const float fa[4] = {__uint_as_float(a.x), __uint_as_float(a.y), __uint_as_float(a.z), __uint_as_float(a.w)};
    const float fv[4] = {__uint_as_float(b.x), __uint_as_float(b.y), __uint_as_float(b.z), __uint_as_float(b.w)};
    float fy[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        fy[i] = euler_f32(fa[i], fv[i], dt);
        sa += fabsf(fy[i] - fa[i]);
        sn += fabsf(fa[i]);
    }
    out = make_uint4(__float_as_uint(fy[0]), __float_as_uint(fy[1]), __float_as_uint(fy[2]), __float_as_uint(fy[3]));
}

template <int DT>
__device__ __forceinline__ float euler_scalar(void* y_out, long long i, float x, float v, float dt) {
    const float y = euler_f32(x, v, dt);
    if constexpr (DT == kBF16) {
        const uint32_t b = bf16_rne_bits(y);
        static_cast<uint16_t*>(y_out)[i] = (uint16_t)b;
        return __uint_as_float(b << 16);
    } else {
        static_cast<float*>(y_out)[i] = y;
        return y;
    }
}

template <int DT>
__device__ __forceinline__ float load_scalar(const void* p, long long i) {
    if constexpr (DT == kBF16) return bf16_to_f32(static_cast<const uint16_t*>(p)[i]);
    else return static_cast<const float*>(p)[i];
}

// One slab per workgroup.  EULER = false: the second input is X_{t-1}.
// EULER = true: the second input is the velocity v; the kernel writes
// X_{t-1} = X_t + v dt[c] to X_next (which may be X_t itself: every element
// is read before it is written, by the same lane) and sums against it.
template <int DT, bool EULER>
__global__ __launch_bounds__(kThreads) void chunk_l1_partial_kernel(ChunkTable tab, const void* X_t,
                                                                    const void* __restrict__ X_tm1,
                                                                    const int32_t* __restrict__ step,
                                                                    float2* __restrict__ partial,
                                                                    const float* __restrict__ dt, void* X_next) {
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
    const float h = EULER ? dt[c] : 0.f;

    const long long s0 = tab.off[c] + (long long)(bid - tab.blk_start[c]) * EPB;
    const long long e0 = min(s0 + EPB, tab.off[c + 1]);
    const long long a0 = min(e0, (s0 + V - 1) / V * V);
    const long long a1 = max(a0, e0 / V * V);
    float sa = 0.f, sn = 0.f;
    // unaligned head and tail (fewer than V elements each)
    if (threadIdx.x < a0 - s0) {
        const long long i = s0 + threadIdx.x;
        const float x = load_scalar<DT>(X_t, i), b = load_scalar<DT>(X_tm1, i);
        const float y = EULER ? euler_scalar<DT>(X_next, i, x, b, h) : b;
        sa += fabsf(y - x); sn += fabsf(x);
    }
    if (threadIdx.x < e0 - a1) {
        const long long i = a1 + threadIdx.x;
        const float x = load_scalar<DT>(X_t, i), b = load_scalar<DT>(X_tm1, i);
        const float y = EULER ? euler_scalar<DT>(X_next, i, x, b, h) : b;
        sa += fabsf(y - x); sn += fabsf(x);
    }
    const uint4* va = reinterpret_cast<const uint4*>(X_t) + a0 / V;
    const uint4* vb = reinterpret_cast<const uint4*>(X_tm1) + a0 / V;
    uint4* vy = EULER ? reinterpret_cast<uint4*>(X_next) + a0 / V : nullptr;
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
        for (int u = 0; u < kUnroll; ++u) {
            if constexpr (EULER) {
                uint4 y;
                euler16<DT>(xa[u], xb[u], h, y, sa, sn);
                store_stream16(vy + v + u * kThreads, y);
            } else {
                accum16<DT>(xa[u], xb[u], sa, sn);
            }
        }
    }
    for (; v < nvec; v += kThreads) {
        if constexpr (EULER) {
            uint4 y;
            euler16<DT>(va[v], vb[v], h, y, sa, sn);
            vy[v] = y;
        } else {
            accum16<DT>(va[v], vb[v], sa, sn);
        }
    }

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
//   kRuleChunkwise (FlowCache, Key designs item 2): a = f + L1_rel; recompute and
//     reset f to 0 when a > eps (and on the first m steps), else f = a.
//   kRuleHistory (ARCache, History-Guided Cache): the sum of the deviations since
//     the last refresh step, that step included: a = f + L1_rel; a > eps
//     refreshes and restarts the sum at this step's deviation (f = L1_rel),
//     else f = a; the first m steps refresh (f = L1_rel).
template <int RULE>
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
        const float f_reset = RULE == kRuleHistory ? l1 : 0.f;
        float f_new;
        uint8_t rec;
        if (n_step < m) {
            rec = 1; f_new = f_reset;                   // forced recompute
        } else {
            const float a = f[c] + l1;
            if (a > eps) { rec = 1; f_new = f_reset; }  // recompute, restart the sum
            else { rec = 0; f_new = a; }                // reuse and accumulate
        }
        f[c] = f_new;
        recompute[c] = rec;
        step[c] = n_step + 1;
        if (l1_out) l1_out[c] = l1;
    }
}

// Uniform policy: one L1_rel over every active chunk (sum of the numerators
// over sum of the denominators, slab pairs added chunk by chunk in order),
// one accumulator and step counter, the rule of Key designs item 2, and the
// same decision written for every active chunk.  One workgroup.
__global__ __launch_bounds__(kThreads) void uniform_decide_kernel(ChunkTable tab, const float2* __restrict__ partial,
                                                                  const int32_t* __restrict__ chunk_step,
                                                                  int32_t* __restrict__ step, float* __restrict__ f,
                                                                  uint8_t* __restrict__ recompute,
                                                                  float* __restrict__ l1_out, int m, float eps) {
    __shared__ double fin_a[kThreads / kWave], fin_n[kThreads / kWave];
    __shared__ uint8_t rec_s;
    double A = 0.0, N = 0.0;
    for (int c = 0; c < tab.n; ++c) {
        if (chunk_step[c] < 0) continue;
        for (int b = tab.blk_start[c] + threadIdx.x; b < tab.blk_start[c + 1]; b += kThreads) {
            const float2 p = partial[b];
            A += (double)p.x;
            N += (double)p.y;
        }
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
        const int n_step = step[0];
        uint8_t rec;
        float f_new;
        if (n_step < m) {
            rec = 1; f_new = 0.f;
        } else {
            const float a = f[0] + l1;
            if (a > eps) { rec = 1; f_new = 0.f; }
            else { rec = 0; f_new = a; }
        }
        f[0] = f_new;
        step[0] = n_step + 1;
        if (l1_out) l1_out[0] = l1;
        rec_s = rec;
    }
    __syncthreads();
    for (int c = threadIdx.x; c < tab.n; c += kThreads)
        if (chunk_step[c] >= 0) recompute[c] = rec_s;
}

template <int DT>
hipError_t l1_launch(const ChunkTable& tab, const void* X_t, const void* X_tm1, int32_t* step, float* f,
                     uint8_t* recompute, float* l1_out, float2* partial, int m, float eps, hipStream_t s,
                     const float* dt, void* X_next, int rule, int32_t* gstep) {
    const int blocks = tab.blk_start[tab.n];
    if (X_next != nullptr)
        hipLaunchKernelGGL((chunk_l1_partial_kernel<DT, true>), dim3(blocks), dim3(kThreads), 0, s, tab, X_t, X_tm1,
                           step, partial, dt, X_next);
    else
        hipLaunchKernelGGL((chunk_l1_partial_kernel<DT, false>), dim3(blocks), dim3(kThreads), 0, s, tab, X_t, X_tm1,
                           step, partial, nullptr, nullptr);
    if (rule == kRuleUniform)
        hipLaunchKernelGGL(uniform_decide_kernel, dim3(1), dim3(kThreads), 0, s, tab, partial, step, gstep, f,
                           recompute, l1_out, m, eps);
    else if (rule == kRuleHistory)
        hipLaunchKernelGGL(chunk_decide_kernel<kRuleHistory>, dim3(tab.n), dim3(kThreads), 0, s, tab, partial, step,
                           f, recompute, l1_out, m, eps);
    else
        hipLaunchKernelGGL(chunk_decide_kernel<kRuleChunkwise>, dim3(tab.n), dim3(kThreads), 0, s, tab, partial,
                           step, f, recompute, l1_out, m, eps);
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
                           hipStream_t s, const float* step_dt, void* X_next, int rule, int32_t* gstep) {
    if (dt == kBF16)
        return l1_launch<kBF16>(tab, X_t, X_tm1, step, f, recompute, l1_out, partial, m, eps, s, step_dt, X_next,
                                rule, gstep);
    return l1_launch<kF32>(tab, X_t, X_tm1, step, f, recompute, l1_out, partial, m, eps, s, step_dt, X_next, rule,
                           gstep);
}

}  // namespace fc
