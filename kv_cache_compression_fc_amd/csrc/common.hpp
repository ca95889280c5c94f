// Shared device helpers for the gfx950 kernels of libflowcache.
// Wave64 only; no other target is built.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fc {

constexpr int kWave = 64;
constexpr float kLog2e = 1.4426950408889634f;

// Element types of the streamed tensors.
enum Dt : int { kF32 = 0, kBF16 = 1 };

template <int DT> struct Elem;
template <> struct Elem<kF32> { using T = float; static constexpr int kBytes = 4; };
template <> struct Elem<kBF16> { using T = uint16_t; static constexpr int kBytes = 2; };

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

// 16-byte loads and stores that bypass cache allocation (streaming data read
// or written once).
__device__ __forceinline__ uint4 load_stream16(const void* p) {
    const u32x4_t v = __builtin_nontemporal_load(static_cast<const u32x4_t*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void store_stream16(void* p, const uint4& v) {
    u32x4_t w = {v.x, v.y, v.z, v.w};
    __builtin_nontemporal_store(w, static_cast<u32x4_t*>(p));
}

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
    return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Eight consecutive elements of one row: the slice one lane feeds to one
// 16-deep step of a 32x32 MFMA (lanes 0-31 hold depth 0-7, lanes 32-63
// depth 8-15 of that step).
template <int DT> struct Frag8;
template <> struct Frag8<kBF16> {
    uint4 u;  // 8 x bf16
    __device__ __forceinline__ void load(const void* p) { u = *reinterpret_cast<const uint4*>(p); }
    __device__ __forceinline__ void zero() { u = make_uint4(0, 0, 0, 0); }
    __device__ __forceinline__ void unpack(float (&x)[8]) const {
        const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            x[2 * i] = __uint_as_float(w[i] << 16);
            x[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
        }
    }
};
template <> struct Frag8<kF32> {
    float4 lo, hi;
    __device__ __forceinline__ void load(const void* p) {
        lo = reinterpret_cast<const float4*>(p)[0];
        hi = reinterpret_cast<const float4*>(p)[1];
    }
    __device__ __forceinline__ void zero() { lo = hi = make_float4(0.f, 0.f, 0.f, 0.f); }
    __device__ __forceinline__ void unpack(float (&x)[8]) const {
        x[0] = lo.x; x[1] = lo.y; x[2] = lo.z; x[3] = lo.w;
        x[4] = hi.x; x[5] = hi.y; x[6] = hi.z; x[7] = hi.w;
    }
};

// acc(32x32) += A(32 rows x 16 depth) * B(16 depth x 32 cols).
// Lane l supplies row l%32 of A and column l%32 of B, depth slice 8*(l/32)..+8.
// Output: acc[r] is row 8*(r/4) + 4*(l/32) + r%4, column l%32.
__device__ __forceinline__ void mfma16(f32x16_t& acc, const Frag8<kBF16>& a, const Frag8<kBF16>& b) {
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a.u),
                                                  __builtin_bit_cast(bf16x8_t, b.u), acc, 0, 0, 0);
}
// float32 inputs: eight 32x32x2 steps.  Step s takes element s of each lane's
// slice, so depth index k=l/32 of step s is element 8k+s of the 16-deep block;
// A and B use the same mapping, hence the sum covers all 16 depths.
__device__ __forceinline__ void mfma16(f32x16_t& acc, const Frag8<kF32>& a, const Frag8<kF32>& b) {
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a.lo.x, b.lo.x, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a.lo.y, b.lo.y, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a.lo.z, b.lo.z, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a.lo.w, b.lo.w, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a.hi.x, b.hi.x, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a.hi.y, b.hi.y, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a.hi.z, b.hi.z, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a.hi.w, b.hi.w, acc, 0, 0, 0);
}

// 2^x and log2(x) on the hardware transcendental unit (v_exp_f32 / v_log_f32).
__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float log2_hw(float x) { return __builtin_amdgcn_logf(x); }

template <typename T>
__device__ __forceinline__ T wave_sum(T v) {
#pragma unroll
    for (int o = kWave / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
    return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = kWave / 2; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
    return v;
}
// Sum over aligned groups of G lanes (G a power of two, G <= 64).
template <int G>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
    for (int o = G / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
    return v;
}

// The hardware hands linear block b to XCD b % 8.  Give every XCD a
// contiguous range of logical work items (grid padded to a multiple of 8,
// per_xcd = grid / 8), so that the blocks running together on one XCD share
// a head and a key (or query) range in that XCD's L2.
__device__ __forceinline__ int xcd_item(int per_xcd) {
    return (int)(blockIdx.x % 8u) * per_xcd + (int)(blockIdx.x / 8u);
}

// Merge of two partial softmax normalisers (m, s) meaning s * 2^m.
__device__ __forceinline__ void lse2_merge(float& m, float& s, float m2, float s2) {
    float mn = fmaxf(m, m2);
    s = s * exp2_hw(m - mn) + s2 * exp2_hw(m2 - mn);
    m = mn;
}

// Block-wide exclusive prefix sum over 256 threads (4 waves).  `lds` needs
// 4 uint32 slots.  Returns the exclusive prefix; *total receives the sum.
__device__ __forceinline__ uint32_t block256_exclusive_scan(uint32_t v, uint32_t* lds, uint32_t* total) {
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    uint32_t inc = v;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
        uint32_t t = __shfl_up(inc, o, kWave);
        if (lane >= o) inc += t;
    }
    if (lane == kWave - 1) lds[wave] = inc;
    __syncthreads();
    uint32_t w0 = lds[0], w1 = lds[1], w2 = lds[2], w3 = lds[3];
    uint32_t before = (wave > 0 ? w0 : 0u) + (wave > 1 ? w1 : 0u) + (wave > 2 ? w2 : 0u);
    *total = w0 + w1 + w2 + w3;
    __syncthreads();
    return before + inc - v;
}

}  // namespace fc
