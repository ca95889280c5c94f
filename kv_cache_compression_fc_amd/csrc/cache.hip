// KV cache manager kernel: a completed chunk joins the clean tokens of the
// cache (the flowchart under 整体框架 and Key designs item 3 of "Flow Caching
// for Autoregressive Video Generation": a fixed buffer of B_budget clean
// tokens plus the denoising region; a completed chunk enters the cache).
//
// The cache region is the page's fixed buffer, [H][B_budget + B_active] rows
// per tensor: the clean rows first, the chunk being denoised right behind
// them.  This kernel places a chunk held elsewhere into those rows and writes
// the chunk's positions; when the chunk was produced in place it only writes
// the positions.  The compression then reads the clean rows and the chunk as
// one row range and gathers the kept rows into the other region, so no merged
// copy is ever made.
#include "common.hpp"
#include "kernels.hpp"

namespace fc {
namespace {

constexpr int kThreads = 256;
// 32 rows per workgroup and non-temporal accesses: measured on a MAGI-like
// copy (24 heads x 10800 rows of 256 B, K and V) at ~5.7 TB/s, against
// ~3.4 TB/s with cached accesses and 64 rows per workgroup
constexpr int kRowsPerBlock = 32;

// Row j (0 <= j < n_new) of every head h:
//   dst[h][row0 + j] = fresh[h][j]   (K and V; skipped when K_new is null)
//   pos_dst[h][row0 + j] = pos0 + j  (when pos_dst is not null)
// Head strides in rows: n_new (fresh), ld_dst (dst).  16 bytes per lane,
// D * sizeof(element) / 16 lanes per row; every row is read and written once,
// so the accesses bypass cache allocation.
template <int DT, int D>
__global__ __launch_bounds__(kThreads) void cache_append_kernel(const void* __restrict__ K_new,
                                                                const void* __restrict__ V_new, int n_new,
                                                                int32_t pos0, void* __restrict__ K_dst,
                                                                void* __restrict__ V_dst,
                                                                int32_t* __restrict__ pos_dst, int ld_dst, int row0) {
    constexpr int kRowBytes = D * Elem<DT>::kBytes;
    constexpr int kTpr = kRowBytes / 16;   // lanes per row
    constexpr int kRpi = kThreads / kTpr;  // rows per step
    constexpr int kSteps = kRowsPerBlock / kRpi;
    const int h = blockIdx.y;
    const int e = threadIdx.x % kTpr;
    const int j0 = blockIdx.x * kRowsPerBlock + threadIdx.x / kTpr;
    if (K_new != nullptr) {
        uint4 kv[kSteps], vv[kSteps];
#pragma unroll
        for (int i = 0; i < kSteps; ++i) {
            const int j = j0 + i * kRpi;
            if (j >= n_new) continue;
            const size_t off = ((size_t)h * n_new + j) * kRowBytes + e * 16;
            kv[i] = load_stream16(static_cast<const char*>(K_new) + off);
            vv[i] = load_stream16(static_cast<const char*>(V_new) + off);
        }
#pragma unroll
        for (int i = 0; i < kSteps; ++i) {
            const int j = j0 + i * kRpi;
            if (j >= n_new) continue;
            const size_t off = ((size_t)h * ld_dst + row0 + j) * kRowBytes + e * 16;
            store_stream16(static_cast<char*>(K_dst) + off, kv[i]);
            store_stream16(static_cast<char*>(V_dst) + off, vv[i]);
        }
    }
    if (pos_dst != nullptr && e == 0) {
#pragma unroll
        for (int i = 0; i < kSteps; ++i) {
            const int j = j0 + i * kRpi;
            if (j < n_new) pos_dst[(size_t)h * ld_dst + row0 + j] = pos0 + (int32_t)j;
        }
    }
}

template <int DT, int D>
hipError_t append_launch(int H, const void* K_new, const void* V_new, int n_new, int32_t pos0, void* K_dst,
                         void* V_dst, int32_t* pos_dst, int ld_dst, int row0, hipStream_t s) {
    const dim3 grid((n_new + kRowsPerBlock - 1) / kRowsPerBlock, H);
    hipLaunchKernelGGL((cache_append_kernel<DT, D>), grid, dim3(kThreads), 0, s, K_new, V_new, n_new, pos0, K_dst,
                       V_dst, pos_dst, ld_dst, row0);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_cache_append(int dt, int d, int H, const void* K_new, const void* V_new, int n_new, int32_t pos0,
                               void* K_dst, void* V_dst, int32_t* pos_dst, int ld_dst, int row0, hipStream_t s) {
    if (n_new <= 0 || (K_new == nullptr && pos_dst == nullptr)) return hipSuccess;
#define FC_APPEND(DT_, D_) append_launch<DT_, D_>(H, K_new, V_new, n_new, pos0, K_dst, V_dst, pos_dst, ld_dst, row0, s)
    if (dt == kBF16) return d == 128 ? FC_APPEND(kBF16, 128) : FC_APPEND(kBF16, 64);
    return d == 128 ? FC_APPEND(kF32, 128) : FC_APPEND(kF32, 64);
#undef FC_APPEND
}

}  // namespace fc
