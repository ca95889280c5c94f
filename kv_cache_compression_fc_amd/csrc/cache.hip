// KV cache manager kernels: a completed chunk joins the clean tokens of the
// cache (the flowchart under 整体框架 and Key designs item 3 of "Flow Caching
// for Autoregressive Video Generation": a fixed buffer of B_budget clean
// tokens plus the denoising region; a completed chunk enters the cache).
//
// One copy kernel serves both branches of a commit: appending the chunk
// behind the clean rows (cache not full) and assembling the merged set that
// the compression then reads (cache full).
#include "common.hpp"
#include "kernels.hpp"

namespace fc {
namespace {

constexpr int kThreads = 256;
// 32 rows per workgroup and non-temporal accesses: measured on the MAGI-like
// merge (24 heads x 10800 rows of 256 B, K and V) at ~5.7 TB/s, against
// ~3.4 TB/s with cached accesses and 64 rows per workgroup
constexpr int kRowsPerBlock = 32;

// Row j (0 <= j < n_old + n_new) of every head h:
//   dst[h][row0 + j] = j < n_old ? old[h][j] : fresh[h][j - n_old]      (K and V)
//   pos_dst[h][row0 + j] = j < n_old ? pos_old[h][j] : pos0 + (j - n_old)
// Head strides in rows: ld_old (old), n_new (fresh), ld_dst (dst).  16 bytes
// per lane, D * sizeof(element) / 16 lanes per row; every row is read and
// written once, so the accesses bypass cache allocation.
template <int DT, int D>
__global__ __launch_bounds__(kThreads) void cache_rows_kernel(const void* __restrict__ K_old,
                                                              const void* __restrict__ V_old,
                                                              const int32_t* __restrict__ pos_old, int ld_old,
                                                              int n_old, const void* __restrict__ K_new,
                                                              const void* __restrict__ V_new, int n_new, int32_t pos0,
                                                              void* __restrict__ K_dst, void* __restrict__ V_dst,
                                                              int32_t* __restrict__ pos_dst, int ld_dst, int row0) {
    constexpr int kRowBytes = D * Elem<DT>::kBytes;
    constexpr int kTpr = kRowBytes / 16;   // lanes per row
    constexpr int kRpi = kThreads / kTpr;  // rows per step
    constexpr int kSteps = kRowsPerBlock / kRpi;
    const int h = blockIdx.y;
    const int e = threadIdx.x % kTpr;
    const int j0 = blockIdx.x * kRowsPerBlock + threadIdx.x / kTpr;
    const int n = n_old + n_new;
    const bool with_pos = pos_dst != nullptr && e == 0;
    uint4 kv[kSteps], vv[kSteps];
    int32_t pv[kSteps];
#pragma unroll
    for (int i = 0; i < kSteps; ++i) {
        const int j = j0 + i * kRpi;
        if (j >= n) continue;
        const char *ks, *vs;
        if (j < n_old) {
            const size_t off = ((size_t)h * ld_old + j) * kRowBytes + e * 16;
            ks = static_cast<const char*>(K_old) + off;
            vs = static_cast<const char*>(V_old) + off;
        } else {
            const size_t off = ((size_t)h * n_new + (j - n_old)) * kRowBytes + e * 16;
            ks = static_cast<const char*>(K_new) + off;
            vs = static_cast<const char*>(V_new) + off;
        }
        kv[i] = load_stream16(ks);
        vv[i] = load_stream16(vs);
        if (with_pos) pv[i] = j < n_old ? pos_old[(size_t)h * ld_old + j] : pos0 + (int32_t)(j - n_old);
    }
#pragma unroll
    for (int i = 0; i < kSteps; ++i) {
        const int j = j0 + i * kRpi;
        if (j >= n) continue;
        const size_t off = ((size_t)h * ld_dst + row0 + j) * kRowBytes + e * 16;
        store_stream16(static_cast<char*>(K_dst) + off, kv[i]);
        store_stream16(static_cast<char*>(V_dst) + off, vv[i]);
        if (with_pos) pos_dst[(size_t)h * ld_dst + row0 + j] = pv[i];
    }
}

template <int DT, int D>
hipError_t rows_launch(int H, const void* K_old, const void* V_old, const int32_t* pos_old, int ld_old, int n_old,
                       const void* K_new, const void* V_new, int n_new, int32_t pos0, void* K_dst, void* V_dst,
                       int32_t* pos_dst, int ld_dst, int row0, hipStream_t s) {
    const int n = n_old + n_new;
    const dim3 grid((n + kRowsPerBlock - 1) / kRowsPerBlock, H);
    hipLaunchKernelGGL((cache_rows_kernel<DT, D>), grid, dim3(kThreads), 0, s, K_old, V_old, pos_old, ld_old, n_old,
                       K_new, V_new, n_new, pos0, K_dst, V_dst, pos_dst, ld_dst, row0);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_cache_rows(int dt, int d, int H, const void* K_old, const void* V_old, const int32_t* pos_old,
                             int ld_old, int n_old, const void* K_new, const void* V_new, int n_new, int32_t pos0,
                             void* K_dst, void* V_dst, int32_t* pos_dst, int ld_dst, int row0, hipStream_t s) {
    if (n_old + n_new <= 0) return hipSuccess;
    if (dt == kBF16)
        return d == 128 ? rows_launch<kBF16, 128>(H, K_old, V_old, pos_old, ld_old, n_old, K_new, V_new, n_new, pos0,
                                                  K_dst, V_dst, pos_dst, ld_dst, row0, s)
                        : rows_launch<kBF16, 64>(H, K_old, V_old, pos_old, ld_old, n_old, K_new, V_new, n_new, pos0,
                                                 K_dst, V_dst, pos_dst, ld_dst, row0, s);
    return d == 128 ? rows_launch<kF32, 128>(H, K_old, V_old, pos_old, ld_old, n_old, K_new, V_new, n_new, pos0,
                                             K_dst, V_dst, pos_dst, ld_dst, row0, s)
                    : rows_launch<kF32, 64>(H, K_old, V_old, pos_old, ld_old, n_old, K_new, V_new, n_new, pos0, K_dst,
                                            V_dst, pos_dst, ld_dst, row0, s);
}

}  // namespace fc
