// Issue-rate microbenchmark of the instructions that bound the importance
// passes on gfx950: v_exp_f32, v_fma_f32, their mix, the softmax body (one
// FMA, one exponential and one add per logit), v_mfma_f32_32x32x16_bf16
// alone, and the importance loop's mix (per 32x32 logit block: eight MFMAs
// and, for another block, 16 FMAs, 16 exponentials and 16 adds per lane).
//
// A measurement program, not part of libflowcache.  One workgroup per compute
// unit (a large LDS allocation keeps a second one off), with 1 or 4 waves per
// SIMD; every wave times its own loop with the core-cycle counter, so clock
// changes under the power limit do not enter the per-cycle rates.  Prints one
// JSON object.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdio>
#include <vector>

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

enum Mode { kExp = 0, kFma, kExpFma, kSoftmax, kMfma, kMfmaSoftmax, kModes };
const char* kNames[kModes] = {"exp", "fma", "exp_fma_mix", "softmax_body", "mfma_32x32x16_bf16",
                              "mfma_with_softmax"};
// instructions per wave per loop iteration: VALU (exp counted with VALU), exp alone, MFMA
const int kValu[kModes] = {16, 16, 16, 48, 0, 96};
const int kExps[kModes] = {16, 0, 8, 16, 0, 32};
const int kMfmas[kModes] = {0, 0, 0, 0, 8, 16};

#define SB() __builtin_amdgcn_sched_barrier(0)

template <int MODE>
__global__ void rate_kernel(float* __restrict__ sink, long long* __restrict__ cycles, float a, float b, int iters) {
    extern __shared__ float pad[];  // one workgroup per CU
    if (a > 1e30f) pad[threadIdx.x] = 0.f;
    const int lane = threadIdx.x & 63;
    float x[16], s[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        x[i] = 0.5f + 0.01f * i + 1e-5f * lane;
        s[i] = 0.f;
    }
    f32x16_t acc0 = {}, acc1 = {};
    const uint4 fa = make_uint4(0x3f803f80u ^ lane, 0x3f00bf00u, 0x3e803e80u, 0xbf40bf40u ^ (lane << 3));
    const uint4 fb = make_uint4(0x3f003f00u, 0x3e80be80u ^ lane, 0x3f403f40u, 0x3d803d80u);
    const bf16x8_t A = __builtin_bit_cast(bf16x8_t, fa), B = __builtin_bit_cast(bf16x8_t, fb);
    const float c = a * 1e-7f;  // keeps 2^(c acc + b) finite as the accumulators grow
    __syncthreads();
    const long long t0 = clock64();
    for (int it = 0; it < iters; ++it) {
        if constexpr (MODE == kExp) {
#pragma unroll
            for (int i = 0; i < 16; ++i) x[i] = __builtin_amdgcn_exp2f(-x[i]);  // fixed point near 0.64
        } else if constexpr (MODE == kFma) {
#pragma unroll
            for (int i = 0; i < 16; ++i) x[i] = fmaf(x[i], a, b);
        } else if constexpr (MODE == kExpFma) {
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                x[i] = __builtin_amdgcn_exp2f(-x[i]);
                x[i + 8] = fmaf(x[i + 8], a, b);
            }
        } else if constexpr (MODE == kSoftmax) {
            // one FMA, one exponential, one add per element: s += 2^(b - a s)
#pragma unroll
            for (int i = 0; i < 16; ++i) s[i] += __builtin_amdgcn_exp2f(fmaf(s[i], -a, b));
        } else if constexpr (MODE == kMfma) {
            // eight dependent MFMAs on one accumulator, as one 32x32x128 block
#pragma unroll
            for (int k = 0; k < 8; ++k) acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, B, acc0, 0, 0, 0);
        } else {
            // block A's eight MFMAs, each followed by the vector work of two
            // logits of block B (the other accumulator, finished in the last
            // half-step), then the same with the roles swapped
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, B, acc0, 0, 0, 0);
                SB();
#pragma unroll
                for (int r = 2 * k; r < 2 * k + 2; ++r) s[r] += __builtin_amdgcn_exp2f(fmaf(acc1[r], c, b));
                SB();
            }
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, B, acc1, 0, 0, 0);
                SB();
#pragma unroll
                for (int r = 2 * k; r < 2 * k + 2; ++r) s[r] += __builtin_amdgcn_exp2f(fmaf(acc0[r], c, b));
                SB();
            }
        }
    }
    const long long t1 = clock64();
    float tot = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) tot += x[i] + s[i] + acc0[i] + acc1[i];
    if (tot == 1234.5f) sink[blockIdx.x * blockDim.x + threadIdx.x] = tot;  // keeps the work live
    if (lane == 0) cycles[blockIdx.x * (blockDim.x / 64) + threadIdx.x / 64] = t1 - t0;
}

template <int MODE>
void run(int cus, int waves_per_simd, int iters, float* sink, long long* cyc_d, FILE* out, bool first) {
    const int threads = 256 * waves_per_simd;
    const size_t lds = 96 * 1024;
    hipFuncSetAttribute(reinterpret_cast<const void*>(rate_kernel<MODE>),
                        hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    hipLaunchKernelGGL(rate_kernel<MODE>, dim3(cus), dim3(threads), lds, 0, sink, cyc_d, 0.999f, -0.25f, 64);
    hipEvent_t e0, e1;
    hipEventCreate(&e0);
    hipEventCreate(&e1);
    hipEventRecord(e0, 0);
    hipLaunchKernelGGL(rate_kernel<MODE>, dim3(cus), dim3(threads), lds, 0, sink, cyc_d, 0.999f, -0.25f, iters);
    hipEventRecord(e1, 0);
    hipEventSynchronize(e1);
    float ms = 0.f;
    hipEventElapsedTime(&ms, e0, e1);
    const int nw = cus * threads / 64;
    std::vector<long long> cyc(nw);
    hipMemcpy(cyc.data(), cyc_d, nw * sizeof(long long), hipMemcpyDeviceToHost);
    std::sort(cyc.begin(), cyc.end());
    const double med = (double)cyc[nw / 2], mx = (double)cyc[nw - 1];
    // The waves of one SIMD start together but the arbiter does not share
    // issue evenly, so they end at different times: the SIMD's work of
    // waves_per_simd loops ends with its slowest wave.  Per-SIMD rates come
    // from the slowest wave's cycles.
    const double per_it = mx / iters;  // SIMD cycles per loop iteration (all its waves)
    auto per_instr = [&](int n) { return n > 0 ? per_it / ((double)n * waves_per_simd) : 0.0; };
    const double mfma_busy = kMfmas[MODE] > 0 ? 32.0 * kMfmas[MODE] * waves_per_simd / per_it : 0.0;
    fprintf(out,
            "%s    {\"mode\": \"%s\", \"waves_per_simd\": %d, \"iters\": %d, \"ms\": %.4f, "
            "\"cycles_median\": %.0f, \"cycles_max\": %.0f, \"cycles_per_iter\": %.2f, "
            "\"simd_cycles_per_valu\": %.3f, \"simd_cycles_per_exp\": %.3f, \"simd_cycles_per_mfma\": %.3f, "
            "\"mfma_pipe_busy_at_32_cycles\": %.3f, \"effective_clock_ghz\": %.3f}",
            first ? "" : ",\n", kNames[MODE], waves_per_simd, iters, ms, med, mx, per_it, per_instr(kValu[MODE]),
            per_instr(kExps[MODE]), per_instr(kMfmas[MODE]), mfma_busy, mx / (ms * 1e6));
    hipEventDestroy(e0);
    hipEventDestroy(e1);
}

}  // namespace

int main() {
    int dev = 0, cus = 0;
    hipGetDevice(&dev);
    hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    hipDeviceProp_t prop;
    hipGetDeviceProperties(&prop, dev);
    float* sink = nullptr;
    long long* cyc = nullptr;
    if (hipMalloc(&sink, (size_t)cus * 1024 * sizeof(float)) != hipSuccess ||
        hipMalloc(&cyc, (size_t)cus * 16 * sizeof(long long)) != hipSuccess) {
        fprintf(stderr, "hipMalloc failed\n");
        return 1;
    }
    printf("{\"device\": \"%s\", \"arch\": \"%s\", \"cus\": %d, \"results\": [\n", prop.name, prop.gcnArchName, cus);
    bool first = true;
    for (int w : {1, 4}) {
        const int iters = 20000;
        run<kExp>(cus, w, iters, sink, cyc, stdout, first);
        first = false;
        run<kFma>(cus, w, iters, sink, cyc, stdout, first);
        run<kExpFma>(cus, w, iters, sink, cyc, stdout, first);
        run<kSoftmax>(cus, w, iters, sink, cyc, stdout, first);
        run<kMfma>(cus, w, iters / 4, sink, cyc, stdout, first);
        run<kMfmaSoftmax>(cus, w, iters / 8, sink, cyc, stdout, first);
    }
    printf("\n]}\n");
    const hipError_t e = hipDeviceSynchronize();
    hipFree(sink);
    hipFree(cyc);
    return e == hipSuccess ? 0 : 1;
}
