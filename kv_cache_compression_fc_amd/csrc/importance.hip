// Importance of the clean keys, "Flow Caching for Autoregressive Video
// Generation" (papernotes digest), Key designs item 3: the attention softmax
// of the current denoising queries over the clean keys, averaged across the
// queries.  Per head h:
//     Imp_j = (1/L_q) sum_i exp(s_ij - lse_i),   s_ij = scale * q_i . k_j,
//     lse_i = log sum_j exp(s_ij).
// Two passes over Q K^T on bf16 MFMA (v_mfma_f32_32x32x16_bf16, fp32
// accumulate); neither materialises the L_q x L_k matrix:
//   pass 1 (imp_lse_kernel)    a workgroup owns 256 queries and one range of
//                              keys, streams K tiles through LDS and sums
//                              2^(x - m) per query, x = scale*log2(e) q.k;
//   pass 2 (imp_colsum_kernel) a workgroup owns 256 keys, streams Q tiles
//                              and their -lse2 through LDS, recomputes the
//                              logits and accumulates column sums of
//                              2^(x - lse2) in registers.
// Layout and scheduling for gfx950:
//   * 8 waves per workgroup, one register-resident 32-row operand block per
//     wave and at most 128 VGPRs, so four waves share each SIMD and the
//     vector work of one wave (one FMA, one v_exp_f32 and one add per logit)
//     fills the MFMA shadow of the others;
//   * the streamed tiles go global -> LDS directly (buffer_load ... lds, no
//     registers), three buffers deep, so each tile is requested two tiles
//     before it is used; rows past the end read as zero;
//   * LDS tiles are unpadded with an XOR swizzle of the 16-byte chunks, so the
//     16-byte fragment reads of 16 consecutive rows hit distinct banks;
//   * inside a tile the MFMAs of block 1 are interleaved with the
//     exponentials of block 0.
// Pass 1 does not track a running maximum: the shift m is the maximum over the
// range's first 32 keys, and a workgroup whose sums leave the safe range (a
// logit more than ~100 binary orders above m) redoes its range with an exact
// running maximum.  No atomics: the result is deterministic.
#include <atomic>
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"
#include "red_rows.hpp"

namespace fc {

namespace {

constexpr int kThreads = 512;
constexpr int kWaves = kThreads / kWave;
// __launch_bounds__ minimum waves per SIMD: four caps bf16 kernels at 128
// VGPRs; fp32 operand blocks are twice as large and run two.
template <int DT> constexpr int min_waves_per_simd() { return DT == kBF16 ? 4 : 2; }
constexpr int kRowsPerBlock = kWaves * 32;    // 256 queries (pass 1) or keys (pass 2)
constexpr int kNBuf = 3;                      // LDS tile buffers
constexpr int kPersistRounds = 8;             // items per slot from which a pass runs persistent
constexpr uint32_t kRsrcWord3 = 0x00020000u;  // raw buffer, 32-bit dwords (gfx9 family)
// A byte offset past every resource built here (a head's rows are < 2^31
// bytes, checked on the host, plus < 2^16 bytes of in-tile offsets).
constexpr uint32_t kNoRecord = 0x80000000u;

// Byte-addressed view of one head's rows for buffer loads: reads at or past
// num_bytes return zeros.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t head_rsrc(const void* base, uint32_t num_bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)num_bytes, (int)kRsrcWord3);
}

template <int DT> constexpr int tile_rows() { return DT == kBF16 ? 64 : 32; }

// A ROWS x D tile in LDS: rows of D*E bytes, 16-byte chunks XOR-swizzled so
// that the same logical chunk of 16 consecutive rows lands in 16 distinct
// bank groups.  Loaded straight from global memory by buffer_load ... lds: a
// wave instruction writes 1 KiB of consecutive LDS, lane i to chunk i, so
// each lane fetches the global chunk that the swizzle puts there.
template <int DT, int D, int ROWS>
struct SwizzledTile {
    static constexpr int kRowBytes = D * Elem<DT>::kBytes;
    static constexpr int kCpr = kRowBytes / 16;                 // chunks per row
    static constexpr int kBytes = ROWS * kRowBytes;
    static constexpr int kWaveLoads = ROWS * kCpr / kWave;      // 1 KiB wave loads per tile
    static constexpr int kLoadsPerWave = kWaveLoads / kWaves;
    static constexpr int kRowGroup = kCpr >= 16 ? 1 : 16 / kCpr;
    static constexpr int kSwzMod = kCpr >= 16 ? 16 : kCpr;
    static_assert(kLoadsPerWave >= 1 && kWaveLoads % kWaves == 0, "tile must split evenly over the waves");

    __device__ static __forceinline__ int swz(int r) { return (r / kRowGroup) % kSwzMod; }
    __device__ static __forceinline__ int offset(int r, int c) { return r * kRowBytes + ((c ^ swz(r)) << 4); }

    // This wave's share of the tile whose first row is at byte `off` of `rs`.
    __device__ static __forceinline__ void issue(__amdgpu_buffer_rsrc_t rs, uint32_t off, char* buf, int wave,
                                                 int lane) {
#pragma unroll
        for (int j = 0; j < kLoadsPerWave; ++j) {
            const int wl = wave * kLoadsPerWave + j;
            const int p = wl * kWave + lane;
            const int r = p / kCpr, c = (p % kCpr) ^ swz(p / kCpr);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, buf + wl * 1024, 16, off + r * kRowBytes + c * 16, 0, 0, 0);
        }
    }
};

// Byte offsets, inside a swizzled tile, of the fragments this lane reads for
// a 32-row block: row lane%32, elements 16*kk + 8*(lane/32) .. +8 (fp32: two
// 16-byte chunks).  The swizzle repeats every 16 rows, so a block starting at
// row r0 (a multiple of 16) reads at r0 * kRowBytes + these offsets: computed
// once per lane, independent of the buffer, and each LDS read is then one
// register plus an immediate.
template <int DT, int D, int ROWS>
struct FragOffsets {
    using T = SwizzledTile<DT, D, ROWS>;
    static constexpr int NKK = D / 16;
    static constexpr int kParts = DT == kBF16 ? 1 : 2;
    static_assert(T::kRowGroup * T::kSwzMod == 16, "swizzle period must be 16 rows");
    int o[NKK * kParts];
    __device__ __forceinline__ explicit FragOffsets(int lane) {
        const int r = lane & 31, half = lane >> 5;
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk)
#pragma unroll
            for (int p = 0; p < kParts; ++p) o[kk * kParts + p] = T::offset(r, kParts * (2 * kk + half) + p);
    }
};

template <int DT, int D, int ROWS>
__device__ __forceinline__ void load_frag(Frag8<DT>& f, const char* blk, const FragOffsets<DT, D, ROWS>& fo, int kk) {
    if constexpr (DT == kBF16) {
        f.u = *reinterpret_cast<const uint4*>(blk + fo.o[kk]);
    } else {
        f.lo = *reinterpret_cast<const float4*>(blk + fo.o[2 * kk]);
        f.hi = *reinterpret_cast<const float4*>(blk + fo.o[2 * kk + 1]);
    }
}

// Wait until at most n vector-memory operations of this wave are in flight.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt");
    // gfx9 encoding: vmcnt[3:0] | expcnt[6:4]=7 | lgkmcnt[11:8]=15 | vmcnt[5:4] in [15:14]
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// Workgroup barrier for the tile pipeline.  __syncthreads() would also wait
// for every LDS-DMA load in flight (they count as LDS stores), which drains
// the prefetch of the next-but-one tile; the waits before this barrier are
// explicit (wait_vmcnt for the tile about to be read; the compiler's lgkmcnt
// waits retire this wave's LDS reads before their results feed the MFMAs).
// The empty asm statements keep the compiler from moving memory accesses
// across the barrier.
__device__ __forceinline__ void tile_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

template <int B> using Buf = std::integral_constant<int, B>;

#define FC_SB() __builtin_amdgcn_sched_barrier(0)

// The work loop of a workgroup.  kPersist = false: the workgroup runs `own`
// (its item from the grid, or none if negative) and returns.  kPersist =
// true: the workgroup is persistent: items are in two groups (na of the first kind, nb of the
// second); XCD x owns [x ceil(na/8), ...) of the first and
// [x ceil(nb/8), ...) of the second, handed out by queue[x] in that order.
// Thread 0 takes the next item, own XCD (blockIdx % 8, the dispatcher's
// rotation) first, then the others; the workgroup runs it and loops until
// every queue is spent.  No item is taken twice, every item is taken (a
// counter past its XCD's count moves on), and no workgroup waits for
// another.  queue[0..8) must be zero before the launch.
template <bool kPersist, typename Run>
__device__ __forceinline__ void work_loop(uint32_t* __restrict__ queue, int na, int nb, int own, Run&& run) {
    if constexpr (!kPersist) {
        if (own >= 0) run(own);
        return;
    }
    __shared__ int s_item;
    const int pa = (na + 7) / 8, pb = (nb + 7) / 8;
    const int xcd = (int)(blockIdx.x % 8u);
    int qi = 0;  // thread 0's XCD cursor: queues before it are spent
    for (;;) {
        int item = -1;
        if (threadIdx.x == 0) {
            int it = -1;
            for (; qi < 8; ++qi) {
                const int x = (xcd + qi) % 8;
                const int ca = max(0, min(pa, na - x * pa)), cb = max(0, min(pb, nb - x * pb));
                if (ca + cb == 0) continue;
                const int k = (int)atomicAdd(&queue[x], 1u);
                if (k < ca) { it = x * pa + k; break; }
                if (k < ca + cb) { it = na + x * pb + (k - ca); break; }
            }
            s_item = it;
        }
        __syncthreads();
        item = s_item;
        __syncthreads();  // s_item is rewritten only after every wave has read it
        if (item < 0) return;
        run(item);
    }
}

// acc = (32 streamed rows starting at row r0 of the tile) x (register operand):
// a 32x32 fp32 tile; with kRegRows the register operand supplies the rows of
// acc and the streamed rows its columns instead.  Fragment reads run two
// MFMAs ahead of the ones that consume them; with `slice` each MFMA is
// followed, in a fixed order, by vector work on another block (16/NKK of its
// rows), so that work runs in the MFMA shadow.
template <int DT, int D, int ROWS, bool kRegRows = false, typename Slice>
__device__ __forceinline__ void mfma_block(f32x16_t& acc, const char* buf, int r0, const FragOffsets<DT, D, ROWS>& fo,
                                           const Frag8<DT> (&b)[D / 16], Slice&& slice) {
    constexpr int NKK = D / 16;
    constexpr int P = NKK >= 4 ? 2 : 1;  // fragment reads kept ahead of the MFMA that uses them
    const char* blk = buf + r0 * SwizzledTile<DT, D, ROWS>::kRowBytes;
    Frag8<DT> a[NKK];
#pragma unroll
    for (int kk = 0; kk < P; ++kk) load_frag<DT, D, ROWS>(a[kk], blk, fo, kk);
    acc = f32x16_t{};
    FC_SB();
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
        if (kk + P < NKK) load_frag<DT, D, ROWS>(a[kk + P], blk, fo, kk + P);
        if constexpr (kRegRows) mfma16(acc, b[kk], a[kk]);
        else mfma16(acc, a[kk], b[kk]);
        FC_SB();
        slice(kk * (16 / NKK), 16 / NKK);
        FC_SB();
    }
}
struct NoSlice {
    __device__ void operator()(int, int) const {}
};

// Masks logits of streamed rows at or past `valid` (relative to the block).
__device__ __forceinline__ void mask_rows(f32x16_t& acc, int valid, int half) {
#pragma unroll
    for (int r = 0; r < 16; ++r)
        if (8 * (r >> 2) + 4 * half + (r & 3) >= valid) acc[r] = -INFINITY;
}

template <int DT, int D, bool kPersist>
__global__ __launch_bounds__(kThreads, min_waves_per_simd<DT>()) void imp_lse_kernel(const void* __restrict__ Q,
                                                                            const void* __restrict__ K,
                                                                            float2* __restrict__ part, int Lq,
                                                                            int Lk, int ldk, int keys_per_split,
                                                                            int nsplit,
                                                                            int nqb, int n_items, float c,
                                                                            float* __restrict__ u_part, int nbu,
                                                                            int n_lse_blocks,
                                                                            uint32_t* __restrict__ queue, int H) {
    constexpr int kE = Elem<DT>::kBytes;
    constexpr int KT = tile_rows<DT>();
    constexpr int NKK = D / 16;
    using Tile = SwizzledTile<DT, D, KT>;
    constexpr int L = Tile::kLoadsPerWave;
    // One LDS array per buffer, each named at compile time (the tile loop is
    // unrolled by kNBuf): the compiler can then tell a buffer being read from
    // the buffer an LDS-DMA load is filling, and does not wait for that load.
    __shared__ __align__(1024) char lds0[Tile::kBytes];
    __shared__ __align__(1024) char lds1[Tile::kBytes];
    __shared__ __align__(1024) char lds2[Tile::kBytes];
    auto lds = [&](auto b) -> char* {
        if constexpr (decltype(b)::value == 0) return lds0;
        else if constexpr (decltype(b)::value == 1) return lds1;
        else return lds2;
    };

    // Redundancy pass A (partial sums of the normalised keys over one range
    // of one head's keys): it only feeds pass 2, so it runs as extra work
    // items of this launch, in the slots pass 1's last round leaves free,
    // instead of a launch of its own before pass 1.
    auto run_red = [&](const int b) {
        const int h = b / nbu, blk = b % nbu;
        const int rows = (Lk + nbu - 1) / nbu;
        const int r0 = blk * rows, r1 = min(Lk, r0 + rows);
        red_norm_sum_rows<DT, D, kThreads>(static_cast<const char*>(K) + (size_t)h * ldk * D * kE, r0, r1,
                                           reinterpret_cast<float*>(lds0), u_part + ((size_t)h * nbu + blk) * D);
    };
    auto run_lse = [&](const int item) {
        const int qblk = item % nqb, hs = item / nqb;
        const int split = hs % nsplit, h = hs / nsplit;

        const int lane = threadIdx.x & (kWave - 1);
        // the wave index as a scalar: the LDS-DMA destinations (M0) then need
        // no readfirstlane per load (0.3 % off the long-video stage)
        const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
        const int half = lane >> 5;
        const FragOffsets<DT, D, KT> fo(lane);
        const int q = qblk * kRowsPerBlock + wave * 32 + (lane & 31);
        // A wave whose 32 queries all lie past L_q (the last query block of a head
        // is padded to kRowsPerBlock) does no arithmetic: it only issues its share
        // of every tile load and takes every barrier, so the workgroup's barriers
        // and waits stay the same on all waves.
        const bool live = qblk * kRowsPerBlock + wave * 32 < Lq;
        const char* Qh = static_cast<const char*>(Q) + (size_t)h * Lq * D * kE;
        const __amdgpu_buffer_rsrc_t krs = head_rsrc(static_cast<const char*>(K) + (size_t)h * ldk * D * kE,
                                                     (uint32_t)Lk * D * kE);

        const int k_begin = split * keys_per_split;
        const int nkeys = min(Lk, k_begin + keys_per_split) - k_begin;  // >= 1
        const int ntiles = (nkeys + KT - 1) / KT;
        const uint32_t off0 = (uint32_t)k_begin * D * kE;
        const uint32_t tile_bytes = KT * D * kE;

        // Tiles 0 and 1 in flight while the Q fragments load.
        Tile::issue(krs, off0, lds(Buf<0>{}), wave, lane);
        Tile::issue(krs, ntiles > 1 ? off0 + tile_bytes : kNoRecord, lds(Buf<1>{}), wave, lane);

        // Q^T fragments (B operand): query q, depth 16*kk + 8*half .. +8.
        Frag8<DT> qf[NKK];
    #pragma unroll
        for (int kk = 0; kk < NKK; ++kk) {
            if (q < Lq) qf[kk].load(Qh + ((size_t)q * D + 16 * kk + 8 * half) * kE);
            else qf[kk].zero();
        }
        wait_vmcnt<L>();  // tile 0 landed (tile 1 may be in flight)
        tile_barrier();

        // Shift: the maximum logit over the first 32 keys of the range (exact,
        // masked), per query.
        float nm = 0.f;
        if (live) {
            f32x16_t acc;
            mfma_block<DT, D, KT>(acc, lds(Buf<0>{}), 0, fo, qf, NoSlice{});
            mask_rows(acc, nkeys, half);
            float t = acc[0];
    #pragma unroll
            for (int r = 1; r < 16; ++r) t = fmaxf(t, acc[r]);
            t = fmaxf(t, __shfl_xor(t, 32, kWave));
            nm = -t * c;
        }

        float s0 = 0.f, s1 = 0.f, s2 = 0.f, s3 = 0.f;
        auto acc_rows = [&](const f32x16_t& acc, int r0, int nr) {
    #pragma unroll
            for (int r = r0; r < r0 + nr; ++r) {
                const float p = exp2_hw(fmaf(acc[r], c, nm));
                if ((r & 3) == 0) s0 += p; else if ((r & 3) == 1) s1 += p; else if ((r & 3) == 2) s2 += p; else s3 += p;
            }
        };
        // Tile t is read from buffer t % 3; tile t+2 goes into the buffer tile t-1
        // used, which every wave has left (barrier at the end of step t-1).
        // The exponentials of each 32-key block run in the MFMA shadow of the
        // next block: block 1 of tile t is finished during block 0 of tile t+1
        // (`carry`), so every wave alternates MFMA and vector work throughout
        // instead of all waves of the workgroup doing one, then the other, between
        // barriers.  carry starts at -inf (adds 0).
        f32x16_t carry;
    #pragma unroll
        for (int r = 0; r < 16; ++r) carry[r] = -INFINITY;
        // A step on a tile whose rows all lie inside the range (`full`) has no
        // masking and so no branch: the whole step is one basic block, and the
        // scheduling barriers keep the exponentials of one block between the
        // MFMAs of the other.  (With the masking branches in the step, the
        // compiler moves that vector work out of the MFMA sequence.)  The last
        // tiles of a range take the masked form.
        auto step = [&](auto b, auto full, int t) {
            constexpr int B = decltype(b)::value;
            // Past the last tile the offset lies outside the resource: the load
            // moves no data (zeros land in a buffer nobody reads), and every step
            // issues the same loads, so the waits below stay uniform.
            Tile::issue(krs, t + 2 < ntiles ? off0 + (uint32_t)(t + 2) * tile_bytes : kNoRecord,
                        lds(Buf<(B + 2) % kNBuf>{}), wave, lane);
            const char* buf = lds(b);
            f32x16_t a0;
            mfma_block<DT, D, KT>(a0, buf, 0, fo, qf, [&](int r0, int nr) { acc_rows(carry, r0, nr); });
            if constexpr (decltype(full)::value) {
                if constexpr (KT == 64)
                    mfma_block<DT, D, KT>(carry, buf, 32, fo, qf, [&](int r0, int nr) { acc_rows(a0, r0, nr); });
                else
                    carry = a0;
            } else {
                const int valid = nkeys - t * KT;  // rows of this tile inside the range
                if (valid < 32) mask_rows(a0, valid, half);
                if constexpr (KT == 64) {
                    if (valid > 32) {
                        mfma_block<DT, D, KT>(carry, buf, 32, fo, qf, [&](int r0, int nr) { acc_rows(a0, r0, nr); });
                        if (valid < 64) mask_rows(carry, valid - 32, half);
                    } else {
                        acc_rows(a0, 0, 16);
    #pragma unroll
                        for (int r = 0; r < 16; ++r) carry[r] = -INFINITY;
                    }
                } else {
                    carry = a0;
                }
            }
            wait_vmcnt<L>();  // tile t+1 landed, tile t+2 may be in flight
            tile_barrier();
        };
        // A padding wave's step: the same loads, waits and barrier, no arithmetic.
        auto idle_step = [&](auto b, auto, int t) {
            constexpr int B = decltype(b)::value;
            Tile::issue(krs, t + 2 < ntiles ? off0 + (uint32_t)(t + 2) * tile_bytes : kNoRecord,
                        lds(Buf<(B + 2) % kNBuf>{}), wave, lane);
            wait_vmcnt<L>();
            tile_barrier();
        };
        // Whole rounds of three full tiles, then the rest (at most two full tiles
        // and a partial one) in the masked form: the loop's back edge only
        // follows a buffer-2 step, so the compiler sees on every path which loads
        // the explicit waits have retired and adds no waits of its own.
        using Full = std::true_type;
        using Part = std::false_type;
        const int nfull = nkeys / KT;
        auto run_tiles = [&](auto&& st) {
            int t = 0;
            for (; t + 2 < nfull; t += kNBuf) {
                st(Buf<0>{}, Full{}, t);
                st(Buf<1>{}, Full{}, t + 1);
                st(Buf<2>{}, Full{}, t + 2);
            }
            if (t < ntiles) {
                st(Buf<0>{}, Part{}, t);
                if (t + 1 < ntiles) {
                    st(Buf<1>{}, Part{}, t + 1);
                    if (t + 2 < ntiles) st(Buf<2>{}, Part{}, t + 2);
                }
            }
        };
        if (live) run_tiles(step);
        else run_tiles(idle_step);
        wait_vmcnt<0>();
        if (live) acc_rows(carry, 0, 16);

        float m = -nm, tot = (s0 + s1) + (s2 + s3);
        if (__syncthreads_or(!(tot < 0x1p100f))) {  // overflow (or NaN) under the fixed shift
            // Exact path for this range: running maximum per block of 32 keys.
            m = -1e30f;
            tot = 0.f;
            for (int t = 0; t < ntiles; ++t) {
                Tile::issue(krs, off0 + (uint32_t)t * tile_bytes, lds(Buf<0>{}), wave, lane);
                wait_vmcnt<0>();
                __syncthreads();
    #pragma unroll
                for (int kb = 0; kb < KT / 32; ++kb) {
                    const int valid = nkeys - t * KT - kb * 32;
                    if (valid <= 0) break;
                    if (!live) continue;
                    f32x16_t acc;
                    mfma_block<DT, D, KT>(acc, lds(Buf<0>{}), kb * 32, fo, qf, NoSlice{});
                    mask_rows(acc, valid, half);
                    float tmax = acc[0];
    #pragma unroll
                    for (int r = 1; r < 16; ++r) tmax = fmaxf(tmax, acc[r]);
                    const float mn = fmaxf(m, tmax * c);
                    float p = 0.f;
    #pragma unroll
                    for (int r = 0; r < 16; ++r) p += exp2_hw(fmaf(acc[r], c, -mn));
                    tot = fmaf(tot, exp2_hw(m - mn), p);
                    m = mn;
                }
                __syncthreads();
            }
        }
        // Lanes l and l^32 hold disjoint key subsets of the same query.
        const float m2 = __shfl_xor(m, 32, kWave), t2 = __shfl_xor(tot, 32, kWave);
        lse2_merge(m, tot, m2, t2);
        if (lane < 32 && q < Lq) part[((size_t)h * nsplit + split) * Lq + q] = make_float2(m, tot);

    };
    // One work item per workgroup without a queue: the lse items in
    // XCD-contiguous ranges, then the redundancy items.
    // Persistent workgroups (with a queue), one per slot.  XCD x owns the lse items
    // [x pl, x pl + pl) and the redundancy items [x pr, x pr + pr), handed out
    // in that order by its counter queue[x]; a workgroup takes its own XCD's
    // items first (they share K ranges in that XCD's L2), then the other
    // XCDs' while any remain, so faster XCDs do more of the work.  Every
    // item is computed as in the one-item form: the same bits.
    const int n_red = u_part != nullptr ? H * nbu : 0;
    int own = -1;
    if ((int)blockIdx.x >= n_lse_blocks) {
        own = n_items + ((int)blockIdx.x - n_lse_blocks);
    } else {
        const int it = xcd_item((n_items + 7) / 8);
        own = it < n_items ? it : -1;
    }
    work_loop<kPersist>(queue, n_items, n_red, own, [&](int item) {
        if (item < n_items) run_lse(item);
        else run_red(item - n_items);
    });
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

constexpr int kSmallThreads = 256;

// Per query: the natural-log lse (optional) and -lse2 padded with -inf to
// lq_pad (optional), from the pass-1 partials.  Block 0 of each head also
// sums the redundancy partials u_part[h][0..nbu) into u[h] (fixed order).
__global__ __launch_bounds__(kSmallThreads) void imp_lse_merge_kernel(const float2* __restrict__ part,
                                                                      float* __restrict__ lse,
                                                                      float* __restrict__ nlse2, int Lq, int lq_pad,
                                                                      int nsplit, const float* __restrict__ u_part,
                                                                      int nbu, float* __restrict__ u, int d) {
    const int h = blockIdx.y;
    if (u_part != nullptr && blockIdx.x == 0) {
        for (int c = threadIdx.x; c < d; c += kSmallThreads) {
            // four independent chains keep four loads in flight
            const float* pc = u_part + (size_t)h * nbu * d + c;
            float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
            int i = 0;
            for (; i + 4 <= nbu; i += 4) {
                a0 += pc[(size_t)i * d];
                a1 += pc[(size_t)(i + 1) * d];
                a2 += pc[(size_t)(i + 2) * d];
                a3 += pc[(size_t)(i + 3) * d];
            }
            for (; i < nbu; ++i) a0 += pc[(size_t)i * d];
            u[(size_t)h * d + c] = (a0 + a1) + (a2 + a3);
        }
    }
    const int q = blockIdx.x * kSmallThreads + threadIdx.x;
    if (q >= lq_pad) return;
    const float l2 = q < Lq ? merged_lse2(part + (size_t)h * nsplit * Lq, Lq, nsplit, q) : INFINITY;
    if (lse && q < Lq) lse[(size_t)h * Lq + q] = l2 / kLog2e;
    if (nlse2) nlse2[(size_t)h * lq_pad + q] = -l2;
}

// The persistent passes' item counters start at zero (a kernel, not a
// memset, so that graph capture records no memset node).
__global__ void imp_queue_zero_kernel(uint32_t* __restrict__ q) {
    if (threadIdx.x < kImpQueueWords) q[threadIdx.x] = 0u;
}

// imp[h][j] = sum of the nqs partial planes (fixed order).
__global__ __launch_bounds__(kSmallThreads) void imp_sum_planes_kernel(const float* __restrict__ part,
                                                                       float* __restrict__ imp, size_t n, int nqs) {
    for (size_t i = (size_t)blockIdx.x * kSmallThreads + threadIdx.x; i < n; i += (size_t)gridDim.x * kSmallThreads) {
        float a = part[i];
        for (int q = 1; q < nqs; ++q) a += part[(size_t)q * n + i];
        imp[i] = a;
    }
}

// -lse2 padded with -inf from a natural-log lse.
__global__ __launch_bounds__(kSmallThreads) void imp_nlse2_kernel(const float* __restrict__ lse,
                                                                  float* __restrict__ nlse2, int Lq, int lq_pad) {
    const int h = blockIdx.y;
    const int q = blockIdx.x * kSmallThreads + threadIdx.x;
    if (q < lq_pad) nlse2[(size_t)h * lq_pad + q] = q < Lq ? -lse[(size_t)h * Lq + q] * kLog2e : -INFINITY;
}

// Redundancy of the keys a pass-2 workgroup holds in registers (Key designs
// item 3: cosine similarity of l2-normalised keys, diagonal zeroed, averaged
// over the L_k tokens).  With khat = k / max(||k||, 1e-12) and u = sum_i khat_i,
//     r_j = (u . khat_j - khat_j . khat_j) / L_k.
// Lane l holds depths 16*kk + 8*(l/32) .. +8 of key l%32, so the two halves
// of the wave add their partial dot products.  Also writes the workgroup's
// softmax partial (max, sum 2^(x - max)) of x = r * log2(e).
template <int DT, int D>
__device__ __forceinline__ void redundancy_of_keys(const Frag8<DT> (&kf)[D / 16], const float* __restrict__ uh,
                                                   int key, int lane, int Lk, float* __restrict__ r_h,
                                                   float2* __restrict__ red_out) {
    __shared__ float2 wstat[kWaves];
    const int half = lane >> 5;
    float dot = 0.f, n2 = 0.f;
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
        float x[8];
        kf[kk].unpack(x);
        const float4 u0 = *reinterpret_cast<const float4*>(uh + 16 * kk + 8 * half);
        const float4 u1 = *reinterpret_cast<const float4*>(uh + 16 * kk + 8 * half + 4);
        const float uv[8] = {u0.x, u0.y, u0.z, u0.w, u1.x, u1.y, u1.z, u1.w};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            dot = fmaf(x[e], uv[e], dot);
            n2 = fmaf(x[e], x[e], n2);
        }
    }
    dot += __shfl_xor(dot, 32, kWave);
    n2 += __shfl_xor(n2, 32, kWave);
    const float inv = 1.0f / fmaxf(sqrtf(n2), 1e-12f);
    const float rj = (dot * inv - n2 * inv * inv) / (float)Lk;
    const bool own = lane < 32 && key < Lk;
    if (own) r_h[key] = rj;
    float m = own ? rj * kLog2e : -1e30f, s = own ? 1.f : 0.f;
#pragma unroll
    for (int o = kWave / 2; o > 0; o >>= 1) {
        const float m2 = __shfl_xor(m, o, kWave), s2 = __shfl_xor(s, o, kWave);
        lse2_merge(m, s, m2, s2);
    }
    if (lane == 0) wstat[threadIdx.x / kWave] = make_float2(m, s);
    __syncthreads();
    if (threadIdx.x == 0) {
        float M = wstat[0].x, S = wstat[0].y;
        for (int w = 1; w < kWaves; ++w) lse2_merge(M, S, wstat[w].x, wstat[w].y);
        *red_out = make_float2(M, S);
    }
}

template <int DT, int D, bool kPersist>
__global__ __launch_bounds__(kThreads, min_waves_per_simd<DT>()) void imp_colsum_kernel(const void* __restrict__ Q,
                                                                               const void* __restrict__ K,
                                                                               const float* __restrict__ nlse2,
                                                                               float* __restrict__ imp, int H,
                                                                               int Lq, int lq_pad, int Lk, int ldk,
                                                                               int nkb,
                                                                               int nqs, int tpi, int n_items,
                                                                               float c, float inv_lq,
                                                                               const float* __restrict__ u,
                                                                               float* __restrict__ r_out,
                                                                               float2* __restrict__ red_part,
                                                                               uint32_t* __restrict__ queue) {
    constexpr int kE = Elem<DT>::kBytes;
    constexpr int QT = tile_rows<DT>();
    constexpr int NKK = D / 16;
    using Tile = SwizzledTile<DT, D, QT>;
    constexpr int L = Tile::kLoadsPerWave + 1;  // + the load of the tile's -lse2
    // Per buffer: a Q tile and the tile's -lse2 (64 floats, QT <= 64), each a
    // separate LDS array named at compile time (see imp_lse_kernel).
    __shared__ __align__(1024) char lds0[Tile::kBytes];
    __shared__ __align__(1024) char lds1[Tile::kBytes];
    __shared__ __align__(1024) char lds2[Tile::kBytes];
    __shared__ float nl0[kWave], nl1[kWave], nl2[kWave];
    auto lds = [&](auto b) -> char* {
        if constexpr (decltype(b)::value == 0) return lds0;
        else if constexpr (decltype(b)::value == 1) return lds1;
        else return lds2;
    };
    auto nl_lds = [&](auto b) -> float* {
        if constexpr (decltype(b)::value == 0) return nl0;
        else if constexpr (decltype(b)::value == 1) return nl1;
        else return nl2;
    };

    // item = (h * nqs + qs) * nkb + kblk: consecutive items (one XCD) share
    // a head and a query range, so they stream the same Q tiles.
    auto run = [&](const int item) {
        const int kblk = item % nkb, hq = item / nkb;
        const int qs = hq % nqs, h = hq / nqs;

        const int lane = threadIdx.x & (kWave - 1);
        // the wave index as a scalar: the LDS-DMA destinations (M0) then need
        // no readfirstlane per load (0.3 % off the long-video stage)
        const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
        const int half = lane >> 5;
        const FragOffsets<DT, D, QT> fo(lane);
        const int key = kblk * kRowsPerBlock + wave * 32 + (lane & 31);
        const __amdgpu_buffer_rsrc_t qrs = head_rsrc(static_cast<const char*>(Q) + (size_t)h * Lq * D * kE,
                                                     (uint32_t)Lq * D * kE);
        const __amdgpu_buffer_rsrc_t nrs = head_rsrc(nlse2 + (size_t)h * lq_pad, (uint32_t)lq_pad * 4);
        const char* Kh = static_cast<const char*>(K) + (size_t)h * ldk * D * kE;
        // this item's query tiles [t_begin, t_end)
        const int t_begin = qs * tpi;
        const int t_end = min((Lq + QT - 1) / QT, t_begin + tpi);
        const uint32_t tile_bytes = QT * D * kE;

        // Tile t into buffer b = (t - t_begin) % 3: Q rows (all waves share the copy) and its
        // -lse2 (4 bytes per lane; every wave writes the same values, so the
        // per-wave load counts match and the copy needs no extra synchronisation).
        // Tiles past the last are issued with an offset outside the resources
        // (no data moves), as in imp_lse_kernel.
        auto issue = [&](auto b, int t) {
            const bool real = t < t_end;
            Tile::issue(qrs, real ? (uint32_t)t * tile_bytes : kNoRecord, lds(b), wave, lane);
            const int qi = t * QT + (lane < QT ? lane : 0);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(nrs, nl_lds(b), 4, real ? (uint32_t)qi * 4 : kNoRecord, 0, 0, 0);
        };
        issue(Buf<0>{}, t_begin);
        issue(Buf<1>{}, t_begin + 1);  // (out of range when there is one tile)

        // K fragments, the register operand: key (lane%32 of the wave's 32),
        // depth 16*kk + 8*half .. +8.  They supply the rows of every product, so
        // acc[r] is key row 8*(r/4) + 4*half + r%4 and query lane%32 of the
        // streamed 32-row block, and a query's -lse2 is one value per lane.
        Frag8<DT> kf[NKK];
    #pragma unroll
        for (int kk = 0; kk < NKK; ++kk) {
            if (key < Lk) kf[kk].load(Kh + ((size_t)key * D + 16 * kk + 8 * half) * kE);
            else kf[kk].zero();
        }
        if (u != nullptr && qs == 0)
            redundancy_of_keys<DT, D>(kf, u + (size_t)h * D, key, lane, Lk, r_out + (size_t)h * Lk,
                                      red_part + (size_t)h * nkb + kblk);
        wait_vmcnt<L>();  // tile 0 landed (tile 1 may be in flight)
        tile_barrier();

        // Per key row r: this lane's share of sum_i exp2(x_ij - lse2_i).  Rows
        // past L_q are zero in Q and -inf in -lse2, so they add nothing.
        float cs[16];
    #pragma unroll
        for (int r = 0; r < 16; ++r) cs[r] = 0.f;
        auto acc_rows = [&](const f32x16_t& acc, float nl, int r0, int nr) {
    #pragma unroll
            for (int r = r0; r < r0 + nr; ++r) cs[r] += exp2_hw(fmaf(acc[r], c, nl));
        };
        // As in imp_lse_kernel, the second block of tile t is finished in the MFMA
        // shadow of the first block of tile t+1 (carry, with its -lse2 value).
        f32x16_t carry;
    #pragma unroll
        for (int r = 0; r < 16; ++r) carry[r] = 0.f;
        float nl_carry = -INFINITY;  // adds 0
        auto step = [&](auto b, int t) {
            constexpr int B = decltype(b)::value;
            issue(Buf<(B + 2) % kNBuf>{}, t + 2);
            const char* buf = lds(b);
            const float nl_a = nl_lds(b)[lane & 31];
            f32x16_t a0;
            mfma_block<DT, D, QT, true>(a0, buf, 0, fo, kf, [&](int r0, int nr) { acc_rows(carry, nl_carry, r0, nr); });
            if constexpr (QT == 64) {
                const float nl_b = nl_lds(b)[32 + (lane & 31)];
                mfma_block<DT, D, QT, true>(carry, buf, 32, fo, kf, [&](int r0, int nr) { acc_rows(a0, nl_a, r0, nr); });
                nl_carry = nl_b;
            } else {
                carry = a0;
                nl_carry = nl_a;
            }
            wait_vmcnt<L>();
            tile_barrier();
        };
        // Whole rounds of three tiles, then the tail: the loop's back edge then
        // only follows a buffer-2 step, so the compiler sees on every path which
        // loads the explicit waits have retired and adds no waits of its own.
        int t = t_begin;
        for (; t + 2 < t_end; t += kNBuf) {
            step(Buf<0>{}, t);
            step(Buf<1>{}, t + 1);
            step(Buf<2>{}, t + 2);
        }
        if (t < t_end) {
            step(Buf<0>{}, t);
            if (t + 1 < t_end) step(Buf<1>{}, t + 1);
        }
        wait_vmcnt<0>();
        acc_rows(carry, nl_carry, 0, 16);

        // Sum each key row over the 32 query lanes of its half (fixed butterfly
        // order), then lane r of each half writes row r.
        float v = 0.f;
    #pragma unroll
        for (int r = 0; r < 16; ++r) {
            float x = cs[r];
    #pragma unroll
            for (int o = 16; o >= 1; o >>= 1) x += __shfl_xor(x, o, kWave);
            if ((lane & 31) == r) v = x;
        }
        const int kr = kblk * kRowsPerBlock + wave * 32 + 8 * ((lane & 15) >> 2) + 4 * half + (lane & 3);
        // partial importance of this query range: plane qs of [nqs][H][Lk]
        if ((lane & 31) < 16 && kr < Lk) imp[((size_t)qs * H + h) * Lk + kr] = v * inv_lq;

    };
    // one item per workgroup, or persistent workgroups over XCD-owned
    // ranges of items (see pass 1)
    const int it = xcd_item((n_items + 7) / 8);
    work_loop<kPersist>(queue, n_items, 0, it < n_items ? it : -1, run);
}

template <int DT, int D>
hipError_t lse_launch(const void* Q, const void* K, float2* part, int H, int Lq, int Lk, const ImpPlan& p,
                      float c, hipStream_t s, float* u_part, int nbu, uint32_t* queue, int ldk) {
    static_assert(kThreads / kWave * D * 4 <= SwizzledTile<DT, D, tile_rows<DT>()>::kBytes,
                  "redundancy scratch must fit in one tile buffer");
    const int nqb = (Lq + kRowsPerBlock - 1) / kRowsPerBlock;
    const long long n_items = (long long)H * p.nsplit * nqb;
    const int lse_blocks = (int)((n_items + 7) / 8 * 8);
    const int red_blocks = u_part != nullptr ? H * nbu : 0;
    if (queue != nullptr && p.persistent_lse)  // one workgroup per slot
        hipLaunchKernelGGL((imp_lse_kernel<DT, D, true>), dim3(p.slots_lse / 8 * 8), dim3(kThreads), 0, s, Q, K,
                           part, Lq, Lk, ldk, p.keys_per_split, p.nsplit, nqb, (int)n_items, c, u_part, nbu, lse_blocks,
                           queue, H);
    else
        hipLaunchKernelGGL((imp_lse_kernel<DT, D, false>), dim3(lse_blocks + red_blocks), dim3(kThreads), 0, s, Q, K,
                           part, Lq, Lk, ldk, p.keys_per_split, p.nsplit, nqb, (int)n_items, c, u_part, nbu, lse_blocks,
                           nullptr, H);
    return hipGetLastError();
}

template <int DT, int D>
hipError_t colsum_launch(const void* Q, const void* K, const float* nlse2, float* imp_part, int H, int Lq, int Lk,
                         const ImpPlan& p, float c, hipStream_t s, const float* u, float* r, float2* red_part,
                         uint32_t* queue, int ldk) {
    const int nkb = (Lk + kRowsPerBlock - 1) / kRowsPerBlock;
    const long long n_items = (long long)H * p.nqs * nkb;
    const int blocks = (int)((n_items + 7) / 8 * 8);
    if (queue != nullptr && p.persistent_colsum)  // one workgroup per slot
        hipLaunchKernelGGL((imp_colsum_kernel<DT, D, true>), dim3(p.slots_colsum / 8 * 8), dim3(kThreads), 0, s, Q,
                           K, nlse2, imp_part, H, Lq, imp_lq_pad(Lq), Lk, ldk, nkb, p.nqs, p.qtiles_per_split, (int)n_items,
                           c, 1.0f / (float)Lq, u, r, red_part, queue);
    else
        hipLaunchKernelGGL((imp_colsum_kernel<DT, D, false>), dim3(blocks), dim3(kThreads), 0, s, Q, K, nlse2,
                           imp_part, H, Lq, imp_lq_pad(Lq), Lk, ldk, nkb, p.nqs, p.qtiles_per_split, (int)n_items, c,
                           1.0f / (float)Lq, u, r, red_part, nullptr);
    return hipGetLastError();
}

// Workgroups of a kernel that fit on one CU at once (at least 1).
template <typename Kern>
int occupancy(Kern kern) {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kern, kThreads, 0) != hipSuccess || n < 1) n = 1;
    return n;
}

// Concurrent workgroup slots of the two importance passes on the current
// device, cached per device and variant.
struct Slots {
    int lse, colsum;
};
Slots imp_slots(int dt, int d) {
    constexpr int kMaxDev = 64;
    static std::atomic<int> cache[kMaxDev][2][2][2];  // 0 = not computed yet
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDev) dev = 0;
    const int di = dt == kBF16 ? 1 : 0, dd = d == 128 ? 1 : 0;
    int a = cache[dev][di][dd][0].load(), b = cache[dev][di][dd][1].load();
    if (a == 0 || b == 0) {
        int cus = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1) cus = 1;
        int ol, oc;
        if (dt == kBF16) {
            ol = d == 128 ? occupancy(imp_lse_kernel<kBF16, 128, false>) : occupancy(imp_lse_kernel<kBF16, 64, false>);
            oc = d == 128 ? occupancy(imp_colsum_kernel<kBF16, 128, false>) : occupancy(imp_colsum_kernel<kBF16, 64, false>);
        } else {
            ol = d == 128 ? occupancy(imp_lse_kernel<kF32, 128, false>) : occupancy(imp_lse_kernel<kF32, 64, false>);
            oc = d == 128 ? occupancy(imp_colsum_kernel<kF32, 128, false>) : occupancy(imp_colsum_kernel<kF32, 64, false>);
        }
        a = cus * ol;
        b = cus * oc;
        cache[dev][di][dd][0].store(a);
        cache[dev][di][dd][1].store(b);
    }
    return Slots{a, b};
}

// Split n_tiles tiles of work per (item group) into parts, choosing the
// count that minimises (rounds of the grid) x (tiles per part + overhead):
// a partial last round of workgroups costs a whole round.
void choose_split(long long groups, int n_tiles, int min_tiles, int max_parts, int slots, int* parts,
                  int* tiles_per_part) {
    constexpr double kOverheadTiles = 2.0;  // prologue and epilogue of a workgroup, in tiles
    int best_p = 1, best_t = n_tiles;
    double best = 1e300;
    int p_max = n_tiles / (min_tiles > 0 ? min_tiles : 1);
    if (p_max < 1) p_max = 1;
    if (p_max > max_parts) p_max = max_parts;
    for (int p = 1; p <= p_max; ++p) {
        const int t = (n_tiles + p - 1) / p;
        const int p_eff = (n_tiles + t - 1) / t;  // every part non-empty
        const long long items = groups * p_eff;
        const long long rounds = (items + slots - 1) / slots;
        const double cost = (double)rounds * (t + kOverheadTiles);
        if (cost < best - 1e-9) {
            best = cost;
            best_p = p_eff;
            best_t = t;
        }
    }
    *parts = best_p;
    *tiles_per_part = best_t;
}

}  // namespace

int imp_lq_pad(int Lq) { return (Lq + 63) / 64 * 64; }

ImpPlan imp_plan(int H, int Lq, int Lk, int dt, int d) {
    const int kt = dt == kBF16 ? tile_rows<kBF16>() : tile_rows<kF32>();
    const Slots sl = imp_slots(dt, d);
    ImpPlan p{};
    // pass 1: key ranges of whole K tiles (>= 4 tiles each)
    int kps_tiles;
    choose_split((long long)H * ((Lq + kRowsPerBlock - 1) / kRowsPerBlock), (Lk + kt - 1) / kt, 4, 1 << 20,
                 sl.lse, &p.nsplit, &kps_tiles);
    p.keys_per_split = kps_tiles * kt;
    p.slots_lse = sl.lse;
    p.slots_colsum = sl.colsum;
    // Persistent pass 1 when finer key ranges give at least kPersistRounds
    // items per workgroup slot (ranges of >= 32 tiles): the XCDs run at
    // different clocks, and items handed out by counters let the faster ones
    // do more.  Measured on the long-video shape: 1.5 % off the importance
    // stage with pass 2 persistent too; a few rounds (the MAGI-like shape) lose.
    {
        const long long hq = (long long)H * ((Lq + kRowsPerBlock - 1) / kRowsPerBlock);
        const int tiles = (Lk + kt - 1) / kt;
        long long ns = ((long long)kPersistRounds * sl.lse + hq - 1) / hq;
        if (ns > tiles / 32) ns = tiles / 32;
        if (ns >= p.nsplit && hq * ns >= (long long)kPersistRounds * sl.lse) {
            const int t = (tiles + (int)ns - 1) / (int)ns;
            p.nsplit = (tiles + t - 1) / t;
            p.keys_per_split = t * kt;
            p.persistent_lse = true;
        }
    }
    // pass 2: one range of queries per key block when the key blocks alone
    // fill the device's workgroup slots; otherwise just enough query ranges
    // (whole Q tiles, >= 4 each, at most kMaxQSplit) to fill them
    const long long groups = (long long)H * ((Lk + kRowsPerBlock - 1) / kRowsPerBlock);
    const int qtiles = (Lq + kt - 1) / kt;
    long long parts = groups >= sl.colsum ? 1 : sl.colsum / groups;
    if (parts > qtiles / 4) parts = qtiles / 4;
    if (parts > kMaxQSplit) parts = kMaxQSplit;
    if (parts < 1) parts = 1;
    p.qtiles_per_split = (int)((qtiles + parts - 1) / parts);
    p.nqs = (qtiles + p.qtiles_per_split - 1) / p.qtiles_per_split;  // every range non-empty
    p.persistent_colsum = groups * p.nqs >= (long long)kPersistRounds * sl.colsum;
    return p;
}

hipError_t launch_imp_lse(int dt, int d, const void* Q, const void* K, float2* part, int H, int Lq, int Lk,
                          const ImpPlan& plan, float c, hipStream_t s, float* u_part, int nbu, uint32_t* queue,
                          int ldk) {
    if (ldk < Lk) ldk = Lk;
    if (dt == kBF16)
        return d == 128 ? lse_launch<kBF16, 128>(Q, K, part, H, Lq, Lk, plan, c, s, u_part, nbu, queue, ldk)
                        : lse_launch<kBF16, 64>(Q, K, part, H, Lq, Lk, plan, c, s, u_part, nbu, queue, ldk);
    return d == 128 ? lse_launch<kF32, 128>(Q, K, part, H, Lq, Lk, plan, c, s, u_part, nbu, queue, ldk)
                    : lse_launch<kF32, 64>(Q, K, part, H, Lq, Lk, plan, c, s, u_part, nbu, queue, ldk);
}

int imp_colsum_blocks(int Lk) { return (Lk + kRowsPerBlock - 1) / kRowsPerBlock; }

bool imp_grids_fit(int H, int Lq, int Lk, const ImpPlan& p, int nbu) {
    // one-dimensional grids: a dispatch counts its work-items in 32 bits
    const long long nqb = (Lq + kRowsPerBlock - 1) / kRowsPerBlock;
    const long long lse = ((long long)H * p.nsplit * nqb + 7) / 8 * 8 + (long long)H * nbu;
    const long long col = ((long long)H * p.nqs * imp_colsum_blocks(Lk) + 7) / 8 * 8;
    return lse * kThreads < (1LL << 32) && col * kThreads < (1LL << 32);
}

hipError_t launch_imp_colsum(int dt, int d, const void* Q, const void* K, const float* nlse2, float* imp_part, int H,
                             int Lq, int Lk, const ImpPlan& p, float c, hipStream_t s, const float* u, float* r,
                             float2* red_part, uint32_t* queue, int ldk) {
    if (ldk < Lk) ldk = Lk;
    if (dt == kBF16)
        return d == 128
                   ? colsum_launch<kBF16, 128>(Q, K, nlse2, imp_part, H, Lq, Lk, p, c, s, u, r, red_part, queue, ldk)
                   : colsum_launch<kBF16, 64>(Q, K, nlse2, imp_part, H, Lq, Lk, p, c, s, u, r, red_part, queue, ldk);
    return d == 128 ? colsum_launch<kF32, 128>(Q, K, nlse2, imp_part, H, Lq, Lk, p, c, s, u, r, red_part, queue, ldk)
                    : colsum_launch<kF32, 64>(Q, K, nlse2, imp_part, H, Lq, Lk, p, c, s, u, r, red_part, queue, ldk);
}

hipError_t launch_imp_lse_merge(const float2* part, float* lse, float* nlse2, int H, int Lq, int nsplit,
                                hipStream_t s, const float* u_part, int nbu, float* u, int d) {
    const int lq_pad = imp_lq_pad(Lq);
    hipLaunchKernelGGL(imp_lse_merge_kernel, dim3((lq_pad + kSmallThreads - 1) / kSmallThreads, H),
                       dim3(kSmallThreads), 0, s, part, lse, nlse2, Lq, lq_pad, nsplit, u_part, nbu, u, d);
    return hipGetLastError();
}

hipError_t launch_imp_sum_planes(const float* part, float* imp, int H, int Lk, int nqs, hipStream_t s) {
    const size_t n = (size_t)H * Lk;
    size_t blocks = (n + kSmallThreads - 1) / kSmallThreads;
    if (blocks > 4096) blocks = 4096;
    hipLaunchKernelGGL(imp_sum_planes_kernel, dim3((unsigned)blocks), dim3(kSmallThreads), 0, s, part, imp, n, nqs);
    return hipGetLastError();
}

hipError_t launch_imp_queue_zero(uint32_t* queue, hipStream_t s) {
    hipLaunchKernelGGL(imp_queue_zero_kernel, dim3(1), dim3(kWave), 0, s, queue);
    return hipGetLastError();
}

hipError_t launch_imp_nlse2(const float* lse, float* nlse2, int H, int Lq, hipStream_t s) {
    const int lq_pad = imp_lq_pad(Lq);
    hipLaunchKernelGGL(imp_nlse2_kernel, dim3((lq_pad + kSmallThreads - 1) / kSmallThreads, H), dim3(kSmallThreads),
                       0, s, lse, nlse2, Lq, lq_pad);
    return hipGetLastError();
}

}  // namespace fc
