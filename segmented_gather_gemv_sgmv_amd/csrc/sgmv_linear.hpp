// sgmv_linear.hpp -- an adapted linear layer in one pass over its output:
//
//     y = round( x W^T + bias + scale * (x A_a) B_a ),   a = adapter of the row
//
// i.e. the layer y = xW + xAB of Punica walkthrough (omica.com.cn/news/959180,
// section 2.1) with the base product and the LoRA correction fused, as
// aivaro.ru answer 959 (section 3.2) describes: the correction is added to
// the base tile while it is still in registers, so y is written once and
// never read.  W is stored [H2][H1] (one row of weights per output feature),
// which makes both operands of the base product K-contiguous.
//
// The rank-r intermediate v = x A_a has to be complete for a row before its
// correction, and it needs all of H1, so it comes from the shrink launch
// that precedes this kernel on the stream (its float32 chunk partials, summed
// here in chunk order).  This kernel then computes, per output tile of
// kBM x kBN:
//
//  * the base product on the matrix cores (v_mfma_f32_16x16x32_{f16,bf16},
//    float32 accumulation).  K advances in chunks of 64 staged through LDS,
//    double-buffered, with kD chunks of global loads in flight per thread
//    (a register ring) so that the skinny decode shapes, which stream W from
//    HBM and do little arithmetic per byte, keep enough bytes in flight.  In
//    LDS each 128-byte row keeps its 16-byte piece p at p ^ (row & 7), which
//    spreads the 16 rows an MFMA operand read touches over the banks.
//  * when the tile's K range is split over ksplit workgroups (decode shapes
//    have few tiles), each stores a float32 partial tile and the last one to
//    arrive -- counted on a per-tile counter that it returns to zero -- sums
//    the ksplit partials in a fixed order, so the bits do not depend on
//    which workgroup came last.
//  * the epilogue: the accumulator tile passes through LDS into row-
//    contiguous pieces of 8 columns; each piece adds scale * sum_k v[i][k]
//    B_a[k][cols] in float32 (16-byte B loads) and the bias, is rounded
//    once to the dtype and stored with one 16-byte store.  With a split K
//    range, the rank sum is split over the same workgroups (workgroup q adds
//    ranks [q*ceil(r/ksplit), ...)), so the B reads are spread over them.
//
// Operand layout of the 16x16x32 MFMA: lane l holds A[l % 16][8 (l / 16) + j]
// and B[8 (l / 16) + j][l % 16], j = 0..7, and receives D[4 (l / 16) + i]
// [l % 16], i = 0..3.  With A = a 16-row block of x and B[k][n] = W[n][k],
// both operands are 16-byte reads of 8 consecutive k from one row.
#pragma once

#include "sgmv_device.hpp"
#include "sgmv_fused.hpp"
#include "sgmv_mfma.hpp"

#include <type_traits>

namespace sgmv {

constexpr int kLinThreads = 256;
constexpr int kLinBK = 64;  // K per chunk: 8 pieces of 16 bytes per row
constexpr int kLinRG = 16;  // ranks per pass of the correction
constexpr int kLinSegLds = 1024;  // segment-table entries staged in LDS

template <int WM_, int WN_, int TM_, int TN_, int D_>
struct LinearShape {
    static constexpr int WM = WM_, WN = WN_;  // waves along rows and columns
    static constexpr int TM = TM_, TN = TN_;  // 16 x 16 blocks per wave
    static_assert(WM * WN * kWave == kLinThreads, "four waves per workgroup");
    static constexpr int kD = D_;                      // chunks of loads in flight
    static constexpr int kBM = WM * TM * 16;           // tile rows
    static constexpr int kBN = WN * TN * 16;           // tile columns
    static constexpr int kXP = kBM * 8 / kLinThreads;  // x pieces per thread and chunk
    static constexpr int kWP = kBN * 8 / kLinThreads;  // W pieces per thread and chunk
    static constexpr int kStage = (kBM + kBN) * kLinBK;  // 16-bit elements per buffer
    static constexpr int kTP = kBN + 4;                  // padded row of the float tile
    static constexpr int kPieces = kBM * kBN / 8 / kLinThreads;  // epilogue pieces per thread
    static constexpr int kLdsBytes =
        (2 * kStage * 2 > kBM * kTP * 4) ? 2 * kStage * 2 : kBM * kTP * 4;
    static_assert(kXP >= 1 && kWP >= 1 && kPieces >= 1, "tile too small for the workgroup");
    static_assert(kBM * 8 % kLinThreads == 0 && kBN * 8 % kLinThreads == 0, "uneven chunk");
    static_assert(kBM * kBN % (8 * kLinThreads) == 0, "uneven epilogue");
};

// Workgroup barrier for LDS hand-offs only.  __syncthreads() also waits for
// every outstanding global load of the wave (vmcnt(0)), which would drain
// the chunks in flight at every K step; this waits for the wave's LDS
// operations alone.  The memory clobber keeps the compiler from moving
// memory accesses across it; loads still in flight are waited for where
// their registers are used.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Adapter of row `row` (or -1 if no segment covers it or the segment's
// adapter id is outside [0, num_adapters)): the last segment starting at or
// before the row, if the row lies before its end.  Works on a global or an
// LDS copy of the table.
template <typename P>
__device__ __forceinline__ int row_adapter(P seg_indptr, P adapter_ids, int S, int row,
                                           int num_adapters) {
    int lo = 0, hi = S;
    while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (seg_indptr[mid] <= row) lo = mid + 1;
        else hi = mid;
    }
    const int s = lo - 1;
    if (s < 0 || row >= seg_indptr[s + 1]) return -1;
    const int a = adapter_ids[s];
    return (a >= 0 && a < num_adapters) ? a : -1;
}

// Ranks [k_lo, k_hi) of the correction handled by K range q of ksplit.
__device__ __forceinline__ void linear_rank_share(int r, int ksplit, int q, int& k_lo, int& k_hi) {
    const int rs = (r + ksplit - 1) / ksplit;
    k_lo = q * rs < r ? q * rs : r;
    k_hi = k_lo + rs < r ? k_lo + rs : r;
}

// The first pass of v for this workgroup's share of the ranks (its first
// kLinRG ranks), summed over the shrink's chunks in order, for every tile
// row below M.
template <bool kCoherent>
__device__ __forceinline__ void linear_prepare_v(float* s_v, const float* __restrict__ vpart,
                                                 long long vstride, int vsplit, int M, int r,
                                                 int ksplit, int q, int m0, int BM) {
    int k_lo, k_hi;
    linear_rank_share(r, ksplit, q, k_lo, k_hi);
    const int gn = k_hi - k_lo < kLinRG ? k_hi - k_lo : kLinRG;
    for (int e = threadIdx.x; e < BM * gn; e += kLinThreads) {
        const int il = e / gn, kk = e - il * gn;
        const float* p = vpart + (long long)(m0 + il) * r + k_lo + kk;
        float v = 0.f;
        if (m0 + il < M)
            v = kCoherent ? sum_partials_coherent(const_cast<float*>(p), vstride, vsplit)
                          : sum_partials(p, vstride, vsplit);
        s_v[il * kLinRG + kk] = v;
    }
}

// What the correction needs that does not depend on the base product, done
// before the main loop so that its round trips overlap the first chunks'
// loads: each tile row's adapter (s_aid) and the first pass of v (the
// workgroup's first kLinRG ranks, s_v, summed over the shrink's chunks in
// order).  v is summed for every row below M; rows without an adapter
// never use theirs.  The caller must make s_seg / s_ids visible first and
// synchronise before s_aid / s_v are read.
// With kCoherent, v's partials are read with agent-scope loads: they were
// published during this launch (the folded shrink) rather than by an
// earlier one.  kWithV = false leaves s_v to the caller.
template <bool kCoherent = false, bool kWithV = true>
__device__ __forceinline__ void linear_prepare(int* s_aid, float* s_v, const int* s_seg,
                                               const int* s_ids, bool seg_lds,
                                               const float* __restrict__ vpart, long long vstride,
                                               int vsplit, const int* __restrict__ seg_indptr,
                                               const int* __restrict__ adapter_ids, int S, int M,
                                               int num_adapters, int r, int ksplit, int q, int m0,
                                               int BM) {
    const int tid = threadIdx.x;
    for (int i = tid; i < BM; i += kLinThreads) {
        int a = -1;
        if (m0 + i < M)
            a = seg_lds ? row_adapter((const int*)s_seg, (const int*)s_ids, S, m0 + i, num_adapters)
                        : row_adapter(seg_indptr, adapter_ids, S, m0 + i, num_adapters);
        s_aid[i] = a;
    }
    if constexpr (kWithV)
        linear_prepare_v<kCoherent>(s_v, vpart, vstride, vsplit, M, r, ksplit, q, m0, BM);
}

// The part of an adapted-linear tile that follows the base product, shared
// by the tile kernels.  On entry s_t holds the tile's float32 base product
// for this workgroup's K range ([BM][TP], written by the caller; the barrier
// here makes it visible).  Finds each row's adapter, adds this workgroup's
// share of the ranks of scale * v B_a, combines the K ranges (the last
// workgroup of a tile to arrive sums them in a fixed order), adds the bias,
// rounds once and stores y.
// The B rows of the correction's first four ranks for this thread's
// epilogue pieces, as linear_finish reads them: loads that do not depend on
// v or on the base product, so a caller can issue them before waiting for
// either.
template <typename DT, int BM, int BN>
__device__ __forceinline__ void linear_prefetch_b(uint4 (&pre)[BM * BN / 8 / kLinThreads][4],
                                                  const int* s_aid,
                                                  const typename DT::storage* __restrict__ B_stack,
                                                  int H2, int r, int ksplit, int q, int n0) {
    constexpr int kPieces = BM * BN / 8 / kLinThreads;
    int k_lo, k_hi;
    linear_rank_share(r, ksplit, q, k_lo, k_hi);
    const int gn = k_hi - k_lo < kLinRG ? k_hi - k_lo : kLinRG;
#pragma unroll
    for (int u = 0; u < kPieces; ++u) {
        const int pid = threadIdx.x + u * kLinThreads;
        const int il = pid / (BN / 8), c8 = pid % (BN / 8);
        const int a = s_aid[il];
        const int col = n0 + c8 * 8;
        const bool on = a >= 0 && col < H2;
        const typename DT::storage* bp = B_stack + ((long long)(on ? a : 0) * r + k_lo) * H2 + col;
#pragma unroll
        for (int d = 0; d < 4; ++d)
            pre[u][d] = (on && d < gn) ? load16(bp + (long long)d * H2) : make_uint4(0, 0, 0, 0);
    }
}

// kPre: pre holds the first four ranks' B rows (linear_prefetch_b).
template <typename DT, int BM, int BN, int TP, bool kCoherent = false, bool kPre = false>
__device__ __forceinline__ void linear_finish(
    const float* s_t, int* s_aid, float* s_v, const int* s_seg, const int* s_ids, int* s_last,
    bool seg_lds, typename DT::storage* __restrict__ y,
    const typename DT::storage* __restrict__ bias,
    const typename DT::storage* __restrict__ B_stack, const float* __restrict__ vpart,
    long long vstride, int vsplit, const int* __restrict__ seg_indptr,
    const int* __restrict__ adapter_ids, int S, int M, int num_adapters, int H2, int r,
    float scale, float* __restrict__ part, int* __restrict__ counters, int counter_stride,
    int ksplit, int q, int t, int m0, int n0,
    const uint4 (&pre)[BM * BN / 8 / kLinThreads][4]) {
    constexpr int kPieces = BM * BN / 8 / kLinThreads;
    static_assert(BM * BN % (8 * kLinThreads) == 0, "uneven epilogue");
    const int tid = threadIdx.x;
    __syncthreads();  // the caller's s_t (s_aid and the first s_v are older)

    // ---- epilogue: row-contiguous pieces of 8 columns --------------------
    float val[kPieces][8];
#pragma unroll
    for (int u = 0; u < kPieces; ++u) {
        const int pid = tid + u * kLinThreads;
        const int il = pid / (BN / 8), c8 = pid % (BN / 8);
        const float4 lo = *reinterpret_cast<const float4*>(s_t + il * TP + c8 * 8);
        const float4 hi = *reinterpret_cast<const float4*>(s_t + il * TP + c8 * 8 + 4);
        val[u][0] = lo.x; val[u][1] = lo.y; val[u][2] = lo.z; val[u][3] = lo.w;
        val[u][4] = hi.x; val[u][5] = hi.y; val[u][6] = hi.z; val[u][7] = hi.w;
    }

    // The correction for ranks [k_lo, k_hi): this workgroup's share.  The
    // first pass's v came from linear_prepare; later passes (shares above
    // kLinRG ranks) sum theirs here.
    int k_lo, k_hi;
    linear_rank_share(r, ksplit, q, k_lo, k_hi);
    for (int g0 = k_lo; g0 < k_hi; g0 += kLinRG) {
        const int gn = k_hi - g0 < kLinRG ? k_hi - g0 : kLinRG;
        if (g0 > k_lo) {
            __syncthreads();  // s_v free (previous pass done)
            for (int e = tid; e < BM * gn; e += kLinThreads) {
                const int il = e / gn, kk = e - il * gn;
                float sum = 0.f;
                if (s_aid[il] >= 0) {
                    // chunk order, eight loads in flight
                    const float* p = vpart + (long long)(m0 + il) * r + g0 + kk;
                    sum = kCoherent ? sum_partials_coherent(const_cast<float*>(p), vstride, vsplit)
                                    : sum_partials(p, vstride, vsplit);
                }
                s_v[il * kLinRG + kk] = sum;
            }
            __syncthreads();
        }
#pragma unroll
        for (int u = 0; u < kPieces; ++u) {
            const int pid = tid + u * kLinThreads;
            const int il = pid / (BN / 8), c8 = pid % (BN / 8);
            const int a = s_aid[il];
            const int col = n0 + c8 * 8;
            if (a < 0 || col >= H2) continue;
            const typename DT::storage* bp = B_stack + ((long long)a * r + g0) * H2 + col;
            float ls[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
            // ranks in order, four B rows in flight at a time
            for (int k0 = 0; k0 < gn; k0 += 4) {
                uint4 braw[4];
                if (kPre && g0 == k_lo && k0 == 0) {
#pragma unroll
                    for (int d = 0; d < 4; ++d) braw[d] = pre[u][d];
                } else {
#pragma unroll
                    for (int d = 0; d < 4; ++d)
                        braw[d] = k0 + d < gn ? load16(bp + (long long)(k0 + d) * H2)
                                              : make_uint4(0, 0, 0, 0);
                }
#pragma unroll
                for (int d = 0; d < 4; ++d) {
                    if (k0 + d < gn) {
                        float bv[8];
                        DT::unpack(braw[d], bv);
                        const float vk = s_v[il * kLinRG + k0 + d];
#pragma unroll
                        for (int j = 0; j < 8; ++j) ls[j] = fmaf(vk, bv[j], ls[j]);
                    }
                }
            }
#pragma unroll
            for (int j = 0; j < 8; ++j) val[u][j] = fmaf(scale, ls[j], val[u][j]);
        }
    }

    // ---- combine the K ranges, add the bias, round, store ------------------
    // A partial tile is stored as 8 planes of BM * BN / 8 floats, plane j
    // holding column j of every piece, so that each store and load
    // instruction of a wave covers consecutive words.
    constexpr int kPlane = BM * BN / 8;
    const long long tile_floats = (long long)BM * BN;
    if (ksplit > 1) {
        float* mine = part + ((long long)t * ksplit + q) * tile_floats;
#pragma unroll
        for (int u = 0; u < kPieces; ++u) {
            const int pid = tid + u * kLinThreads;
            const int il = pid / (BN / 8), c8 = pid % (BN / 8);
            if (m0 + il >= M || n0 + c8 * 8 >= H2) continue;
#pragma unroll
            for (int j = 0; j < 8; ++j) store_partial(mine + j * kPlane + pid, val[u][j]);
        }
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();  // every wave's partial stores have completed
        if (tid == 0) {
            int* cnt = counters + (long long)t * counter_stride;
            const int before =
                __hip_atomic_fetch_add(cnt, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            const int last = before == ksplit - 1;
            if (last) __hip_atomic_store(cnt, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            *s_last = last;
        }
        __syncthreads();
        if (!*s_last) return;
        const float* tp = part + (long long)t * ksplit * tile_floats;
#pragma unroll
        for (int u = 0; u < kPieces; ++u) {
            const int pid = tid + u * kLinThreads;
            const int il = pid / (BN / 8), c8 = pid % (BN / 8);
            if (m0 + il >= M || n0 + c8 * 8 >= H2) continue;
            float sum[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
            // K ranges in order, the other ranges' partials four at a time
            // with all their loads in flight (one round trip per four).
            for (int c0 = 0; c0 < ksplit; c0 += 4) {
                float pv[4][8];
#pragma unroll
                for (int d = 0; d < 4; ++d) {
                    const int c = c0 + d;
                    float* p = const_cast<float*>(tp) + c * tile_floats + pid;
#pragma unroll
                    for (int j = 0; j < 8; ++j)
                        pv[d][j] = (c < ksplit && c != q)
                                       ? __hip_atomic_load(p + j * kPlane, __ATOMIC_RELAXED,
                                                           __HIP_MEMORY_SCOPE_AGENT)
                                       : val[u][j];
                }
#pragma unroll
                for (int d = 0; d < 4; ++d)
                    if (c0 + d < ksplit) {
#pragma unroll
                        for (int j = 0; j < 8; ++j) sum[j] += pv[d][j];
                    }
            }
#pragma unroll
            for (int j = 0; j < 8; ++j) val[u][j] = sum[j];
        }
    }
#pragma unroll
    for (int u = 0; u < kPieces; ++u) {
        const int pid = tid + u * kLinThreads;
        const int il = pid / (BN / 8), c8 = pid % (BN / 8);
        const int row = m0 + il, col = n0 + c8 * 8;
        if (row >= M || col >= H2) continue;
        if (bias) {
            float bv[8];
            DT::unpack(load16(bias + col), bv);
#pragma unroll
            for (int j = 0; j < 8; ++j) val[u][j] += bv[j];
        }
        store16(y + (long long)row * H2 + col, DT::pack(val[u]));
    }
}

// One row's partial sum of v = x A_a over [h_lo, h_hi) (multiples of 8) on
// the matrix cores, staged through s_raw (32 KB): one LDS chunk of A
// (shrink_chunk_mfma) or, for longer ranges, the streaming form
// (shrink_long_mfma).  Calls emit(k, value) once per k < R from thread k;
// an empty range emits nothing.  The shrink workgroups and the fallback
// both take their partials from here, so their bits agree.
template <typename DT, int R, typename Emit>
__device__ __forceinline__ void linear_row_partial(const typename DT::storage* __restrict__ A,
                                                   const typename DT::storage* __restrict__ xr,
                                                   int H1, int h_lo, int h_hi,
                                                   unsigned char* s_raw, Emit&& emit) {
    constexpr int KC = 16384 / R < 512 ? 16384 / R : 512;  // A chunk within 32 KB of LDS
    uint16_t* s_a = reinterpret_cast<uint16_t*>(s_raw);
    float* s_red = reinterpret_cast<float*>(s_raw);
    auto e = [&](int, int k, float v) { emit(k, v); };
    if (h_hi <= h_lo) return;
    if (h_hi - h_lo <= KC)
        shrink_chunk_mfma<DT, R, true, KC>(A, xr, 1, H1, h_lo, h_hi, s_a, s_red, e);
    else
        shrink_long_mfma<DT, R, KC>(A, xr, 1, H1, h_lo, h_hi, s_a, s_red, e);
}

// A shrink workgroup of the one-launch layer (decode shapes): item s is
// row s / ksplit over K range s % ksplit -- the ranges the tile workgroups
// split W over -- and publishes that partial of the row's v (zeros for a
// row without an adapter), then counts itself in on fold_cnt.  It never
// waits, and the shrink workgroups come first in the grid, so the tile
// workgroups that wait for them always see them finish.
template <typename DT>
__device__ __forceinline__ void linear_shrink_item(
    int s, const typename DT::storage* __restrict__ x,
    const typename DT::storage* __restrict__ A_stack, float* __restrict__ vpart,
    long long vstride, const int* __restrict__ seg_indptr, const int* __restrict__ adapter_ids,
    int S, int M, int num_adapters, int H1, int r, int ksplit, int chunks_per_split,
    unsigned char* s_raw, float* s_fv, int* s_seg, int* s_ids, int* s_row_aid, int* fold_cnt,
    int fold_total) {
    const int tid = threadIdx.x;
    const int row = s / ksplit, qq = s - row * ksplit;
    // The row's adapter: the table through LDS (one coalesced read) when it
    // fits, else a search in global memory.
    if (S <= kLinSegLds) {
        for (int e = tid; e <= S; e += kLinThreads) s_seg[e] = seg_indptr[e];
        for (int e = tid; e < S; e += kLinThreads) s_ids[e] = adapter_ids[e];
        __syncthreads();
        if (tid == 0)
            *s_row_aid = row < M ? row_adapter((const int*)s_seg, (const int*)s_ids, S, row,
                                               num_adapters)
                                 : -1;
    } else if (tid == 0) {
        *s_row_aid = row < M ? row_adapter(seg_indptr, adapter_ids, S, row, num_adapters) : -1;
    }
    __syncthreads();
    const int a = *s_row_aid;
    const int h_lo = qq * chunks_per_split * kLinBK;
    const int h_hi = min(H1, h_lo + chunks_per_split * kLinBK);
    float* out = vpart + (long long)qq * vstride + (long long)row * r;
    auto emit = [&](int k, float v) { s_fv[k] = v; };
    if (a >= 0) {
        const typename DT::storage* xr = x + (long long)row * H1;
        switch (r) {
            case 16:
                linear_row_partial<DT, 16>(A_stack + (long long)a * H1 * 16, xr, H1, h_lo, h_hi,
                                           s_raw, emit);
                break;
            case 32:
                linear_row_partial<DT, 32>(A_stack + (long long)a * H1 * 32, xr, H1, h_lo, h_hi,
                                           s_raw, emit);
                break;
            case 64:
                linear_row_partial<DT, 64>(A_stack + (long long)a * H1 * 64, xr, H1, h_lo, h_hi,
                                           s_raw, emit);
                break;
            default:
                linear_row_partial<DT, 128>(A_stack + (long long)a * H1 * 128, xr, H1, h_lo,
                                            h_hi, s_raw, emit);
                break;
        }
    }
    // Each value was written by the thread that stores it (emit(k) is
    // called from thread k).
    if (row < M)
        for (int k = tid; k < r; k += kLinThreads)
            store_partial(out + k, (a >= 0 && h_hi > h_lo) ? s_fv[k] : 0.f);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();  // every wave's partial stores have completed
    if (tid == 0) depart(fold_cnt, 1, fold_total);
}

// The folded shrink's fallback when its wait gives up: v for the tile's
// rows and this workgroup's first pass of ranks, from x and A with the
// shrink workgroups' arithmetic -- each K range's partial by
// linear_row_partial, then the partials added in K-range order starting
// from zero, as linear_prepare_v sums them -- so the result does not depend
// on whether the wait succeeded.  Slow (one row and one K range at a time);
// it uses the staging buffers, so it runs between the main loop and the
// tile.
template <typename DT, int R>
__device__ __forceinline__ void linear_v_refold(
    float* s_v, float* s_fv, const int* s_aid, const typename DT::storage* __restrict__ x,
    const typename DT::storage* __restrict__ A_stack, unsigned char* s_raw, int M, int H1,
    int m0, int BM, int ksplit, int chunks_per_split, int q) {
    const int tid = threadIdx.x;
    int k_lo, k_hi;
    linear_rank_share(R, ksplit, q, k_lo, k_hi);
    const int gn = k_hi - k_lo < kLinRG ? k_hi - k_lo : kLinRG;
    for (int il = 0; il < BM; ++il) {
        const int a = m0 + il < M ? s_aid[il] : -1;
        float sum = 0.f;  // thread k < R: rank k of this row
        if (a >= 0) {
            const typename DT::storage* A = A_stack + (long long)a * H1 * R;
            const typename DT::storage* xr = x + (long long)(m0 + il) * H1;
            for (int qq = 0; qq < ksplit; ++qq) {
                const int h_lo = qq * chunks_per_split * kLinBK;
                const int h_hi = min(H1, h_lo + chunks_per_split * kLinBK);
                linear_row_partial<DT, R>(A, xr, H1, h_lo, h_hi, s_raw,
                                          [&](int k, float v) { s_fv[k] = v; });
                if (tid < R) sum += h_hi > h_lo ? s_fv[tid] : 0.f;
                __syncthreads();  // s_fv read before the next range writes it
            }
        }
        if (tid >= k_lo && tid < k_lo + gn) s_v[il * kLinRG + tid - k_lo] = sum;
    }
}

// Grid: tiles * ksplit workgroups (rounded up; the extra ones return at
// once), workgroup b taking K range q = b % ksplit of tile b / ksplit.  With
// ksplit a multiple of the 8 XCDs, which receive workgroups round-robin,
// every XCD then streams one K range of x for all tiles.
//
// kFold: the shrink runs inside this launch.  The first n_shrink workgroups
// are shrink workgroups (linear_shrink_item; v's partials are then the K
// ranges', vsplit == ksplit) and count themselves in on fold_cnt (low 16
// bits); each tile workgroup after them waits for all of them once its
// main loop is done, reads its v, and counts itself out (high bits; the
// participant completing the total returns the counter to zero).  Past
// wait_ticks a tile workgroup recomputes its v (linear_v_refold, same
// bits) and raises the sticky flag.
template <typename DT, typename SH, bool kFold = false>
__global__ __launch_bounds__(kLinThreads) void linear_lora_kernel(
    typename DT::storage* __restrict__ y, const typename DT::storage* __restrict__ x,
    const typename DT::storage* __restrict__ W, const typename DT::storage* __restrict__ bias,
    const typename DT::storage* __restrict__ B_stack, const float* __restrict__ vpart,
    long long vstride, int vsplit, const int* __restrict__ seg_indptr,
    const int* __restrict__ adapter_ids, int S, int M, int num_adapters, int H1, int H2, int r,
    float scale, float* __restrict__ part, int* __restrict__ counters, int counter_stride,
    int ksplit, int chunks_per_split, int tiles_n, int tiles,
    const typename DT::storage* __restrict__ A_stack, int* __restrict__ fold_cnt,
    int* __restrict__ flag, long long wait_ticks, int n_shrink) {
    constexpr int BM = SH::kBM, BN = SH::kBN, XP = SH::kXP, WP = SH::kWP, PD = SH::kD;
    constexpr int TM = SH::TM, TN = SH::TN, TP = SH::kTP;
    __shared__ __attribute__((aligned(16))) unsigned char s_raw[SH::kLdsBytes];
    __shared__ int s_aid[BM];
    __shared__ float s_v[BM * kLinRG];
    __shared__ int s_seg[kLinSegLds + 1];
    __shared__ int s_ids[kLinSegLds];
    __shared__ int s_last;
    __shared__ int s_fold_ok;
    __shared__ float s_fv[kFold ? 128 : 1];  // one row's v partial (folded shrink)
    __shared__ int s_row_aid;
    uint16_t* s_stage = reinterpret_cast<uint16_t*>(s_raw);
    float* s_t = reinterpret_cast<float*>(s_raw);

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wid = tid / kWave;
    const int fold_total = n_shrink + (((int)gridDim.x - n_shrink) << 16);
    if constexpr (kFold) {
        if ((int)blockIdx.x < n_shrink) {
            linear_shrink_item<DT>((int)blockIdx.x, x, A_stack, const_cast<float*>(vpart),
                                   vstride, seg_indptr, adapter_ids, S, M, num_adapters, H1, r,
                                   ksplit, chunks_per_split, s_raw, s_fv, s_seg, s_ids,
                                   &s_row_aid, fold_cnt, fold_total);
            return;
        }
    }
    const unsigned b = blockIdx.x - (unsigned)n_shrink;
    const int q = (int)(b % (unsigned)ksplit);
    const int t = (int)(b / (unsigned)ksplit);
    if (t >= tiles) return;  // whole workgroup (never in the folded grid, which is exact)
    const int m0 = (t / tiles_n) * BM;
    const int n0 = (t % tiles_n) * BN;
    const int k_begin = q * chunks_per_split * kLinBK;
    int k_end = k_begin + chunks_per_split * kLinBK;
    if (k_end > H1) k_end = H1;
    const int nchunks = k_end > k_begin ? (k_end - k_begin + kLinBK - 1) / kLinBK : 0;

    // The segment table (when it fits LDS) is loaded up front, beside the
    // first chunks: the epilogue then finds each row's adapter in LDS rather
    // than by a chain of dependent global loads.
    const bool seg_lds = S > 0 && S <= kLinSegLds;  // no table is read when S == 0
    constexpr int kSegU = (kLinSegLds + 1 + kLinThreads - 1) / kLinThreads;
    int seg_r[kSegU], ids_r[kSegU];
#pragma unroll
    for (int u = 0; u < kSegU; ++u) {
        const int e = tid + u * kLinThreads;
        seg_r[u] = (seg_lds && e <= S) ? seg_indptr[e] : 0;
        ids_r[u] = (seg_lds && e < S) ? adapter_ids[e] : -1;
    }

    // ---- base product ----------------------------------------------------
    uint4 ring[PD][XP + WP];
    auto load_chunk = [&](int c, uint4(&dst)[XP + WP]) {
        const int k0 = k_begin + c * kLinBK;
#pragma unroll
        for (int u = 0; u < XP; ++u) {
            const int id = tid + u * kLinThreads;
            const int row = id >> 3, gk = k0 + (id & 7) * 8;
            dst[u] = (m0 + row < M && gk < k_end) ? load16(x + (long long)(m0 + row) * H1 + gk)
                                                  : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int u = 0; u < WP; ++u) {
            const int id = tid + u * kLinThreads;
            const int row = id >> 3, gk = k0 + (id & 7) * 8;
            dst[XP + u] = (n0 + row < H2 && gk < k_end)
                              ? load16(W + (long long)(n0 + row) * H1 + gk)
                              : make_uint4(0, 0, 0, 0);
        }
    };
    auto store_chunk = [&](int buf, const uint4(&src)[XP + WP]) {
        uint16_t* sx = s_stage + buf * SH::kStage;
        uint16_t* sw = sx + BM * kLinBK;
#pragma unroll
        for (int u = 0; u < XP; ++u) {
            const int id = tid + u * kLinThreads;
            const int row = id >> 3, p = id & 7;
            *reinterpret_cast<uint4*>(sx + row * kLinBK + ((p ^ (row & 7)) << 3)) = src[u];
        }
#pragma unroll
        for (int u = 0; u < WP; ++u) {
            const int id = tid + u * kLinThreads;
            const int row = id >> 3, p = id & 7;
            *reinterpret_cast<uint4*>(sw + row * kLinBK + ((p ^ (row & 7)) << 3)) = src[XP + u];
        }
    };

    const int wr0 = (wid / SH::WN) * TM * 16;  // first tile row of this wave
    const int wc0 = (wid % SH::WN) * TN * 16;  // first tile column of this wave
    const int lr = lane & 15, lg = lane >> 4;
    mf32x4 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = mf32x4{0.f, 0.f, 0.f, 0.f};

    auto compute = [&](int buf) {
        const uint16_t* sx = s_stage + buf * SH::kStage;
        const uint16_t* sw = sx + BM * kLinBK;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            const int p = 4 * ks + lg;  // 16-byte piece of the 32-k step
            uint4 a[TM], b[TN];
#pragma unroll
            for (int i = 0; i < TM; ++i) {
                const int row = wr0 + 16 * i + lr;
                a[i] = *reinterpret_cast<const uint4*>(sx + row * kLinBK + ((p ^ (row & 7)) << 3));
            }
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                const int row = wc0 + 16 * j + lr;
                b[j] = *reinterpret_cast<const uint4*>(sw + row * kLinBK + ((p ^ (row & 7)) << 3));
            }
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j) acc[i][j] = MfmaOps<DT>::mma(a[i], b[j], acc[i][j]);
        }
    };

    // Chunk c lives in ring[c % PD] from its load until its LDS store, which
    // frees the slot for chunk c + PD.  One barrier per chunk: a wave stores
    // chunk c into buffer c & 1 only after every wave has passed the barrier
    // of chunk c - 1, i.e. finished computing chunk c - 2 from that buffer.
#pragma unroll
    for (int d = 0; d < PD; ++d)
        if (d < nchunks) load_chunk(d, ring[d]);

    // The segment table, into LDS, then what the correction needs that does
    // not depend on the base product (its loads overlap the first chunks').
#pragma unroll
    for (int u = 0; u < kSegU; ++u) {
        const int e = tid + u * kLinThreads;
        if (seg_lds && e <= S) s_seg[e] = seg_r[u];
        if (seg_lds && e < S) s_ids[e] = ids_r[u];
    }
    lds_barrier();
    linear_prepare<false, !kFold>(s_aid, s_v, s_seg, s_ids, seg_lds, vpart, vstride, vsplit,
                                  seg_indptr, adapter_ids, S, M, num_adapters, r, ksplit, q, m0,
                                  BM);

    for (int c0 = 0; c0 < nchunks; c0 += PD) {
#pragma unroll
        for (int d = 0; d < PD; ++d) {
            const int c = c0 + d;
            if (c < nchunks) {
                store_chunk(c & 1, ring[d]);
                if (c + PD < nchunks) load_chunk(c + PD, ring[d]);
                lds_barrier();
                compute(c & 1);
            }
        }
    }
    __syncthreads();  // every wave is done with the staging buffers

    // Folded: the correction's first B rows requested now, then the wait
    // for every shrink workgroup and this workgroup's first pass of v (or,
    // past the patience, v recomputed); the B loads overlap both.
    uint4 bpre[BM * BN / 8 / kLinThreads][4];
    if constexpr (kFold)
        linear_prefetch_b<DT, BM, BN>(bpre, s_aid, B_stack, H2, r, ksplit, q, n0);
    if constexpr (kFold) {
        if (tid == 0) s_fold_ok = wait_for_producers(fold_cnt, n_shrink, wait_ticks);
        __syncthreads();
        if (s_fold_ok) {
            linear_prepare_v<true>(s_v, vpart, vstride, vsplit, M, r, ksplit, q, m0, BM);
        } else {
            if (tid == 0) __hip_atomic_store(flag, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            switch (r) {
                case 16:
                    linear_v_refold<DT, 16>(s_v, s_fv, s_aid, x, A_stack, s_raw, M, H1, m0, BM,
                                            ksplit, chunks_per_split, q);
                    break;
                case 32:
                    linear_v_refold<DT, 32>(s_v, s_fv, s_aid, x, A_stack, s_raw, M, H1, m0, BM,
                                            ksplit, chunks_per_split, q);
                    break;
                case 64:
                    linear_v_refold<DT, 64>(s_v, s_fv, s_aid, x, A_stack, s_raw, M, H1, m0, BM,
                                            ksplit, chunks_per_split, q);
                    break;
                default:
                    linear_v_refold<DT, 128>(s_v, s_fv, s_aid, x, A_stack, s_raw, M, H1, m0, BM,
                                             ksplit, chunks_per_split, q);
                    break;
            }
        }
        __syncthreads();  // every thread's v loads have returned
        if (tid == 0) depart(fold_cnt, 1 << 16, fold_total);
    }

    // ---- accumulators -> float tile in LDS -------------------------------
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                s_t[(wr0 + 16 * i + 4 * lg + e) * TP + wc0 + 16 * j + lr] = acc[i][j][e];

    linear_finish<DT, BM, BN, TP, kFold, kFold>(
        s_t, s_aid, s_v, s_seg, s_ids, &s_last, seg_lds, y, bias, B_stack, vpart, vstride, vsplit,
        seg_indptr, adapter_ids, S, M, num_adapters, H2, r, scale, part, counters, counter_stride,
        ksplit, q, t, m0, n0, bpre);
}

// ---- many rows: 256 x 256 tiles ----------------------------------------------
// For batches of many rows (prefill) the base product dominates and the tile
// size sets how often x and W are re-read from L2: with 256 x 256 tiles a
// 4096 x 4096 output is 256 tiles, one per compute unit, each reading its 256
// rows of x and of W once.  A workgroup is one of the WideShape forms below:
// eight waves of 128 rows x 64 columns, or four of 128 x 128.
//
// K moves through four 32 KB LDS arrays.  When H1 is a multiple of 128 they
// are four stages of 32 K filled by direct global-to-LDS loads three steps
// ahead (kDma); otherwise they are two buffers of 64 K (x rows in one array,
// W rows in the other), loaded through registers one chunk ahead.  In LDS a
// row keeps its 16-byte pieces XOR-swizzled by its row index, which spreads
// the rows an MFMA operand read touches over the banks.
//
// The product is computed transposed, Y^T = W X^T (W as the MFMA's A
// operand), so that each lane's accumulator holds four consecutive columns
// of one row: the epilogue adds the bias and stores 8-byte pieces of y
// straight from the registers.
//
// The correction s (x A_a) B_a runs on the same accumulators, also on the
// matrix cores, one segment of the tile at a time: for ranks in passes of
// 16, D += B'^T V'^T with the rows outside the segment masked to zero in V'.
// The 16-bit MFMA operands carry float32 precision through term splits in
// bf16 (whose exponent range is float32's, so no scaling is needed):
// s v = vh + vm + vl (three bf16 terms, 24 significant bits) and, for fp16
// weights, B = Bh + Bl exactly (11 significant bits in two bf16 terms).  The
// K dimension pairs them as [vh Bh | vm Bh | vl Bh | vh Bl | vm Bl | 0]
// (fp16; the dropped vl Bl is below float32 rounding of the product) or
// [vh B | vm B | vl B | 0] (bf16), in MFMA steps of 32.
constexpr int kWideBM = 256, kWideBN = 256;        // tile
constexpr int kWideTM = 8;                         // 16-row blocks per wave: 128 rows
constexpr int kWideBK = 64;                        // K per chunk
constexpr int kWideHalf = kWideBM * kWideBK;       // 16-bit elements of one operand's chunk
constexpr int kWideRG = 16;                        // ranks per correction pass
constexpr int kWideStages = 4;                     // direct-load stages of 32 K
constexpr int kWideLdB = kWideBN + 16;  // padded row of B' (transposing reads)
static_assert(kWideBM == kWideBN, "square tile");

// Workgroup shapes of the 256 x 256 tile: TN 16-column blocks per wave (two
// waves along the rows, 256 / (16 TN) along the columns) and PD chunks of
// loads in flight.  <4, 1>: eight waves of 128 x 64, two per SIMD (the one
// in use).  <8, 1> and <8, 2>: four waves of 128 x 128, one per SIMD with
// the accumulators in AGPRs; they read a third fewer LDS bytes per MFMA, but
// with one wave per SIMD nothing hides a wave's own waits, and at 4096 x
// 4096 x 4096 they took 205 and 218 us against 187 us for <4, 1>.
template <int TN_, int PD_>
struct WideShape {
    static constexpr int TN = TN_, PD = PD_;
    static constexpr int WN = kWideBN / (16 * TN);  // waves along the columns
    static constexpr int kNT = 2 * WN * kWave;      // threads
    static constexpr int kSegLds = kNT - 1;         // segment-table entries staged in LDS
    static_assert(2 * 16 * kWideTM == kWideBM, "two waves along the rows");
};

template <typename DT>
struct WideTerms;
template <>
struct WideTerms<F16> {
    static constexpr int kK = 96;  // five products of 16 ranks, padded to 3 MFMA steps
};
template <>
struct WideTerms<BF16> {
    static constexpr int kK = 64;  // three products of 16 ranks, padded to 2 steps
};

// LDS: buffer 0 is (s_wide0: x rows, s_wide1: W rows), buffer 1 is
// (s_wide2, s_wide3); the correction reuses all four.
__shared__ __attribute__((aligned(16))) uint16_t s_wide0[kWideHalf];
__shared__ __attribute__((aligned(16))) uint16_t s_wide1[kWideHalf];
__shared__ __attribute__((aligned(16))) uint16_t s_wide2[kWideHalf];
__shared__ __attribute__((aligned(16))) uint16_t s_wide3[kWideHalf];

// The four LDS arrays by index (compile time), for the direct-load stages.
template <int B>
__device__ __forceinline__ uint16_t* wide_stage() {
    if constexpr (B == 0) return s_wide0;
    else if constexpr (B == 1) return s_wide1;
    else if constexpr (B == 2) return s_wide2;
    else return s_wide3;
}

// bf16 terms of a float: hi, and the rounded remainder (0 for inf / NaN,
// whose remainder is not a number).
__device__ __forceinline__ uint32_t bf16_rest(float f, uint32_t hi) {
    return (hi & 0x7F80u) == 0x7F80u ? 0u : BF16::f2b(f - BF16::b2f(hi));
}

// Grid: exactly `tiles` workgroups.  Workgroup b runs on XCD b % 8; when the
// tile count is a multiple of 8, each XCD takes a contiguous range of tiles
// (whole rows of tiles at the usual shapes), so its L2 serves the x rows
// those tiles share.  H1 and H2 are multiples of 8; x, W, y and bias are
// 16-byte aligned.
template <typename DT, typename WS, bool kDma>
__global__ __launch_bounds__(WS::kNT) void linear_wide_kernel(
    typename DT::storage* __restrict__ y, const typename DT::storage* __restrict__ x,
    const typename DT::storage* __restrict__ W, const typename DT::storage* __restrict__ bias,
    const typename DT::storage* __restrict__ B_stack, const float* __restrict__ vpart,
    long long vstride, int vsplit, const int* __restrict__ seg_indptr,
    const int* __restrict__ adapter_ids, int S, int M, int num_adapters, int H1, int H2, int r,
    float scale, int tiles_n, int tiles) {
    using T = typename DT::storage;
    using Ops = MfmaOps<DT>;
    using BOps = MfmaOps<BF16>;
    constexpr int NT = WS::kNT, TN = WS::TN, WN = WS::WN, PD = WS::PD;
    constexpr int KQ = WideTerms<DT>::kK;
    constexpr int VQ = KQ + 8;  // padded row of V' (bank spread of the operand reads)
    constexpr bool kSplitB = std::is_same<DT, F16>::value;
    // Epilogue: V' rows [0, 128) in stage 0 and [128, 256) in stage 1, B'
    // rows [0, KQ / 2) in stage 2 and the rest in stage 3.
    static_assert(kWideBM / 2 * VQ <= kWideHalf && KQ / 2 * kWideLdB <= kWideHalf,
                  "V' and B' fit the buffers");
    static_assert((KQ / 2) % 8 == 0, "an operand's 8 rows of B' lie in one stage");
    __shared__ __attribute__((aligned(16))) float s_v[kWideBM * kWideRG];
    __shared__ int s_seg[WS::kSegLds + 1];
    __shared__ int s_ids[WS::kSegLds];

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wid = tid / kWave;
    const int lr = lane & 15, lg = lane >> 4;
    int t = (int)blockIdx.x;
    if ((tiles & 7) == 0) t = (t & 7) * (tiles >> 3) + (t >> 3);
    if (t >= tiles) return;  // whole workgroup (the grid is exact)
    const int m0 = (t / tiles_n) * kWideBM;
    const int n0 = (t % tiles_n) * kWideBN;
    const int nchunks = (H1 + kWideBK - 1) / kWideBK;
    const int wr0 = (wid / WN) * (16 * kWideTM);  // first tile row of this wave
    const int wc0 = (wid % WN) * (16 * TN);  // first tile column of this wave

    // The segment table when it fits LDS.
    const bool seg_lds = S <= WS::kSegLds;  // no table is read when S == 0
    if (seg_lds && S > 0) {
        if (tid <= S) s_seg[tid] = seg_indptr[tid];
        if (tid < S) s_ids[tid] = adapter_ids[tid];
    }
    __syncthreads();
    auto seg_at = [&](int s) { return seg_lds ? s_seg[s] : seg_indptr[s]; };
    auto id_at = [&](int s) { return seg_lds ? s_ids[s] : adapter_ids[s]; };
    const int row_end = min(m0 + kWideBM, M);
    // The next segment from s on that covers rows of this tile and has a
    // valid adapter (S if none).  Uniform over the workgroup.
    auto next_segment = [&](int s) {
        for (; s < S; ++s) {
            const int lo = seg_at(s);
            if (lo >= row_end) return S;
            const int hi = min(seg_at(s + 1), row_end);
            const int a = id_at(s);
            if (hi > max(lo, m0) && a >= 0 && a < num_adapters) return s;
        }
        return S;
    };
    // First segment ending after m0 (segment ends are non-decreasing).
    int first = 0;
    {
        int lo = 0, hi = S;
        while (lo < hi) {
            const int mid = (lo + hi) >> 1;
            if (seg_at(mid + 1) <= m0) lo = mid + 1;
            else hi = mid;
        }
        first = lo;
    }
    // The first pass of v (before the main loop, whose loads it overlaps).
    auto fill_v = [&](int g0) {
        for (int e = tid; e < kWideBM * kWideRG; e += NT) {
            const int il = e / kWideRG, k = e % kWideRG;
            float v = 0.f;
            if (m0 + il < M && g0 + k < r)
                v = sum_partials(vpart + (long long)(m0 + il) * r + g0 + k, vstride, vsplit);
            s_v[e] = v;
        }
    };
    if (next_segment(first) < S) fill_v(0);  // uniform; tiles without adapted rows skip it

    // ---- base product ------------------------------------------------------
    mf32x4 acc[kWideTM][TN];
#pragma unroll
    for (int i = 0; i < kWideTM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = mf32x4{0.f, 0.f, 0.f, 0.f};
    if constexpr (kDma) {
        // Steps of 32 K through four stages (s_wide0..3: 256 rows of x then
        // 256 rows of W, 64 bytes each), filled by direct global-to-LDS loads
        // three steps ahead: global_load_lds_dwordx4 writes lane i's 16 bytes
        // at the wave's LDS base + 16 i, so wave w fills stage rows
        // [kRowsW w, kRowsW (w + 1)) with loads of 16 rows, each lane fetching the
        // piece its slot holds (piece p of row r sits at slot
        // p ^ ((r >> 1) & 3)).  Rows past M or H2 read the last valid row
        // (their results are never stored).  Step c waits for its own loads
        // (the later two steps' stay in flight) and for its LDS reads of step
        // c - 1, then for every wave; after that barrier stage (c + 3) % 4,
        // read in step c - 1, takes step c + 3.  Every step issues loads (past
        // the last step they re-read it into a stage no step reads) and the
        // loop has no early exit, H1 being a multiple of 128.
        //
        // The compiler then adds no wait of its own for these loads before a
        // stage's LDS reads, because it can tell the stages apart: each is
        // an LDS array of its own; the count of later loads does not depend
        // on the path; and the first load it records into a stage spans the
        // whole stage in its offset range (wave w's first load sits at row
        // kRowsW w).  Short of any of these it waits for every outstanding
        // load (vmcnt(0)) before each step's first read.
        const int nsteps = H1 / 32;
        const int lrow = lane >> 2;
        using lds_t = __attribute__((address_space(3))) void;
        // kRowsW stage rows per wave in kLoadsW loads of 16 rows (64 rows and
        // 4 loads with eight waves).
        constexpr int kRowsW = 2 * kWideBM / (NT / kWave);
        constexpr int kLoadsW = kRowsW / 16;
        static_assert(kLoadsW * 16 * (NT / kWave) == 2 * kWideBM, "whole loads per wave");
        static_assert(2 * kLoadsW < 64, "the wait count fits vmcnt");
        constexpr int kWaitSteps = (2 * kLoadsW & 15) | ((2 * kLoadsW >> 4) << 14) | 0x0070;
        const T* gsrc[kLoadsW];
#pragma unroll
        for (int u = 0; u < kLoadsW; ++u) {
            const int row = kRowsW * wid + 16 * u + lrow;
            const int piece = (lane & 3) ^ ((row >> 1) & 3);
            gsrc[u] = row < kWideBM
                          ? x + (long long)min(m0 + row, M - 1) * H1 + piece * 8
                          : W + (long long)min(n0 + row - kWideBM, H2 - 1) * H1 + piece * 8;
        }
        auto issue = [&](uint16_t* st, int step) {
#pragma unroll
            for (int u = 0; u < kLoadsW; ++u)
                __builtin_amdgcn_global_load_lds((const void*)(gsrc[u] + step * 32),
                                                 (lds_t*)(st + (kRowsW * wid + 16 * u) * 32), 16,
                                                 0, 0);
        };
        auto compute = [&](const uint16_t* st) {
            auto rd = [&](int row) {
                return *reinterpret_cast<const uint4*>(st + row * 32 +
                                                       ((lg ^ ((row >> 1) & 3)) << 3));
            };
            uint4 b[TN];
#pragma unroll
            for (int j = 0; j < TN; ++j) b[j] = rd(kWideBM + wc0 + 16 * j + lr);
#pragma unroll
            for (int i = 0; i < kWideTM; ++i) {
                const uint4 a = rd(wr0 + 16 * i + lr);
#pragma unroll
                for (int j = 0; j < TN; ++j) acc[i][j] = Ops::mma(b[j], a, acc[i][j]);
            }
        };
        auto step = [&](auto stage_c, int c) {
            constexpr int B = decltype(stage_c)::value;
            __builtin_amdgcn_s_waitcnt(kWaitSteps);  // vmcnt(two steps' loads), lgkmcnt(0)
            asm volatile("" ::: "memory");       // no LDS access moves across the barrier
            __builtin_amdgcn_s_barrier();
            asm volatile("" ::: "memory");
            issue(wide_stage<(B + 3) & 3>(), min(c + 3, nsteps - 1));
            compute(wide_stage<B>());
        };
        static_assert(kWideStages == 4, "four stages");
        issue(wide_stage<0>(), 0);
        issue(wide_stage<1>(), min(1, nsteps - 1));
        issue(wide_stage<2>(), min(2, nsteps - 1));
        for (int c0 = 0; c0 < nsteps; c0 += 4) {
            step(std::integral_constant<int, 0>{}, c0);
            step(std::integral_constant<int, 1>{}, c0 + 1);
            step(std::integral_constant<int, 2>{}, c0 + 2);
            step(std::integral_constant<int, 3>{}, c0 + 3);
        }
        __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0), lgkmcnt(0): the stages are quiet
    } else {
        // A chunk of one operand is 256 rows x 8 pieces of 16 bytes: 4 pieces
        // per thread.
        constexpr int kP = kWideBM * (kWideBK / 8) / NT;
        static_assert(kP * NT == kWideBM * (kWideBK / 8), "whole pieces per thread");
        // ring[d]: a chunk's pieces for this thread, x rows then W rows.
        uint4 ring[PD][2 * kP];
        auto load_chunk = [&](int c, uint4(&dst)[2 * kP]) {
            const int k0 = c * kWideBK;
    #pragma unroll
            for (int u = 0; u < kP; ++u) {
                const int id = tid + u * NT;
                const int row = id >> 3, gk = k0 + (id & 7) * 8;
                dst[u] = (m0 + row < M && gk < H1) ? load16(x + (long long)(m0 + row) * H1 + gk)
                                                   : make_uint4(0, 0, 0, 0);
                dst[kP + u] = (n0 + row < H2 && gk < H1) ? load16(W + (long long)(n0 + row) * H1 + gk)
                                                         : make_uint4(0, 0, 0, 0);
            }
        };
        auto store_chunk = [&](uint16_t* sx, uint16_t* sw, const uint4(&src)[2 * kP]) {
    #pragma unroll
            for (int u = 0; u < kP; ++u) {
                const int id = tid + u * NT;
                const int row = id >> 3, p = id & 7;  // row < kWideBM: off < kWideHalf
                const int off = row * kWideBK + ((p ^ (row & 7)) << 3);
                *reinterpret_cast<uint4*>(sx + off) = src[u];
                *reinterpret_cast<uint4*>(sw + off) = src[kP + u];
            }
        };


        // One chunk: two K steps of 32, each the wave's 4 W blocks against its 8
        // x blocks.
        auto compute = [&](const uint16_t* sx, const uint16_t* sw) {
            auto rd = [&](const uint16_t* base, int row, int ks) {
                const int p = 4 * ks + lg;  // 16-byte piece of the 32-k step
                return *reinterpret_cast<const uint4*>(base + row * kWideBK + ((p ^ (row & 7)) << 3));
            };
            uint4 b0[TN], b1[TN];
    #pragma unroll
            for (int j = 0; j < TN; ++j) b0[j] = rd(sw, wc0 + 16 * j + lr, 0);
            uint4 a = rd(sx, wr0 + lr, 0);
    #pragma unroll
            for (int i = 0; i < kWideTM; ++i) {
                const uint4 an = rd(sx, wr0 + 16 * ((i + 1) % kWideTM) + lr, i + 1 < kWideTM ? 0 : 1);
                if (i == kWideTM / 2) {
    #pragma unroll
                    for (int j = 0; j < TN; ++j) b1[j] = rd(sw, wc0 + 16 * j + lr, 1);
                }
    #pragma unroll
                for (int j = 0; j < TN; ++j) acc[i][j] = Ops::mma(b0[j], a, acc[i][j]);
                a = an;
            }
    #pragma unroll
            for (int i = 0; i < kWideTM; ++i) {
                uint4 an = a;
                if (i + 1 < kWideTM) an = rd(sx, wr0 + 16 * (i + 1) + lr, 1);
    #pragma unroll
                for (int j = 0; j < TN; ++j) acc[i][j] = Ops::mma(b1[j], a, acc[i][j]);
                a = an;
            }
        };
        // Chunk c (parity P): its registers (ring slot c % PD) into buffer P
        // (every wave is past the barrier of chunk c - 1, so done with chunk
        // c - 2 there), chunk c + PD's loads issued into the freed slot, then the
        // barrier and the MFMAs.
        static_assert(PD == 1 || PD == 2, "ring slot c % PD has the parity's index");
        auto chunk = [&](auto parity, int c, uint16_t* sx, uint16_t* sw) {
            constexpr int P = decltype(parity)::value;
            store_chunk(sx, sw, ring[P % PD]);
            if (c + PD < nchunks) load_chunk(c + PD, ring[P % PD]);
            lds_barrier();
            compute(sx, sw);
        };
        load_chunk(0, ring[0]);
        if constexpr (PD == 2)
            if (1 < nchunks) load_chunk(1, ring[1 % PD]);
        for (int c = 0; c < nchunks; c += 2) {
            chunk(std::integral_constant<int, 0>{}, c, s_wide0, s_wide1);
            if (c + 1 < nchunks) chunk(std::integral_constant<int, 1>{}, c + 1, s_wide2, s_wide3);
        }
    }

    // ---- correction ---------------------------------------------------------
    auto vq_row = [&](int il) {  // row il of V'
        return il < kWideBM / 2 ? s_wide0 + il * VQ : s_wide1 + (il - kWideBM / 2) * VQ;
    };
    auto bq_row = [&](int k) {  // row k of B'
        return k < KQ / 2 ? s_wide2 + k * kWideLdB : s_wide3 + (k - KQ / 2) * kWideLdB;
    };
    // This thread's pieces of a B' pass (16 ranks x 32 pieces of 8 columns):
    // piece q is rank (tid + q NT) / 32, columns ((tid + q NT) % 32) * 8.
    constexpr int kBP = kWideRG * 32 / NT;
    static_assert(kBP * NT == kWideRG * 32, "whole pieces per thread");
    uint4 braw[kBP];
    auto load_b = [&](int s, int g0) {
        const int a = id_at(s);
#pragma unroll
        for (int q = 0; q < kBP; ++q) {
            const int id = tid + q * NT;
            const int bk = id >> 5, bc = n0 + (id & 31) * 8;
            braw[q] = (g0 + bk < r && bc < H2)
                          ? load16(B_stack + ((long long)a * r + g0 + bk) * H2 + bc)
                          : make_uint4(0, 0, 0, 0);
        }
    };
    int seg_cur = next_segment(first);
    if (seg_cur < S) load_b(seg_cur, 0);
    for (int g0 = 0; g0 < r && seg_cur < S; g0 += kWideRG) {
        // The stages (and, from the second pass, s_v) are free: every wave is
        // past its last step and, by the barrier's fence (vmcnt(0)), its
        // loads into the stages have landed.
        __syncthreads();
        if (g0 > 0) {
            fill_v(g0);
            __syncthreads();
        }
        // V' rows: the terms of s v in the slot order of B'.
        for (int e = tid; e < kWideBM * kWideRG; e += NT) {
            const int il = e / kWideRG, k = e % kWideRG;
            const float v = scale * s_v[e];
            const uint32_t vh = BF16::f2b(v);
            const uint32_t vm = bf16_rest(v, vh);
            const float r1 = (vh & 0x7F80u) == 0x7F80u ? 0.f : v - BF16::b2f(vh);
            const uint32_t vl = bf16_rest(r1, vm);
            uint16_t* q = vq_row(il);
            q[k] = (uint16_t)vh;
            q[kWideRG + k] = (uint16_t)vm;
            q[2 * kWideRG + k] = (uint16_t)vl;
            if constexpr (kSplitB) {
                q[3 * kWideRG + k] = (uint16_t)vh;
                q[4 * kWideRG + k] = (uint16_t)vm;
                q[5 * kWideRG + k] = 0;
            } else {
                q[3 * kWideRG + k] = 0;
            }
        }
        if (g0 > 0) load_b(seg_cur, g0);
        while (seg_cur < S) {
            __syncthreads();  // V' written; the previous segment's reads of B' done
#pragma unroll
            for (int q = 0; q < kBP; ++q) {
                const int id = tid + q * NT;
                const int bk = id >> 5, c8 = (id & 31) * 8;
                float f[8];
                DT::unpack(braw[q], f);
                uint4 hi, lo;
                if constexpr (kSplitB) {
                    uint32_t h[8], l[8];
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        h[e] = BF16::f2b(f[e]);
                        l[e] = bf16_rest(f[e], h[e]);
                    }
                    hi = make_uint4(h[0] | h[1] << 16, h[2] | h[3] << 16, h[4] | h[5] << 16,
                                    h[6] | h[7] << 16);
                    lo = make_uint4(l[0] | l[1] << 16, l[2] | l[3] << 16, l[4] | l[5] << 16,
                                    l[6] | l[7] << 16);
                } else {
                    hi = braw[q];
                    lo = make_uint4(0, 0, 0, 0);
                }
                store16(bq_row(bk) + c8, hi);
                store16(bq_row(kWideRG + bk) + c8, hi);
                store16(bq_row(2 * kWideRG + bk) + c8, hi);
                if constexpr (kSplitB) {
                    store16(bq_row(3 * kWideRG + bk) + c8, lo);
                    store16(bq_row(4 * kWideRG + bk) + c8, lo);
                    store16(bq_row(5 * kWideRG + bk) + c8, make_uint4(0, 0, 0, 0));
                } else {
                    store16(bq_row(3 * kWideRG + bk) + c8, make_uint4(0, 0, 0, 0));
                }
            }
            __syncthreads();
            const int lo_row = max(seg_at(seg_cur), m0);
            const int hi_row = min(seg_at(seg_cur + 1), row_end);
            const int seg_next = next_segment(seg_cur + 1);
            if (seg_next < S) load_b(seg_next, g0);  // in flight during the MFMAs
#pragma unroll
            for (int ks = 0; ks < KQ / 32; ++ks) {
                // this lane group's 8 rows of B' (one stage holds all of them)
                const int k0 = ks * 32 + lg * 8;
                const uint16_t* bbase = k0 < KQ / 2 ? s_wide2 : s_wide3;
                const int kl = k0 < KQ / 2 ? k0 : k0 - KQ / 2;
                uint4 bb[TN];
#pragma unroll
                for (int j = 0; j < TN; ++j)
                    bb[j] = lds_operand_tr(bbase + wc0 + 16 * j, kl, kWideLdB, lr);
#pragma unroll
                for (int i = 0; i < kWideTM; ++i) {
                    const int rb = m0 + wr0 + 16 * i;
                    if (rb + 16 <= lo_row || rb >= hi_row) continue;  // uniform over the wave
                    const int row = rb + lr;
                    const uint4 vv = (row >= lo_row && row < hi_row)
                                         ? *reinterpret_cast<const uint4*>(
                                               vq_row(wr0 + 16 * i + lr) + ks * 32 + lg * 8)
                                         : make_uint4(0, 0, 0, 0);
#pragma unroll
                    for (int j = 0; j < TN; ++j) acc[i][j] = BOps::mma(bb[j], vv, acc[i][j]);
                }
            }
            seg_cur = seg_next;
        }
        seg_cur = next_segment(first);
        if (g0 + kWideRG >= r) break;
    }

    // ---- bias, one rounding, store ------------------------------------------
#pragma unroll
    for (int j = 0; j < TN; ++j) {
        const int col = n0 + wc0 + 16 * j + 4 * lg;
        if (col >= H2) continue;
        float bv[4] = {0.f, 0.f, 0.f, 0.f};
        if (bias) {
            const uint2 braw2 = load8(bias + col);
            DT::unpack2(braw2.x, bv);
            DT::unpack2(braw2.y, bv + 2);
        }
#pragma unroll
        for (int i = 0; i < kWideTM; ++i) {
            const int row = m0 + wr0 + 16 * i + lr;
            if (row >= M) continue;
            const uint2 o = make_uint2(DT::pack2(acc[i][j][0] + bv[0], acc[i][j][1] + bv[1]),
                                       DT::pack2(acc[i][j][2] + bv[2], acc[i][j][3] + bv[3]));
            store8(y + (long long)row * H2 + col, o);
        }
    }
}

// Any shape and dtype: one thread per output element, the base product as
// a sequential sum over H1, then the bias and the correction.  Slow; it
// serves float32 and shapes the tiled kernel does not take.
template <typename DT>
__global__ __launch_bounds__(256) void linear_lora_generic_kernel(
    typename DT::storage* __restrict__ y, const typename DT::storage* __restrict__ x,
    const typename DT::storage* __restrict__ W, const typename DT::storage* __restrict__ bias,
    const typename DT::storage* __restrict__ B_stack, const float* __restrict__ vpart,
    long long vstride, int vsplit, const int* __restrict__ seg_indptr,
    const int* __restrict__ adapter_ids, int S, int M, int num_adapters, int H1, int H2, int r,
    float scale) {
    const long long e = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    if (e >= (long long)M * H2) return;
    const int row = (int)(e / H2), col = (int)(e - (long long)row * H2);
    const typename DT::storage* xr = x + (long long)row * H1;
    const typename DT::storage* wr = W + (long long)col * H1;
    float acc = 0.f;
    for (int h = 0; h < H1; ++h) acc = fmaf(DT::load1(xr + h), DT::load1(wr + h), acc);
    const int a = row_adapter(seg_indptr, adapter_ids, S, row, num_adapters);
    if (a >= 0) {
        float ls = 0.f;
        for (int k = 0; k < r; ++k) {
            float vk = 0.f;
            for (int c = 0; c < vsplit; ++c) vk += vpart[(long long)c * vstride + (long long)row * r + k];
            ls = fmaf(vk, DT::load1(B_stack + ((long long)a * r + k) * H2 + col), ls);
        }
        acc = fmaf(scale, ls, acc);
    }
    if (bias) acc += DT::load1(bias + col);
    y[e] = DT::from_float(acc);
}

}  // namespace sgmv
