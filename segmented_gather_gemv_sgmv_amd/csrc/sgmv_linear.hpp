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
