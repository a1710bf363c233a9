// sgmv_mixed.hpp -- the work decomposition that chooses the kernel form per
// segment, inside one launch.
//
// The pages split a batch into segments, one per model, and run the shrink
// and the expand over all of them in one kernel (Punica walkthrough,
// omica.com.cn/news/959180, section 2.2; segmented inputs and outputs:
// Punica review, nubint.ai, "Proposed method").  A serving batch mixes
// decode requests, one row each, with prefill requests of many rows.  The
// two shapes want different code: a one-row segment is a matrix-vector
// product bound by reading its adapter (vector units, wide loads), a segment
// of many rows is a dense contraction (matrix cores, 16-row tiles).  So every
// segment is classified on the device, from the table itself, into one of
// three classes:
//
//   long   (n >= TH rows)       tiles of 16 rows on the matrix cores (MFMA)
//   short  (2 <= n < TH rows)   tiles of 4 rows on the vector units
//   single (n == 1)             one-row tiles on the vector units (GEMV)
//
// TH is 2 wherever the matrix cores apply (fp16 and bf16 at ranks 16 to
// 128): a 16-row MFMA tile pays for itself from two rows, since it reads its
// adapter once however few rows it holds and its expand items are at least
// 256 columns wide (there is no short class).  TH is infinite where they do
// not apply (float32, rank 8: no long class; the short class serves 2..n).
// All classes run in the same launch.  Every workgroup scans the segment
// table once (up to kMixedMaxSegments entries, all loads in flight
// together), which gives it the number of tiles of each class and the place
// of every segment's tiles in its class; its index then names an item in
//
//   [long shrink][short shrink][single shrink][long expand][short expand][single expand]
//
// (each block: tiles of the class x its H1 chunks, or x its column chunks).
// Every expand item lies after every shrink item, so the hand-off of
// sgmv_fused.hpp applies unchanged: shrink items publish float32 partial
// sums and count themselves on their tile's counter, expand items wait for
// them.  Each class's chunk sizes are chosen by the host so that a shrink
// item of any class moves about the same number of bytes (its piece of A
// plus, for tall tiles, of x): the work is balanced by bytes, not by segment.
// The host does not know the classes, so it sizes the grid by the largest
// item count any table of its length could need; the workgroups past the
// real count find no item and return.
//
// The same decomposition in two launches (shrink_mixed_kernel, then
// expand_mixed_kernel) serves calls too large for one resident round and
// the separate sgmv_shrink / sgmv_expand entry points.
#pragma once

#include "sgmv_device.hpp"
#include "sgmv_fused.hpp"
#include "sgmv_gemv.hpp"
#include "sgmv_mfma.hpp"

#include <type_traits>

namespace sgmv {

constexpr int kMixedThreads = 256;
constexpr int kMixedPasses = 4;
constexpr int kMixedMaxSegments = kMixedThreads * kMixedPasses;

// ---------------------------------------------------------------------------
// In-kernel reduction of a split shrink (sgmv_shrink): after its partial
// stores, a workgroup counts itself on its tile's counter; the last of the
// tile's ksplit workgroups (told so by the count, so nobody waits) sums the
// partials in chunk order into v_final and returns the counter to zero.
// Partials were stored write-through at agent scope and are read the same
// way, each wave's stores acknowledged before the count.
// ---------------------------------------------------------------------------
template <int R>
__device__ __forceinline__ void reduce_if_last(const Tile& t, int ksplit, float* partials,
                                               long long row_stride, float* v_final, int* cnt,
                                               int* s_last) {
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (threadIdx.x == 0) {
        const int before = __hip_atomic_fetch_add(cnt, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const bool last = before == ksplit - 1;
        if (last) __hip_atomic_store(cnt, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        *s_last = last;
    }
    __syncthreads();
    if (!*s_last) return;
    for (int e = threadIdx.x; e < t.nrows * R; e += kMixedThreads) {
        const int i = e / R;
        const int k = e - i * R;
        v_final[(long long)(t.row0 + i) * R + k] = sum_partials_coherent(
            partials + (long long)(t.row0 + i) * R + k, row_stride, ksplit);
    }
}

// ---------------------------------------------------------------------------
// Vector tiles of RB rows (VALU): the GEMV form of decode segments.  Shrink
// items stream their chunk of A as 16-byte loads (shrink_chunk); expand
// items stream kCW columns of B and y, one 16-byte piece per thread and row,
// KB rows of B in flight per thread.
// ---------------------------------------------------------------------------
// Rank groups of a one-row expand item: from rank 32 an item's threads split
// its ranks into R / 16 groups, each streaming its ranks of B for fewer
// columns, so that an item moves about 64 KB of B whatever the rank (one
// CU streams a few hundred KB far slower than the chip's rate).
constexpr int vec_rank_groups(int R, int RB) { return RB == 1 && R >= 32 ? R / 16 : 1; }

template <typename DT, int R, int RB, int KB = (R < 16 ? R : 16), int KG = vec_rank_groups(R, RB)>
struct VecTile {
    using st = typename DT::storage;
    static constexpr int NT = kMixedThreads;
    static constexpr int kVec = DT::kVec;
    static constexpr int kT = RB;
    static constexpr int LPR = R / kVec;
    static constexpr int NW = NT / kWave;
    static constexpr int N = RB * kVec;
    static constexpr int kPG = 4;
    static constexpr int kGT = NT / KG;              // threads of a rank group
    static constexpr int kRG = R / KG;               // ranks of a group
    static constexpr int kKB = KB < kRG ? KB : kRG;  // rows of B in flight per thread
    static constexpr int kCW = kGT * kVec;           // expand columns per item
    static constexpr int kHUnit = NT / LPR;  // rows of A per block-wide pass
    static constexpr int kHMax = 0;          // a chunk may be any length
    static constexpr int kRedFloats = NW * LPR * N;
    // LDS: s_red [kRedFloats] | s_v [RB * R] | flag | the groups' sums [KG - 1][kCW]
    static constexpr int kLdsBytes = (kRedFloats + RB * R) * 4 + 16 + (KG - 1) * kCW * 4;
    static_assert(R % kVec == 0 && kWave % LPR == 0, "vector rank");
    static_assert(KG == 1 || RB == 1, "rank groups for one-row tiles");
    static_assert(R % KG == 0 && NT % KG == 0 && kRG % kKB == 0, "even rank groups");

    // This thread's rank group and its first column in column chunk c.
    __device__ static __forceinline__ int group() { return (int)threadIdx.x / kGT; }
    __device__ static __forceinline__ int col(int c) {
        return c * kCW + ((int)threadIdx.x % kGT) * kVec;
    }
    // This thread's pieces of B: its group's ranks, from column j.
    __device__ static __forceinline__ const st* b_ptr(const st* __restrict__ B_stack, int adapter,
                                                      int H2, int j) {
        return B_stack + (long long)adapter * R * H2 + (long long)group() * kRG * H2 + j;
    }

    __device__ static __forceinline__ float* s_v(unsigned char* lds) {
        return reinterpret_cast<float*>(lds) + kRedFloats;
    }

    template <typename Emit>
    __device__ static __forceinline__ void shrink_range(const Tile& t, const st* __restrict__ x,
                                                        const st* __restrict__ A_stack, int H1,
                                                        int h_lo, int h_hi, unsigned char* lds,
                                                        Emit&& emit) {
        shrink_chunk<DT, R, NT, RB, kPG>(A_stack + (long long)t.adapter * H1 * R,
                                         x + (long long)t.row0 * H1, t.nrows, H1, h_lo, h_hi,
                                         reinterpret_cast<float*>(lds), emit);
        __syncthreads();
    }

    // One-launch shrink item: publish the chunk's partials, then count.
    __device__ static __forceinline__ void shrink_item(const Tile& t, int p, int hps,
                                                       const st* __restrict__ x,
                                                       const st* __restrict__ A_stack, int H1,
                                                       float* partials, long long row_stride,
                                                       int* cnt, int total, unsigned char* lds) {
        const int h_lo = p * hps;
        const int h_hi = min(H1, h_lo + hps);
        float* out = partials + (long long)p * row_stride + (long long)t.row0 * R;
        shrink_chunk<DT, R, NT, RB, kPG>(A_stack + (long long)t.adapter * H1 * R,
                                         x + (long long)t.row0 * H1, t.nrows, H1, h_lo, h_hi,
                                         reinterpret_cast<float*>(lds),
                                         [&](int i, int k, float v) {
                                             store_partial(&out[i * R + k], v);
                                         });
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        __builtin_amdgcn_s_waitcnt(0);  // this wave's partial stores are acknowledged
        __syncthreads();
        if (threadIdx.x == 0) depart(cnt, 1, total);
    }

    // s_v (RB x R floats, complete and visible) -> y[rows, c0 : c0 + kCW] +=
    // scale * v B, with the first kKB rows of B and the y pieces already in
    // registers.
    __device__ static __forceinline__ void expand_finish(uint4 (&bv)[kKB], uint4 (&yv)[RB],
                                                         const st* __restrict__ Bj,
                                                         st* __restrict__ y, const Tile& t,
                                                         int j, bool active, int H2, float scale,
                                                         const float* s_v) {
        float acc[RB][kVec];
#pragma unroll
        for (int i = 0; i < RB; ++i)
#pragma unroll
            for (int q = 0; q < kVec; ++q) acc[i][q] = 0.f;
        const int g = group();
        const float* sv = s_v + g * kRG;  // this group's ranks
#pragma unroll
        for (int kb = 0; kb < kRG; kb += kKB) {
            if (kb > 0) {
#pragma unroll
                for (int kk = 0; kk < kKB; ++kk)
                    bv[kk] = active ? load16(Bj + (long long)(kb + kk) * H2) : make_uint4(0, 0, 0, 0);
            }
#pragma unroll
            for (int kk = 0; kk < kKB; ++kk) {
                float bf[kVec];
                DT::unpack(bv[kk], bf);
#pragma unroll
                for (int i = 0; i < RB; ++i) {
                    if (i < t.nrows) {
                        const float vv = sv[i * R + kb + kk];
#pragma unroll
                        for (int q = 0; q < kVec; ++q) acc[i][q] = fmaf(vv, bf[q], acc[i][q]);
                    }
                }
            }
        }
        if constexpr (KG > 1) {
            // groups 1.. leave their sums; group 0 adds them in group order
            float* s_part = const_cast<float*>(s_v) + RB * R + 4;
            const int jp = (int)threadIdx.x % kGT;
            if (g > 0) {
#pragma unroll
                for (int q = 0; q < kVec; ++q) s_part[(g - 1) * kCW + jp * kVec + q] = acc[0][q];
            }
            __syncthreads();
            if (g > 0) return;
#pragma unroll
            for (int gg = 1; gg < KG; ++gg)
#pragma unroll
                for (int q = 0; q < kVec; ++q) acc[0][q] += s_part[(gg - 1) * kCW + jp * kVec + q];
        }
        if (!active) return;
#pragma unroll
        for (int i = 0; i < RB; ++i) {
            if (i < t.nrows) {
                float yf[kVec];
                DT::unpack(yv[i], yf);
#pragma unroll
                for (int q = 0; q < kVec; ++q) yf[q] = fmaf(scale, acc[i][q], yf[q]);
                store16_stream(y + (long long)(t.row0 + i) * H2 + j, DT::pack(yf));
            }
        }
    }

    __device__ static __forceinline__ void expand_loads(uint4 (&bv)[kKB], uint4 (&yv)[RB],
                                                        const st* __restrict__ Bj,
                                                        const st* __restrict__ y, const Tile& t,
                                                        int j, bool active, int H2) {
#pragma unroll
        for (int kk = 0; kk < kKB; ++kk)
            bv[kk] = active ? load16(Bj + (long long)kk * H2) : make_uint4(0, 0, 0, 0);
        const bool first = group() == 0;  // only group 0 updates y
#pragma unroll
        for (int i = 0; i < RB; ++i)
            yv[i] = (active && first && i < t.nrows)
                        ? load16_stream(y + (long long)(t.row0 + i) * H2 + j)
                        : make_uint4(0, 0, 0, 0);
    }

    // One-launch expand item: loads that do not need v go out first, then
    // the wait for the tile's shrink items (or, past the patience, the
    // tile's partials recomputed here in the same order), then the update.
    __device__ static __forceinline__ void expand_item(
        const Tile& t, int c, st* __restrict__ y, const st* __restrict__ x,
        const st* __restrict__ A_stack, const st* __restrict__ B_stack, int H1, int H2,
        float scale, float* partials, long long row_stride, int ksplit, int hps, int* cnt,
        int total, int* flag, long long wait_ticks, unsigned char* lds) {
        float* s_v = reinterpret_cast<float*>(lds) + kRedFloats;
        int* s_flag = reinterpret_cast<int*>(s_v + RB * R);
        const int tid = threadIdx.x;
        const int j = col(c);
        const bool active = j < H2;
        const st* Bj = b_ptr(B_stack, t.adapter, H2, j);
        uint4 bv[kKB];
        uint4 yv[RB];
        if (ksplit == 0) {  // no shrink items (small adapters): v computed here
            shrink_range(t, x, A_stack, H1, 0, H1, lds,
                         [&](int i, int k, float v) { s_v[i * R + k] = v; });
            expand_loads(bv, yv, Bj, y, t, j, active, H2);
            expand_finish(bv, yv, Bj, y, t, j, active, H2, scale, s_v);
            return;
        }
        expand_loads(bv, yv, Bj, y, t, j, active, H2);
        if (tid == 0) *s_flag = wait_for_producers(cnt, ksplit, wait_ticks);
        __syncthreads();
        if (*s_flag) {
            for (int e = tid; e < RB * R; e += NT) {
                const int i = e / R;
                const int k = e - i * R;
                s_v[e] = i < t.nrows ? sum_partials_coherent(
                                           partials + (long long)(t.row0 + i) * R + k,
                                           row_stride, ksplit)
                                     : 0.f;
            }
        } else {
            if (tid == 0) __hip_atomic_store(flag, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            for (int e = tid; e < RB * R; e += NT) s_v[e] = 0.f;
            __syncthreads();
            for (int pp = 0; pp < ksplit; ++pp) {
                const int h_lo = pp * hps;
                const int h_hi = min(H1, h_lo + hps);
                shrink_range(t, x, A_stack, H1, h_lo, h_hi, lds,
                             [&](int i, int k, float v) { s_v[i * R + k] += v; });
            }
            expand_loads(bv, yv, Bj, y, t, j, active, H2);
        }
        __syncthreads();
        int before = 0;
        if (tid == 0) before = depart_begin(cnt, 1 << 16);
        expand_finish(bv, yv, Bj, y, t, j, active, H2, scale, s_v);
        if (tid == 0) depart_end(cnt, before, 1 << 16, total);
    }

    // Two-launch shrink item: plain partial stores; with v_final, the
    // tile's last item also reduces them into v (sgmv_shrink).
    __device__ static __forceinline__ void shrink_split(const Tile& t, int p, int hps, int ksplit,
                                                        const st* __restrict__ x,
                                                        const st* __restrict__ A_stack, int H1,
                                                        float* partials, long long row_stride,
                                                        float* v_final, int* cnt, int* s_last,
                                                        unsigned char* lds) {
        const int h_lo = p * hps;
        const int h_hi = min(H1, h_lo + hps);
        float* out = partials + (long long)p * row_stride + (long long)t.row0 * R;
        shrink_range(t, x, A_stack, H1, h_lo, h_hi, lds, [&](int i, int k, float v) {
            if (v_final) store_partial(&out[i * R + k], v);
            else out[i * R + k] = v;
        });
        if (v_final) reduce_if_last<R>(t, ksplit, partials, row_stride, v_final, cnt, s_last);
    }

    // Two-launch expand item: the P partials of each row summed in order.
    __device__ static __forceinline__ void expand_split(const Tile& t, int c, st* __restrict__ y,
                                                        const st* __restrict__ B_stack, int H2,
                                                        float scale,
                                                        const float* __restrict__ partials,
                                                        long long row_stride, int P,
                                                        unsigned char* lds) {
        float* s_v = reinterpret_cast<float*>(lds) + kRedFloats;
        const int tid = threadIdx.x;
        const int j = col(c);
        const bool active = j < H2;
        const st* Bj = b_ptr(B_stack, t.adapter, H2, j);
        uint4 bv[kKB];
        uint4 yv[RB];
        expand_loads(bv, yv, Bj, y, t, j, active, H2);
        for (int e = tid; e < RB * R; e += NT) {
            const int i = e / R;
            const int k = e - i * R;
            s_v[e] = i < t.nrows
                         ? sum_partials(partials + (long long)(t.row0 + i) * R + k, row_stride, P)
                         : 0.f;
        }
        __syncthreads();
        expand_finish(bv, yv, Bj, y, t, j, active, H2, scale, s_v);
    }
};

// ---------------------------------------------------------------------------
// 16-row MFMA tiles (fp16/bf16, R in 16..128): the dense-contraction form of
// long segments (sgmv_mfma.hpp holds the operand layouts and the chunk and
// expand routines).  LDS: region 0 holds the A chunk, then the cross-wave
// sums over it, in shrink items, and the B chunk then the y tile in expand
// items; region 1 holds v, its 16-bit halves and the range maximum.
// ---------------------------------------------------------------------------
// LDS chunks of A hold 16 KB (at least 128 rows): the kernel then keeps
// four or more workgroups per compute unit within 128 registers a lane.
template <int R>
constexpr int mixed_mfma_chunk() { return 8192 / R > 128 ? 8192 / R : 128; }

template <typename DT, int R>
struct MfmaTile {
    using st = typename DT::storage;
    static constexpr int KC = mixed_mfma_chunk<R>();
    using Sh = MfmaShape<R, KC>;
    static constexpr int NT = kMixedThreads;
    static constexpr int kT = Sh::kT;
    static constexpr int kCW = Sh::kCW;
    static constexpr int kHUnit = 128;           // whole K steps of the four waves
    static constexpr int kHMax = Sh::kKcMax;     // one LDS chunk of A
    static constexpr int kRegion0 =
        (Sh::kKcMax * R > Sh::kStageB ? Sh::kKcMax * R : Sh::kStageB) * 2;
    static_assert(Sh::kNW * 16 * R * 4 <= kRegion0, "the sums must fit over the A chunk");
    static constexpr int kOffV = kRegion0;                       // float [16 R]
    static constexpr int kOffVh = kOffV + kT * R * 4;            // uint16 [16 kVK]
    static constexpr int kOffMax = kOffVh + kT * Sh::kVK * 2;    // float [NW]
    static constexpr int kOffFlag = kOffMax + 16;                // int
    static constexpr int kLdsBytes = kOffFlag + 16;

    __device__ static __forceinline__ uint16_t* s_a(unsigned char* lds) {
        return reinterpret_cast<uint16_t*>(lds);
    }
    __device__ static __forceinline__ float* s_red(unsigned char* lds) {
        return reinterpret_cast<float*>(lds);
    }
    __device__ static __forceinline__ float* s_v(unsigned char* lds) {
        return reinterpret_cast<float*>(lds + kOffV);
    }
    __device__ static __forceinline__ uint16_t* s_vh(unsigned char* lds) {
        return reinterpret_cast<uint16_t*>(lds + kOffVh);
    }
    __device__ static __forceinline__ float* s_max(unsigned char* lds) {
        return reinterpret_cast<float*>(lds + kOffMax);
    }

    // The shrink of [h_lo, h_hi) for the tile, any length (ranges longer
    // than one LDS chunk of A stream through shrink_long_mfma).
    template <typename Emit>
    __device__ static __forceinline__ void shrink_range(const Tile& t, const st* __restrict__ x,
                                                        const st* __restrict__ A_stack, int H1,
                                                        int h_lo, int h_hi, unsigned char* lds,
                                                        Emit&& emit) {
        const st* A = A_stack + (long long)t.adapter * H1 * R;
        const st* xr = x + (long long)t.row0 * H1;
        if (h_hi - h_lo <= Sh::kKcMax)
            shrink_chunk_mfma<DT, R, true, KC>(A, xr, t.nrows, H1, h_lo, h_hi, s_a(lds),
                                               s_red(lds), emit);
        else
            shrink_long_mfma<DT, R, (KC >= 256 ? KC / 2 : KC)>(A, xr, t.nrows, H1, h_lo, h_hi,
                                                               s_a(lds), s_red(lds), emit);
    }

    // One-launch ranges are single LDS chunks (the plan keeps them so).
    template <typename Emit>
    __device__ static __forceinline__ void shrink_chunk(const Tile& t, const st* __restrict__ x,
                                                        const st* __restrict__ A_stack, int H1,
                                                        int h_lo, int h_hi, unsigned char* lds,
                                                        Emit&& emit) {
        shrink_chunk_mfma<DT, R, true, KC>(A_stack + (long long)t.adapter * H1 * R,
                                           x + (long long)t.row0 * H1, t.nrows, H1, h_lo, h_hi,
                                           s_a(lds), s_red(lds), emit);
    }

    __device__ static __forceinline__ void shrink_item(const Tile& t, int p, int hps,
                                                       const st* __restrict__ x,
                                                       const st* __restrict__ A_stack, int H1,
                                                       float* partials, long long row_stride,
                                                       int* cnt, int total, unsigned char* lds) {
        const int h_lo = p * hps;
        const int h_hi = min(H1, h_lo + hps);
        float* out = partials + (long long)p * row_stride + (long long)t.row0 * R;
        shrink_chunk(t, x, A_stack, H1, h_lo, h_hi, lds,
                     [&](int i, int k, float v) { store_partial(&out[i * R + k], v); });
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (threadIdx.x == 0) depart(cnt, 1, total);
    }

    __device__ static __forceinline__ void expand_item(
        const Tile& t, int c, st* __restrict__ y, const st* __restrict__ x,
        const st* __restrict__ A_stack, const st* __restrict__ B_stack, int H1, int H2,
        float scale, float* partials, long long row_stride, int ksplit, int hps, int* cnt,
        int total, int* flag, long long wait_ticks, unsigned char* lds) {
        const int tid = threadIdx.x;
        const int c0 = c * kCW;
        float* sv = s_v(lds);
        int* s_flag = reinterpret_cast<int*>(lds + kOffFlag);
        const st* B = B_stack + (long long)t.adapter * R * H2;
        st* yr = y + (long long)t.row0 * H2;
        ExpandRegs<R> er;
        if (ksplit == 0) {  // no shrink items (small adapters): v computed here
            for (int e = tid; e < kT * R; e += NT) sv[e] = 0.f;  // rows past the tile stay 0
            __syncthreads();
            for (int h_lo = 0; h_lo < H1; h_lo += kHMax)
                shrink_chunk(t, x, A_stack, H1, h_lo, min(H1, h_lo + kHMax), lds,
                             [&](int i, int k, float v) { sv[i * R + k] += v; });
            expand_prefetch<DT, R>(er, B, yr, t.nrows, H2, c0);
            expand_apply<DT, R>(er, s_a(lds), sv, s_vh(lds), s_max(lds), yr, t.nrows, H2, c0,
                                scale, B);
            return;
        }
        expand_prefetch<DT, R>(er, B, yr, t.nrows, H2, c0);
        if (tid == 0) *s_flag = wait_for_producers(cnt, ksplit, wait_ticks);
        __syncthreads();
        if (*s_flag) {
            for (int e = tid; e < kT * R; e += NT) {
                const int i = e / R;
                const int k = e - i * R;
                sv[e] = i < t.nrows ? sum_partials_coherent(
                                          partials + (long long)(t.row0 + i) * R + k,
                                          row_stride, ksplit)
                                    : 0.f;
            }
        } else {
            if (tid == 0) __hip_atomic_store(flag, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            for (int e = tid; e < kT * R; e += NT) sv[e] = 0.f;
            __syncthreads();
            for (int pp = 0; pp < ksplit; ++pp) {
                const int h_lo = pp * hps;
                const int h_hi = min(H1, h_lo + hps);
                shrink_chunk(t, x, A_stack, H1, h_lo, h_hi, lds,
                             [&](int i, int k, float v) { sv[i * R + k] += v; });
            }
            expand_prefetch<DT, R>(er, B, yr, t.nrows, H2, c0);
        }
        __syncthreads();
        int before = 0;
        if (tid == 0) before = depart_begin(cnt, 1 << 16);
        expand_apply<DT, R>(er, s_a(lds), sv, s_vh(lds), s_max(lds), yr, t.nrows, H2, c0, scale,
                            B);
        if (tid == 0) depart_end(cnt, before, 1 << 16, total);
    }

    __device__ static __forceinline__ void shrink_split(const Tile& t, int p, int hps, int ksplit,
                                                        const st* __restrict__ x,
                                                        const st* __restrict__ A_stack, int H1,
                                                        float* partials, long long row_stride,
                                                        float* v_final, int* cnt, int* s_last,
                                                        unsigned char* lds) {
        const int h_lo = p * hps;
        const int h_hi = min(H1, h_lo + hps);
        float* out = partials + (long long)p * row_stride + (long long)t.row0 * R;
        shrink_range(t, x, A_stack, H1, h_lo, h_hi, lds, [&](int i, int k, float v) {
            if (v_final) store_partial(&out[i * R + k], v);
            else out[i * R + k] = v;
        });
        if (v_final) reduce_if_last<R>(t, ksplit, partials, row_stride, v_final, cnt, s_last);
    }

    __device__ static __forceinline__ void expand_split(const Tile& t, int c, st* __restrict__ y,
                                                        const st* __restrict__ B_stack, int H2,
                                                        float scale,
                                                        const float* __restrict__ partials,
                                                        long long row_stride, int P,
                                                        unsigned char* lds) {
        const int c0 = c * kCW;
        float* sv = s_v(lds);
        st* yr = y + (long long)t.row0 * H2;
        ExpandRegs<R> er;
        expand_prefetch<DT, R>(er, B_stack + (long long)t.adapter * R * H2, yr, t.nrows, H2, c0);
        for (int e = threadIdx.x; e < kT * R; e += NT) {
            const int i = e / R;
            sv[e] = i < t.nrows ? sum_partials(partials + (long long)(t.row0 + i) * R + (e - i * R),
                                               row_stride, P)
                                : 0.f;
        }
        __syncthreads();
        expand_apply<DT, R>(er, s_a(lds), sv, s_vh(lds), s_max(lds), yr, t.nrows, H2, c0, scale,
                            B_stack + (long long)t.adapter * R * H2);
    }
};

// ---------------------------------------------------------------------------
// A class that a combination of dtype and rank does not use: never called.
// ---------------------------------------------------------------------------
template <typename DT>
struct NoTile {
    using st = typename DT::storage;
    static constexpr int kT = 1;
    static constexpr int kLdsBytes = 16;
    __device__ static __forceinline__ void shrink_item(const Tile&, int, int, const st*,
                                                       const st*, int, float*, long long, int*,
                                                       int, unsigned char*) {}
    __device__ static __forceinline__ void expand_item(const Tile&, int, st*, const st*,
                                                       const st*, const st*, int, int, float,
                                                       float*, long long, int, int, int*, int, int*,
                                                       long long, unsigned char*) {}
    __device__ static __forceinline__ void shrink_split(const Tile&, int, int, int, const st*,
                                                        const st*, int, float*, long long, float*,
                                                        int*, int*, unsigned char*) {}
    __device__ static __forceinline__ void expand_split(const Tile&, int, st*, const st*, int,
                                                        float, const float*, long long, int,
                                                        unsigned char*) {}
};

template <typename P>
struct IsNoTile : std::false_type {};
template <typename DT>
struct IsNoTile<NoTile<DT>> : std::true_type {};

// The short class: 4-row vector tiles with 8 rows of B in flight (its four
// rows of y and 32 accumulators then leave room under 128 registers).
template <typename DT, int R>
using ShortTile = VecTile<DT, R, 4, (R < 8 ? R : 8)>;

// The single class in the two-launch expand: 8 rows of B in flight, which
// keeps that kernel at five workgroups per compute unit beside the MFMA
// tiles (nothing is prefetched ahead of a wait there).
template <typename DT, int R>
using SplitSingle = VecTile<DT, R, 1, (R < 8 ? R : 8)>;

// The three classes' policies and the length at which a segment turns long.
template <typename LP, typename SP, typename GP>
struct MixedClasses {
    static constexpr bool kHasLong = !IsNoTile<LP>::value;
    static constexpr bool kHasShort = !IsNoTile<SP>::value;
    static constexpr int kTH = !kHasLong ? 0x7FFFFFFF : (kHasShort ? 16 : 2);
    static constexpr int kLds0 = LP::kLdsBytes > SP::kLdsBytes ? LP::kLdsBytes : SP::kLdsBytes;
    static constexpr int kLdsBytes = kLds0 > GP::kLdsBytes ? kLds0 : GP::kLdsBytes;
    // tiles of a segment of n rows in class c (0 long, 1 short, 2 single)
    __device__ static __forceinline__ int tiles(int c, int n) {
        if (c == 0) return n >= kTH ? (n + LP::kT - 1) / LP::kT : 0;
        if (c == 1) return (n >= 2 && n < kTH) ? (n + SP::kT - 1) / SP::kT : 0;
        return n == 1 ? 1 : 0;
    }
    __device__ static __forceinline__ int height(int c) {
        return c == 0 ? LP::kT : (c == 1 ? SP::kT : 1);
    }
};

// ---------------------------------------------------------------------------
// The class-aware scan of the segment table.
// ---------------------------------------------------------------------------
struct MixedScan {
    int lo[kMixedPasses], n[kMixedPasses], aid[kMixedPasses];  // n = 0: no rows or no adapter
    int e[3][kMixedPasses];  // tiles of each class before this thread's segment
    int total[3];            // tiles of each class
};

// LDS of the scan: per-pass wave totals of the three classes, then the
// four ints of the found tile.
constexpr int kMixedScanInts = kMixedPasses * 3 * (kMixedThreads / kWave) + 4;

// Every thread of the block calls this.  `lds` holds kMixedScanInts ints;
// each pass has its own slots, so one barrier per pass suffices, and the
// found tile (the last four ints) is set to an empty tile -- no rows of
// adapter 0 -- before that barrier.
template <typename C>
__device__ __forceinline__ void mixed_scan(const int* __restrict__ seg_indptr,
                                           const int* __restrict__ adapter_ids, int S,
                                           int num_rows, int num_adapters, int* lds,
                                           MixedScan& m) {
    constexpr int NT = kMixedThreads;
    constexpr int NW = NT / kWave;
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wid = tid / kWave;
    // Every load in flight before the first use: no load sits in a branch
    // (entries past the table re-read its last one and are masked below).
    int raw_lo[kMixedPasses], raw_hi[kMixedPasses], raw_a[kMixedPasses];
#pragma unroll
    for (int p = 0; p < kMixedPasses; ++p) {
        const int sc = min(p * NT + tid, S - 1);
        raw_lo[p] = seg_indptr[sc];
        raw_hi[p] = seg_indptr[sc + 1];
        raw_a[p] = adapter_ids[sc];
    }
    if (tid == 0) {
        int* found = lds + kMixedScanInts - 4;
        found[0] = 0;
        found[1] = 0;
        found[2] = 0;
        found[3] = -1;
    }
    int run[3] = {0, 0, 0};
#pragma unroll
    for (int p = 0; p < kMixedPasses; ++p) {
        int* tot_lds = lds + p * 3 * NW;
        const bool in = p * NT + tid < S;
        const int lo = min(max(raw_lo[p], 0), num_rows);
        const int hi = min(max(raw_hi[p], lo), num_rows);
        const bool ok = in && raw_a[p] >= 0 && raw_a[p] < num_adapters && hi > lo;
        const int n = ok ? hi - lo : 0;
        m.lo[p] = lo;
        m.n[p] = n;
        m.aid[p] = raw_a[p];
        if (p * NT >= S) {  // block-uniform
#pragma unroll
            for (int c = 0; c < 3; ++c) m.e[c][p] = 0;
            continue;
        }
        int cnt[3], incl[3];
#pragma unroll
        for (int c = 0; c < 3; ++c) {
            cnt[c] = C::tiles(c, n);
            incl[c] = wave_inclusive_scan(cnt[c], lane);
        }
        if (lane == kWave - 1) {
#pragma unroll
            for (int c = 0; c < 3; ++c) tot_lds[c * NW + wid] = incl[c];
        }
        __syncthreads();
#pragma unroll
        for (int c = 0; c < 3; ++c) {
            int off = 0, tot = 0;
#pragma unroll
            for (int w = 0; w < NW; ++w) {
                const int v = tot_lds[c * NW + w];
                off += w < wid ? v : 0;
                tot += v;
            }
            m.e[c][p] = run[c] + off + incl[c] - cnt[c];
            run[c] += tot;
        }
    }
#pragma unroll
    for (int c = 0; c < 3; ++c) m.total[c] = run[c];
}

// The owner of tile t of class CC (a thread whose segment holds it) writes
// the tile to `found`.  CC is a template argument so that the scan state is
// indexed statically and stays in registers.
template <typename C, int CC>
__device__ __forceinline__ void mixed_find_class(const MixedScan& m, int S, int t, int* found) {
    const int h = C::height(CC);
#pragma unroll
    for (int p = 0; p < kMixedPasses; ++p) {
        const int s = p * kMixedThreads + (int)threadIdx.x;
        const int n = m.n[p];
        const int cnt = C::tiles(CC, n);
        const int e = m.e[CC][p];
        if (s < S && cnt > 0 && t >= e && t < e + cnt) {
            const int row0 = m.lo[p] + (t - e) * h;
            found[0] = row0;
            found[1] = min(h, m.lo[p] + n - row0);
            found[2] = m.aid[p];
            found[3] = s;
        }
    }
}

// Tile t of class c (block-uniform); t must be below that class's total.
// Every thread of the block calls this, after mixed_scan on the same LDS
// (`lds`); if no segment held tile t the caller would see the empty tile
// mixed_scan left there.
template <typename C>
__device__ __forceinline__ Tile mixed_find(const MixedScan& m, int S, int c, int t, int* lds) {
    int* found = lds + kMixedScanInts - 4;
    if (c == 0) mixed_find_class<C, 0>(m, S, t, found);
    else if (c == 1) mixed_find_class<C, 1>(m, S, t, found);
    else mixed_find_class<C, 2>(m, S, t, found);
    __syncthreads();
    Tile out;
    out.row0 = found[0];
    out.nrows = found[1];
    out.adapter = found[2];
    out.seg = found[3];
    return out;
}

// Splits of the three classes: chunks of H1 (k), rows of A per chunk (h),
// column chunks (c).
struct MixedSplit {
    int k[3], h[3], c[3];
};


// Item decode: blocks of total * per items, taken in order.  take() moves
// q past a block, or names (tile, sub) inside it.  Everything stays in
// scalars (no array indexed at run time, which would go to scratch).
__device__ __forceinline__ bool take_item(int& q, int total, int per, int& t, int& sub) {
    const int n = total * per;
    if (per > 0 && q < n) {
        t = q / per;
        sub = q - t * per;
        return true;
    }
    q -= n;
    return false;
}

// ---------------------------------------------------------------------------
// lora_apply in one launch, the path chosen per segment.
// ---------------------------------------------------------------------------
template <typename DT, int R, typename LP, typename SP, typename GP>
__global__ __launch_bounds__(kMixedThreads, 4) void lora_mixed_kernel(
    typename DT::storage* __restrict__ y, const typename DT::storage* __restrict__ x,
    const typename DT::storage* __restrict__ A_stack,
    const typename DT::storage* __restrict__ B_stack, const int* __restrict__ seg_indptr,
    const int* __restrict__ adapter_ids, int S, int num_rows, int num_adapters, int H1, int H2,
    float scale, float* __restrict__ partials, int* __restrict__ counters, MixedSplit sp,
    int n_counters, int counter_stride, long long wait_ticks, int guess) {
    using C = MixedClasses<LP, SP, GP>;
    __shared__ __align__(16) unsigned char s_mem[C::kLdsBytes];
    __shared__ int s_scan[kMixedScanInts];
    // guess: a table shape the host expects, so that a shrink item streams
    // its chunk of A before the scan below would have named it.  1 (as many
    // rows as segments, a decode batch): segment i is row i alone, a one-row
    // tile of the single class.  2 (one segment): the segment is every row,
    // cut into tiles of its class.  The guess is checked -- the whole table
    // as guessed, adapters in range, the same table for every workgroup --
    // before anything is published; if it fails, the item runs the scanned
    // path.
    if (guess) {
        int gc, gT;  // the guessed class of every tile, and its tile count
        if (guess == 1) {
            gc = 2;
            gT = S;
        } else {
            gc = num_rows >= C::kTH ? 0 : (num_rows >= 2 ? 1 : 2);
            gT = C::tiles(gc, num_rows);
        }
        if ((int)blockIdx.x < gT * sp.k[gc]) {  // block-uniform
            auto guessed = [&](auto pol) -> bool {
                using P = decltype(pol);
                if constexpr (IsNoTile<P>::value) {
                    return false;
                } else {
                    const int tid = threadIdx.x;
                    int raw_seg[kMixedPasses], raw_id[kMixedPasses];
#pragma unroll
                    for (int p = 0; p < kMixedPasses; ++p) {  // in flight beside the A chunk
                        const int j = p * kMixedThreads + tid;
                        raw_seg[p] = seg_indptr[min(j, S)];
                        raw_id[p] = adapter_ids[min(j, S - 1)];
                    }
                    const int ti = (int)blockIdx.x / sp.k[gc];
                    const int sub = (int)blockIdx.x - ti * sp.k[gc];
                    const int h = C::height(gc);
                    Tile t;
                    t.row0 = guess == 1 ? ti : ti * h;
                    t.nrows = guess == 1 ? 1 : min(h, num_rows - t.row0);
                    const int a_raw = adapter_ids[guess == 1 ? ti : 0];
                    t.adapter = (a_raw >= 0 && a_raw < num_adapters) ? a_raw : 0;  // in range
                    t.seg = guess == 1 ? ti : 0;
                    float* s_gv = P::s_v(s_mem);
                    const int h_lo = sub * sp.h[gc];
                    const int h_hi = min(H1, h_lo + sp.h[gc]);
                    P::shrink_range(t, x, A_stack, H1, h_lo, h_hi, s_mem,
                                    [&](int i, int k, float v) { s_gv[i * R + k] = v; });
                    bool ok = true;
#pragma unroll
                    for (int p = 0; p < kMixedPasses; ++p) {
                        const int j = p * kMixedThreads + tid;
                        const int want = guess == 1 ? j : (j == 0 ? 0 : num_rows);
                        if (j <= S) ok = ok && raw_seg[p] == want;
                        if (j < S) ok = ok && raw_id[p] >= 0 && raw_id[p] < num_adapters;
                    }
                    if (!__syncthreads_and(ok)) {
                        __syncthreads();  // LDS free for the scanned path
                        return false;
                    }
                    float* out = partials + (long long)sub * num_rows * R + (long long)t.row0 * R;
                    for (int e = tid; e < t.nrows * R; e += kMixedThreads)
                        store_partial(&out[e], s_gv[e]);
                    __atomic_signal_fence(__ATOMIC_SEQ_CST);
                    __builtin_amdgcn_s_waitcnt(0);
                    __syncthreads();
                    // every other class is empty, so tile ti has counter slot ti
                    if (tid == 0)
                        depart(&counters[(long long)ti * counter_stride], 1,
                               sp.k[gc] + (sp.c[gc] << 16));
                    return true;
                }
            };
            const bool done =
                gc == 0 ? guessed(LP{}) : (gc == 1 ? guessed(SP{}) : guessed(GP{}));
            if (done) return;
        }
    }
    MixedScan m;
    mixed_scan<C>(seg_indptr, adapter_ids, S, num_rows, num_adapters, s_scan, m);
    const int T0 = m.total[0], T1 = m.total[1], T2 = m.total[2];
    int q = (int)blockIdx.x, ti = 0, sub = 0, kind;
    if (take_item(q, T0, sp.k[0], ti, sub)) kind = 0;
    else if (take_item(q, T1, sp.k[1], ti, sub)) kind = 1;
    else if (take_item(q, T2, sp.k[2], ti, sub)) kind = 2;
    else if (take_item(q, T0, sp.c[0], ti, sub)) kind = 3;
    else if (take_item(q, T1, sp.c[1], ti, sub)) kind = 4;
    else if (take_item(q, T2, sp.c[2], ti, sub)) kind = 5;
    else return;  // past the real item count (block-uniform)
    const int c = kind < 3 ? kind : kind - 3;
    const Tile t = mixed_find<C>(m, S, c, ti, s_scan);
    const long long row_stride = (long long)num_rows * R;
    const int slot = c == 0 ? ti : (c == 1 ? T0 + ti : T0 + T1 + ti);
    int* cnt = &counters[(long long)slot * counter_stride];
    int* flag = &counters[n_counters - 1];
    switch (kind) {
        case 0:
            LP::shrink_item(t, sub, sp.h[0], x, A_stack, H1, partials, row_stride, cnt,
                            sp.k[0] + (sp.c[0] << 16), s_mem);
            break;
        case 1:
            SP::shrink_item(t, sub, sp.h[1], x, A_stack, H1, partials, row_stride, cnt,
                            sp.k[1] + (sp.c[1] << 16), s_mem);
            break;
        case 2:
            GP::shrink_item(t, sub, sp.h[2], x, A_stack, H1, partials, row_stride, cnt,
                            sp.k[2] + (sp.c[2] << 16), s_mem);
            break;
        case 3:
            LP::expand_item(t, sub, y, x, A_stack, B_stack, H1, H2, scale, partials, row_stride,
                            sp.k[0], sp.h[0], cnt, sp.k[0] + (sp.c[0] << 16), flag, wait_ticks,
                            s_mem);
            break;
        case 4:
            SP::expand_item(t, sub, y, x, A_stack, B_stack, H1, H2, scale, partials, row_stride,
                            sp.k[1], sp.h[1], cnt, sp.k[1] + (sp.c[1] << 16), flag, wait_ticks,
                            s_mem);
            break;
        default:
            GP::expand_item(t, sub, y, x, A_stack, B_stack, H1, H2, scale, partials, row_stride,
                            sp.k[2], sp.h[2], cnt, sp.k[2] + (sp.c[2] << 16), flag, wait_ticks,
                            s_mem);
            break;
    }
}

// The expand launch's item table, written by the shrink launch of the same
// call: entry q is expand item q (its tile and its column chunk: row0,
// nrows, adapter, class | chunk << 2), and the int after the last of
// n_max entries holds how many entries this call wrote.  Every entry below
// that count is rewritten by each call, so the table needs no clearing.
__device__ __forceinline__ int* item_count(int4* items, int n_max) {
    return reinterpret_cast<int*>(items + n_max);
}

// The shrink half of the two-launch form: [long][short][single] shrink
// items.  With v_final (sgmv_shrink), each tile's last item reduces the
// partials into v (tile counters: long tiles, then short, then single).
// With items, each tile's first item also writes the tile's expand items
// (the expand launch then reads its item instead of scanning the table).
template <typename DT, int R, typename LP, typename SP, typename GP>
__global__ __launch_bounds__(kMixedThreads, R <= 32 ? 6 : (R == 64 ? 5 : 1)) void shrink_mixed_kernel(
    const typename DT::storage* __restrict__ x, const typename DT::storage* __restrict__ A_stack,
    const int* __restrict__ seg_indptr, const int* __restrict__ adapter_ids, int S, int num_rows,
    int num_adapters, int H1, float* __restrict__ partials, MixedSplit sp,
    float* __restrict__ v_final, int* __restrict__ counters, int counter_stride,
    int4* __restrict__ items, int n_items_max) {
    using C = MixedClasses<LP, SP, GP>;
    __shared__ __align__(16) unsigned char s_mem[C::kLdsBytes];
    __shared__ int s_scan[kMixedScanInts];
    __shared__ int s_last;
    MixedScan m;
    mixed_scan<C>(seg_indptr, adapter_ids, S, num_rows, num_adapters, s_scan, m);
    const int T0 = m.total[0], T1 = m.total[1], T2 = m.total[2];
    const int E1 = T0 * sp.c[0], E2 = E1 + T1 * sp.c[1];  // first expand item of each class
    if (items && blockIdx.x == 0 && threadIdx.x == 0)
        *item_count(items, n_items_max) = min(E2 + T2 * sp.c[2], n_items_max);
    int q = (int)blockIdx.x, ti = 0, sub = 0, c;
    if (take_item(q, T0, sp.k[0], ti, sub)) c = 0;
    else if (take_item(q, T1, sp.k[1], ti, sub)) c = 1;
    else if (take_item(q, T2, sp.k[2], ti, sub)) c = 2;
    else return;
    const Tile t = mixed_find<C>(m, S, c, ti, s_scan);
    const long long row_stride = (long long)num_rows * R;
    const int slot = c == 0 ? ti : (c == 1 ? T0 + ti : T0 + T1 + ti);
    int* cnt = v_final ? &counters[(long long)slot * counter_stride] : nullptr;
    if (c == 0)
        LP::shrink_split(t, sub, sp.h[0], sp.k[0], x, A_stack, H1, partials, row_stride, v_final,
                         cnt, &s_last, s_mem);
    else if (c == 1)
        SP::shrink_split(t, sub, sp.h[1], sp.k[1], x, A_stack, H1, partials, row_stride, v_final,
                         cnt, &s_last, s_mem);
    else
        GP::shrink_split(t, sub, sp.h[2], sp.k[2], x, A_stack, H1, partials, row_stride, v_final,
                         cnt, &s_last, s_mem);
    // after the stream, where its registers are free
    if (items && sub == 0) {
        const int per = sp.c[c];
        const int base = (c == 0 ? 0 : (c == 1 ? E1 : E2)) + ti * per;
        for (int s = (int)threadIdx.x; s < per; s += kMixedThreads)
            if (base + s < n_items_max)
                items[base + s] = make_int4(t.row0, t.nrows, t.adapter, c | (s << 2));
    }
}

// The expand half: [long][short][single] expand items.  Rows of class c
// have P[c] partials (sgmv_expand: 1, the partial is v).  With items (the
// table the shrink launch of the same call wrote), a workgroup reads its
// item there; else it scans the segment table.
template <typename DT, int R, typename LP, typename SP, typename GP>
__global__ __launch_bounds__(kMixedThreads, R >= 64 ? 4 : 5) void expand_mixed_kernel(
    typename DT::storage* __restrict__ y, const typename DT::storage* __restrict__ B_stack,
    const int* __restrict__ seg_indptr, const int* __restrict__ adapter_ids, int S, int num_rows,
    int num_adapters, int H2, float scale, const float* __restrict__ partials, MixedSplit sp,
    int P_long, int P_short, int P_single, const int4* __restrict__ items, int n_items_max) {
    using C = MixedClasses<LP, SP, GP>;
    __shared__ __align__(16) unsigned char s_mem[C::kLdsBytes];
    __shared__ int s_scan[kMixedScanInts];
    Tile t;
    int c, sub;
    if (items) {
        // both loads in flight together; the entry is in the table even
        // for workgroups past the count (the grid is at most n_items_max)
        const int n = *item_count(const_cast<int4*>(items), n_items_max);
        const int4 e = items[blockIdx.x];
        if ((int)blockIdx.x >= n) return;
        t.row0 = e.x;
        t.nrows = e.y;
        t.adapter = e.z;
        t.seg = -1;
        c = e.w & 3;
        sub = e.w >> 2;
    } else {
        MixedScan m;
        mixed_scan<C>(seg_indptr, adapter_ids, S, num_rows, num_adapters, s_scan, m);
        const int T0 = m.total[0], T1 = m.total[1], T2 = m.total[2];
        int q = (int)blockIdx.x, ti = 0;
        if (take_item(q, T0, sp.c[0], ti, sub)) c = 0;
        else if (take_item(q, T1, sp.c[1], ti, sub)) c = 1;
        else if (take_item(q, T2, sp.c[2], ti, sub)) c = 2;
        else return;
        t = mixed_find<C>(m, S, c, ti, s_scan);
    }
    const long long row_stride = (long long)num_rows * R;
    if (c == 0)
        LP::expand_split(t, sub, y, B_stack, H2, scale, partials, row_stride, P_long, s_mem);
    else if (c == 1)
        SP::expand_split(t, sub, y, B_stack, H2, scale, partials, row_stride, P_short, s_mem);
    else
        GP::expand_split(t, sub, y, B_stack, H2, scale, partials, row_stride, P_single, s_mem);
}

}  // namespace sgmv
