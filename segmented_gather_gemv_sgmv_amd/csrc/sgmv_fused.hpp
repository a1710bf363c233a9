// sgmv_fused.hpp -- lora_apply in one launch: shrink and expand of every
// segment tile, with the float32 intermediate handed from the shrink
// workgroups to the expand workgroups through the workspace.
//
// Why one launch: a decode-shaped call moves only tens of MB, so a second
// launch (and the drain and ramp around it) costs as much as the data; the
// expand workgroups also start streaming their B and y while the shrink is
// still running (the pages stress that fusing the gather-multiply avoids
// kernel-launch overhead: Punica walkthrough, omica.com.cn/news/959180,
// section 2.2).
//
// Items.  Workgroup b < slots*ksplit is shrink item (tile g, H1 chunk p): it
// writes the chunk's partial sums of v for the tile rows, waits until those
// stores are acknowledged, then adds one to the tile's arrival counter.
// Workgroup b beyond is expand item (tile g, column chunk c): it issues its
// B and y loads, polls until the tile's counter reaches ksplit, sums the
// partials in chunk order and updates y.  Every access to the partials and
// the counter is a relaxed atomic at agent scope; the ordering comes from
// waiting on the memory counters, not from release/acquire (see "Hand-off
// without L2 write-backs" below).
//
// Progress.  Shrink items never wait, and a workgroup's index is below every
// expand index, so on hardware that dispatches each XCD's workgroups in index
// order the waits always end.  The wait is nevertheless bounded in time; a
// workgroup that runs out of patience computes the tile's partials itself
// with the same code and in the same order, so the result is bit-identical
// either way and the kernel never hangs.
//
// Hand-off without L2 write-backs.  A release fence at agent scope writes
// back the whole L2 of the XCD (measured at microseconds per workgroup) and
// an acquire invalidates it, so the protocol uses neither.  The partials
// are written with relaxed agent-scope atomic stores, which gfx950 performs
// write-through to the device coherence point; every wave waits until its
// stores are acknowledged (s_waitcnt vmcnt(0)) before the workgroup
// barrier, and only then does thread 0 add to the arrival counter.  Readers
// poll the counter and read the partials with relaxed agent-scope atomic
// loads, which bypass the non-coherent caches.  The counter is thus
// published only after the data it announces has reached the coherence
// point, and no reader can see a stale copy.  This rests on how gfx950
// implements agent-scope atomics (write-through stores, cache-bypassing
// loads) and on the store acknowledgement, not on the HIP memory model's
// release/acquire rules, which would demand the fences above; the tests
// exercise it (bit-identity with the self-contained path, determinism,
// graph replays).
//
// Counters.  counters[g * counter_stride] of tile slot g (one cache line per
// tile, so that atomics of different tiles do not contend) counts the
// tile's participants: each
// of its ksplit shrink items adds 1 once its partials are stored, each of
// its csplit expand items adds 1 << 16 once it no longer needs the
// partials.  Expand items wait for the low half to reach ksplit.  The
// participant whose addition completes the count (ksplit + csplit << 16)
// returns the counter to zero, so the workspace is ready for the next call
// (and for a graph replay) without a memset; it must be zero before its
// first use.  Because every participant counts, a late shrink item (one
// whose expand items stopped waiting) still finishes before the reset.  One
// counter per tile keeps same-address atomics to ksplit + csplit per call
// (cross-XCD atomics on one address serialise).  counters[n_counters-1] is
// a sticky flag recording that some expand item stopped waiting.
#pragma once

#include "sgmv_device.hpp"
#include "sgmv_gemv.hpp"

namespace sgmv {

// One H1 chunk of the shrink for one tile, reduced across the workgroup.
// Calls emit(i, k, value) once for every (row i < nrows, column k < R), from
// threads tid < R * RB; the values are bit-identical for identical inputs.
// The caller must synchronise the block before s_red is used again.
template <typename DT, int R, int NT, int RB, int PG, typename Emit>
__device__ __forceinline__ void shrink_chunk(const typename DT::storage* __restrict__ A,
                                             const typename DT::storage* __restrict__ xr,
                                             int nrows, int H1, int h_lo, int h_hi,
                                             float* s_red, Emit&& emit) {
    constexpr int VEC = DT::kVec;
    constexpr int LPR = R / VEC;
    constexpr int HPB = NT / LPR;
    constexpr int NW = NT / kWave;
    constexpr int N = RB * VEC;
    using RS = ReduceScatter<N, LPR>;
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wid = tid / kWave;
    const int h_lane = tid / LPR;
    const int k0 = (tid % LPR) * VEC;

    float acc[N];
#pragma unroll
    for (int i = 0; i < N; ++i) acc[i] = 0.f;

    for (int hb = h_lo; hb < h_hi; hb += HPB * PG) {
        uint4 av[PG];
        float xv[PG][RB];
#pragma unroll
        for (int q = 0; q < PG; ++q) {
            const int h = hb + q * HPB + h_lane;
            const bool in = h < h_hi;
            av[q] = in ? load16(A + (long long)h * R + k0) : make_uint4(0, 0, 0, 0);
#pragma unroll
            for (int i = 0; i < RB; ++i)
                xv[q][i] = (in && i < nrows) ? DT::load1(xr + (long long)i * H1 + h) : 0.f;
        }
#pragma unroll
        for (int q = 0; q < PG; ++q) {
            float af[VEC];
            DT::unpack(av[q], af);
#pragma unroll
            for (int i = 0; i < RB; ++i) {
                if (i < nrows) {
#pragma unroll
                    for (int c = 0; c < VEC; ++c)
                        acc[i * VEC + c] = fmaf(xv[q][i], af[c], acc[i * VEC + c]);
                }
            }
        }
    }

    int offset;
    bool canon;
    RS::run(acc, lane, offset, canon);
    if (canon) {
        const int kq = lane % LPR;
#pragma unroll
        for (int i = 0; i < RS::kRemain; ++i) s_red[wid * (LPR * N) + kq * N + offset + i] = acc[i];
    }
    __syncthreads();
    for (int t = tid; t < LPR * N; t += NT) {
        const int kq = t / N;
        const int idx = t - kq * N;
        const int i = idx / VEC;
        const int k = kq * VEC + (idx - i * VEC);
        float sum = 0.f;
#pragma unroll
        for (int w = 0; w < NW; ++w) sum += s_red[w * (LPR * N) + t];
        if (i < nrows) emit(i, k, sum);
    }
}

// Adds `amount` to a tile counter; the participant that completes `total`
// returns the counter to zero.  The wait makes the workgroup's earlier
// memory operations (partial stores, poll loads) complete first.
__device__ __forceinline__ void depart(int* counter, int amount, int total) {
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0);
    const int before = __hip_atomic_fetch_add(counter, amount, __ATOMIC_RELAXED,
                                              __HIP_MEMORY_SCOPE_AGENT);
    if (before + amount == total)
        __hip_atomic_store(counter, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// An expand item counts itself out in two steps so that the round trip of
// its atomic overlaps its compute: depart_begin() issues the addition once
// the partials are in LDS (nothing it does afterwards touches the partials
// or the counter, so nothing needs to complete first), and depart_end(),
// after the compute, resets the counter if this item completed the count.
__device__ __forceinline__ int depart_begin(int* counter, int amount) {
    return __hip_atomic_fetch_add(counter, amount, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void depart_end(int* counter, int before, int amount, int total) {
    if (before + amount == total)
        __hip_atomic_store(counter, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Thread 0 of an expand item: waits until the tile's ksplit shrink items
// have published (low half of the counter), polling with relaxed loads.
// Bounded by the wall clock and, independently, by a count of polls (each
// poll sleeps >= 128 cycles), so it ends even if the clock stood still.
// Returns false when it gave up (or wait_ticks < 0: do not wait at all).
__device__ __forceinline__ bool wait_for_producers(int* cnt, int ksplit, long long wait_ticks) {
    if (wait_ticks < 0) return false;
    if ((__hip_atomic_load(cnt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) & 0xFFFF) >= ksplit)
        return true;
    const long long t0 = wall_clock64();
    for (int polls = 0;; ++polls) {
        if ((__hip_atomic_load(cnt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) & 0xFFFF) >= ksplit)
            return true;
        if (wall_clock64() - t0 > wait_ticks || polls >= (1 << 22)) return false;
        __builtin_amdgcn_s_sleep(2);
    }
}

// Sum of the ksplit published chunk partials p[0], p[stride], ... in chunk
// order, read with agent-scope loads (batches of 16 in flight: each batch
// is one dependent round trip on the expand's critical path).
__device__ __forceinline__ float sum_partials_coherent(float* p, long long stride, int ksplit) {
    constexpr int kBatch = 16;
    float sum = 0.f;
    for (int p0 = 0; p0 < ksplit; p0 += kBatch) {
        float tv[kBatch];
#pragma unroll
        for (int u = 0; u < kBatch; ++u)
            tv[u] = (p0 + u < ksplit) ? __hip_atomic_load(p + (long long)(p0 + u) * stride,
                                                          __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                                      : 0.f;
#pragma unroll
        for (int u = 0; u < kBatch; ++u)
            if (p0 + u < ksplit) sum += tv[u];
    }
    return sum;
}

// Stores one partial sum so that it is visible at agent scope once the
// storing wave's memory counter drains (write-through, no L2 write-back).
__device__ __forceinline__ void store_partial(float* p, float v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Position of workgroup blockIdx.x among the items: shrink then expand items
// of the first slots_a tile slots, then shrink then expand items of the
// remaining slots_b.  Every expand item follows all shrink items of its tile.
struct Item {
    bool shrink;
    int g;    // tile slot
    int sub;  // H1 chunk (shrink) or column chunk (expand)
};

__device__ __forceinline__ Item decode_item(int slots_a, int slots_b, int ksplit, int csplit) {
    long long item = blockIdx.x;
    int base = 0, nslots = slots_a;
    if (item >= (long long)slots_a * (ksplit + csplit)) {
        item -= (long long)slots_a * (ksplit + csplit);
        base = slots_a;
        nslots = slots_b;
    }
    const long long n_shrink = (long long)nslots * ksplit;
    Item it;
    it.shrink = item < n_shrink;
    if (it.shrink) {
        it.g = base + (int)(item / ksplit);
        it.sub = (int)(item % ksplit);
    } else {
        const long long e = item - n_shrink;
        it.g = base + (int)(e / csplit);
        it.sub = (int)(e % csplit);
    }
    return it;
}

// One item of the single-kernel lora_apply: the shrink of H1 chunk `sub`
// (is_shrink) or the expand of column chunk `sub` of tile slot g.  `counters`
// holds the tile counters of this problem; `flag` is the sticky flag.
template <typename DT, int R, int NT, int RB, int PG, int KB>
__device__ __forceinline__ void fused_item(
    bool is_shrink, int g, int sub, typename DT::storage* __restrict__ y,
    const typename DT::storage* __restrict__ x, const typename DT::storage* __restrict__ A_stack,
    const typename DT::storage* __restrict__ B_stack, const int* __restrict__ seg_indptr,
    const int* __restrict__ adapter_ids, int S, int num_rows, int num_adapters, int H1, int H2,
    float scale, float* __restrict__ partials, int* __restrict__ counters, int ksplit,
    int h_per_split, int csplit, int compact, int* flag, int counter_stride,
    long long wait_ticks) {
    using st = typename DT::storage;
    constexpr int VEC = DT::kVec;
    constexpr int CW = NT * VEC;  // columns per expand item
    constexpr int NW = NT / kWave;
    constexpr int LPR = R / VEC;
    constexpr int N = RB * VEC;
    static_assert(R % KB == 0, "KB must divide R");

    __shared__ int s_scan[tile_scan_ints<NT>()];
    __shared__ float s_red[NW * LPR * N];
    __shared__ float s_v[RB * R];
    __shared__ int s_flag;

    const int tid = threadIdx.x;
    const long long row_stride = (long long)num_rows * R;  // between chunk partials

    auto locate = [&](int g, Tile& t) {
        return compact ? locate_tile_compact<NT>(seg_indptr, adapter_ids, S, num_rows,
                                                 num_adapters, RB, g, s_scan, t)
                       : locate_tile<NT>(seg_indptr, adapter_ids, S, num_rows, num_adapters,
                                         RB, g, s_scan, t);
    };

    if (is_shrink) {
        // ---------------- shrink item ----------------
        const int p = sub;
        Tile tile;
        if (locate(g, tile)) {
            const int h_lo = p * h_per_split;
            const int h_hi = min(H1, h_lo + h_per_split);
            const st* A = A_stack + (long long)tile.adapter * H1 * R;
            const st* xr = x + (long long)tile.row0 * H1;
            float* out = partials + (long long)p * row_stride + (long long)tile.row0 * R;
            shrink_chunk<DT, R, NT, RB, PG>(
                A, xr, tile.nrows, H1, h_lo, h_hi, s_red,
                [&](int i, int k, float v) { store_partial(&out[i * R + k], v); });
            // Each wave waits for its partial stores to be acknowledged; the
            // barrier then lets thread 0 announce them.
            __atomic_signal_fence(__ATOMIC_SEQ_CST);
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
            if (tid == 0) depart(&counters[g * counter_stride], 1, ksplit + (csplit << 16));
        }
    } else {
        // ---------------- expand item ----------------
        const int c = sub;
        Tile tile;
        if (locate(g, tile)) {
            const int nrows = tile.nrows;
            const int j = c * CW + tid * VEC;
            const bool active = j < H2;
            const st* B = B_stack + (long long)tile.adapter * R * H2 + j;

            // Loads that do not depend on v go out before the wait.
            uint4 bv[KB];
#pragma unroll
            for (int kk = 0; kk < KB; ++kk)
                bv[kk] = active ? load16(B + (long long)kk * H2) : make_uint4(0, 0, 0, 0);
            uint4 yv[RB];
#pragma unroll
            for (int i = 0; i < RB; ++i)
                yv[i] = (active && i < nrows)
                            ? load16(y + (long long)(tile.row0 + i) * H2 + j)
                            : make_uint4(0, 0, 0, 0);

            if (tid == 0) {
                // Poll with relaxed agent-scope loads (no cache invalidation
                // per poll); the partials are then read the same way.
                const int ok = wait_for_producers(&counters[g * counter_stride], ksplit, wait_ticks);
                s_flag = ok;
            }
            __syncthreads();
            const bool ready = s_flag != 0;

            if (ready) {
                for (int t = tid; t < RB * R; t += NT) {
                    const int i = t / R;
                    const int k = t - i * R;
                    float sum = 0.f;
                    if (i < nrows)
                        sum = sum_partials_coherent(partials + (long long)(tile.row0 + i) * R + k,
                                                    row_stride, ksplit);
                    s_v[t] = sum;
                }
            } else {
                // The producers are late: compute every chunk here, summing in
                // the same order as the normal path.
                if (tid == 0) __hip_atomic_store(flag, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                for (int t = tid; t < RB * R; t += NT) s_v[t] = 0.f;
                __syncthreads();
                const st* A = A_stack + (long long)tile.adapter * H1 * R;
                const st* xr = x + (long long)tile.row0 * H1;
                for (int pp = 0; pp < ksplit; ++pp) {
                    const int h_lo = pp * h_per_split;
                    const int h_hi = min(H1, h_lo + h_per_split);
                    shrink_chunk<DT, R, NT, RB, PG>(A, xr, nrows, H1, h_lo, h_hi, s_red,
                                                    [&](int i, int k, float v) { s_v[i * R + k] += v; });
                    __syncthreads();
                }
                // Load B and y again, so that the prefetched registers are not
                // held across this rarely taken path.
#pragma unroll
                for (int kk = 0; kk < KB; ++kk)
                    bv[kk] = active ? load16(B + (long long)kk * H2) : make_uint4(0, 0, 0, 0);
#pragma unroll
                for (int i = 0; i < RB; ++i)
                    yv[i] = (active && i < nrows)
                                ? load16(y + (long long)(tile.row0 + i) * H2 + j)
                                : make_uint4(0, 0, 0, 0);
            }
            __syncthreads();
            // The partials are in LDS now: this item no longer needs them.
            int before = 0;
            if (tid == 0) before = depart_begin(&counters[g * counter_stride], 1 << 16);

            float acc[RB][VEC];
#pragma unroll
            for (int i = 0; i < RB; ++i)
#pragma unroll
                for (int q = 0; q < VEC; ++q) acc[i][q] = 0.f;
#pragma unroll
            for (int kb = 0; kb < R; kb += KB) {
                if (kb > 0) {
#pragma unroll
                    for (int kk = 0; kk < KB; ++kk)
                        bv[kk] = active ? load16(B + (long long)(kb + kk) * H2)
                                        : make_uint4(0, 0, 0, 0);
                }
#pragma unroll
                for (int kk = 0; kk < KB; ++kk) {
                    float bf[VEC];
                    DT::unpack(bv[kk], bf);
#pragma unroll
                    for (int i = 0; i < RB; ++i) {
                        if (i < nrows) {
                            const float vv = s_v[i * R + kb + kk];
#pragma unroll
                            for (int q = 0; q < VEC; ++q) acc[i][q] = fmaf(vv, bf[q], acc[i][q]);
                        }
                    }
                }
            }
            if (active) {
#pragma unroll
                for (int i = 0; i < RB; ++i) {
                    if (i < nrows) {
                        float yf[VEC];
                        DT::unpack(yv[i], yf);
#pragma unroll
                        for (int q = 0; q < VEC; ++q) yf[q] = fmaf(scale, acc[i][q], yf[q]);
                        store16(y + (long long)(tile.row0 + i) * H2 + j, DT::pack(yf));
                    }
                }
            }
            if (tid == 0)
                depart_end(&counters[g * counter_stride], before, 1 << 16, ksplit + (csplit << 16));
        }
    }

    // ---------------- completion: the last workgroup resets the counters ----
}

template <typename DT, int R, int NT, int RB, int PG, int KB>
__global__ __launch_bounds__(NT) void lora_fused_kernel(
    typename DT::storage* __restrict__ y, const typename DT::storage* __restrict__ x,
    const typename DT::storage* __restrict__ A_stack,
    const typename DT::storage* __restrict__ B_stack, const int* __restrict__ seg_indptr,
    const int* __restrict__ adapter_ids, int S, int num_rows, int num_adapters, int H1, int H2,
    float scale, float* __restrict__ partials, int* __restrict__ counters, int ksplit,
    int h_per_split, int csplit, int slots_a, int slots_b, int compact, int n_counters,
    int counter_stride, long long wait_ticks) {
    const Item it = decode_item(slots_a, slots_b, ksplit, csplit);
    fused_item<DT, R, NT, RB, PG, KB>(it.shrink, it.g, it.sub, y, x, A_stack, B_stack, seg_indptr,
                                      adapter_ids, S, num_rows, num_adapters, H1, H2, scale,
                                      partials, counters, ksplit, h_per_split, csplit, compact,
                                      &counters[n_counters - 1], counter_stride, wait_ticks);
}

// ---------------------------------------------------------------------------
// Several add-ons over one batch in one launch (e.g. the LoRA projections of
// a layer): problem p has its own y, x, stacks, H1, H2, scale, plan,
// partials and tile counters, and all share the segment table.  Workgroups
// [sbase[p], sbase[p + 1]) are problem p's shrink items and, after every
// shrink item, [ebase[p], ebase[p + 1]) its expand items, so every wait is on
// lower-numbered workgroups, as in lora_fused_kernel.  A decode step pays the
// launch and the hand-off latency once for all its projections instead of
// once per projection (kernel-launch overhead matters at this scale: Punica
// walkthrough, omica.com.cn/news/959180, section 2.2).
// ---------------------------------------------------------------------------
constexpr int kMaxProblems = 8;

template <typename T>
struct MultiProblems {
    T* y[kMaxProblems];
    const T* x[kMaxProblems];
    const T* A[kMaxProblems];
    const T* B[kMaxProblems];
    float* partials[kMaxProblems];
    int* counters[kMaxProblems];
    int H1[kMaxProblems], H2[kMaxProblems];
    int ksplit[kMaxProblems], h_per_split[kMaxProblems], csplit[kMaxProblems];
    float scale[kMaxProblems];
    long long sbase[kMaxProblems + 1];  // shrink items of problem p: [sbase[p], sbase[p + 1])
    long long ebase[kMaxProblems + 1];  // expand items: [ebase[p], ebase[p + 1]), ebase[0] = sbase[num]
    int num;
};

template <typename DT, int R, int NT, int RB, int PG, int KB>
__global__ __launch_bounds__(NT) void lora_fused_multi_kernel(
    MultiProblems<typename DT::storage> P, const int* __restrict__ seg_indptr,
    const int* __restrict__ adapter_ids, int S, int num_rows, int num_adapters, int compact,
    int* flag, int counter_stride, long long wait_ticks) {
    const long long b = blockIdx.x;
    const bool shrink = b < P.sbase[P.num];
    const long long* base = shrink ? P.sbase : P.ebase;
    int p = 0;
    while (p + 1 < P.num && b >= base[p + 1]) ++p;
    const long long local = b - base[p];
    const int split = shrink ? P.ksplit[p] : P.csplit[p];
    fused_item<DT, R, NT, RB, PG, KB>(shrink, (int)(local / split), (int)(local % split), P.y[p],
                                      P.x[p], P.A[p], P.B[p], seg_indptr, adapter_ids, S,
                                      num_rows, num_adapters, P.H1[p], P.H2[p], P.scale[p],
                                      P.partials[p], P.counters[p], P.ksplit[p],
                                      P.h_per_split[p], P.csplit[p], compact, flag,
                                      counter_stride, wait_ticks);
}

}  // namespace sgmv
