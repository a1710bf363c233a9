// sgmv_gemv.hpp -- the decode-shaped (GEMV) SGMV kernels for gfx950.
//
// Shrink, v = x A (H1 -> r), is a segmented gather followed by a
// vector-matrix product: each segment fetches its adapter's A out of the
// stack (Punica walkthrough, omica.com.cn/news/959180, section 2.2, step 1).
// Expand, y += s v B (r -> H2), is the batched matrix-vector step over the
// stacked B matrices (same section, step 2).  Both are bound by HBM: each
// segment's weights are read exactly once per call and are the bulk of the
// bytes, so the kernels aim at wide, fully coalesced weight streams spread
// over every CU, with the short reductions done in registers and LDS.
//
// Work decomposition (integer only): a workgroup owns one (segment tile,
// H-chunk) pair.  The shrink splits the reduction over H1 into `ksplit`
// chunks and writes one float32 partial per chunk; the expand sums the
// partials in chunk order (so results are bit-reproducible) before its own
// reduction over r.
#pragma once

#include "sgmv_device.hpp"

namespace sgmv {

// Sum of P chunk partials p[0], p[stride], ..., in chunk order, with the
// loads issued in batches so that they are in flight together.
__device__ __forceinline__ float sum_partials(const float* __restrict__ p, long long stride, int P) {
    float sum = 0.f;
    for (int p0 = 0; p0 < P; p0 += 8) {
        float t[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) t[u] = (p0 + u < P) ? p[(long long)(p0 + u) * stride] : 0.f;
#pragma unroll
        for (int u = 0; u < 8; ++u)
            if (p0 + u < P) sum += t[u];
    }
    return sum;
}

// ---------------------------------------------------------------------------
// Wave reduce-scatter.  Each lane holds N floats; lanes whose ids differ only
// in the bits LPR, 2*LPR, ..., 32 hold partial sums of the same N quantities.
// Every step exchanges half of the remaining values with the partner lane
// (xor of one bit), so after log2(64/LPR) steps the group's sums are spread
// over its lanes with no value reduced twice.  `offset` returns the index (in
// 0..N) of the lane's first remaining value; `count` values remain (or one,
// replicated, once N is exhausted, in which case `canon` is false on the
// replicas).
// ---------------------------------------------------------------------------
template <int N, int n, int m>
__device__ __forceinline__ void rs_steps(float (&a)[N], int lane, int& offset, bool& canon) {
    if constexpr (m < kWave) {
        const bool up = (lane & m) != 0;
        if constexpr (n > 1) {
            constexpr int half = n / 2;
#pragma unroll
            for (int i = 0; i < half; ++i) {
                const float send = up ? a[i] : a[i + half];
                const float keep = up ? a[i + half] : a[i];
                a[i] = keep + __shfl_xor(send, m);
            }
            if (up) offset += half;
            rs_steps<N, half, m * 2>(a, lane, offset, canon);
        } else {
            a[0] += __shfl_xor(a[0], m);
            if (up) canon = false;
            rs_steps<N, 1, m * 2>(a, lane, offset, canon);
        }
    }
}

template <int N, int LPR>
struct ReduceScatter {
    static constexpr int steps() {
        int s = 0;
        for (int m = LPR; m < kWave; m <<= 1) ++s;
        return s;
    }
    static constexpr int kRemain = (N >> steps()) > 0 ? (N >> steps()) : 1;
    __device__ static __forceinline__ void run(float (&a)[N], int lane, int& offset,
                                               bool& canon) {
        offset = 0;
        canon = true;
        rs_steps<N, N, LPR>(a, lane, offset, canon);
    }
};

// ---------------------------------------------------------------------------
// Shrink, vectorised.  DT = element type, R = rank (compile time), NT =
// threads, RB = rows per tile, PG = 16-byte A loads issued per lane before
// they are consumed.
//
// The A chunk of a workgroup, rows [h_lo, h_hi) of A_stack[a], is contiguous
// (h_hi - h_lo) * R elements.  Thread t reads 16-byte vectors t, t + NT, ...
// of it, so every load instruction of a wave covers one contiguous KB; LPR =
// R / VEC lanes share one row h, and a lane always sees the same k-group.
// x is read as scalars (it is L1/L2-resident: all lanes of the workgroup
// touch the same RB rows).
//
// out[p * out_stride + row * R + k] receives the chunk-p partial sums.  With
// v_final (and zeroed tile counters), the tile's last workgroup also sums
// them into v_final[row * R + k], which spares a separate reduction launch.
// ---------------------------------------------------------------------------
template <typename DT, int R, int NT, int RB, int PG>
__global__ __launch_bounds__(NT) void shrink_vec_kernel(
    float* __restrict__ out, long long out_stride, const typename DT::storage* __restrict__ x,
    const typename DT::storage* __restrict__ A_stack, const int* __restrict__ seg_indptr,
    const int* __restrict__ adapter_ids, int S, int num_rows, int num_adapters, int H1,
    int ksplit, int h_per_split, float* __restrict__ v_final = nullptr,
    int* __restrict__ counters = nullptr, int counter_stride = 0) {
    using st = typename DT::storage;
    constexpr int VEC = DT::kVec;
    static_assert(R % VEC == 0, "rank must be a multiple of the vector width");
    constexpr int LPR = R / VEC;        // lanes per row of A
    static_assert(kWave % LPR == 0, "LPR must divide the wave");
    constexpr int HPB = NT / LPR;       // rows of A per block-wide pass
    constexpr int NW = NT / kWave;
    constexpr int N = RB * VEC;         // accumulators per lane
    using RS = ReduceScatter<N, LPR>;

    __shared__ int s_scan[tile_scan_ints<NT>()];
    __shared__ float s_red[NW][LPR * N];

    const int g = blockIdx.x / ksplit;
    const int p = blockIdx.x - g * ksplit;
    Tile tile;
    if (!locate_tile<NT>(seg_indptr, adapter_ids, S, num_rows, num_adapters, RB, g, s_scan, tile))
        return;

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wid = tid / kWave;
    const int h_lo = p * h_per_split;
    const int h_hi = min(H1, h_lo + h_per_split);
    const int nrows = tile.nrows;

    const st* A = A_stack + (long long)tile.adapter * H1 * R;
    const st* xr = x + (long long)tile.row0 * H1;

    float acc[N];
#pragma unroll
    for (int i = 0; i < N; ++i) acc[i] = 0.f;

    const int h_lane = tid / LPR;             // row offset of this lane within a pass
    const int k0 = (tid % LPR) * VEC;         // first column of this lane
    // With one-row tiles the x value is read together with the A pass (one
    // round trip for both, instead of x after A); taller tiles read theirs
    // as they are used, which keeps their registers down.  The FMA order is
    // the same either way.
    constexpr bool kEarlyX = RB == 1;
    for (int hb = h_lo; hb < h_hi; hb += HPB * PG) {
        uint4 av[PG];
        float x0[PG];
#pragma unroll
        for (int q = 0; q < PG; ++q) {
            const int h = hb + q * HPB + h_lane;
            const bool in = h < h_hi;
            av[q] = in ? load16(A + (long long)h * R + k0) : make_uint4(0, 0, 0, 0);
            x0[q] = (kEarlyX && in && nrows > 0) ? DT::load1(xr + h) : 0.f;
        }
#pragma unroll
        for (int q = 0; q < PG; ++q) {
            const int h = hb + q * HPB + h_lane;
            if (h < h_hi) {
                float af[VEC];
                DT::unpack(av[q], af);
#pragma unroll
                for (int i = 0; i < RB; ++i) {
                    if (i < nrows) {
                        const float x1 = (kEarlyX && i == 0) ? x0[q]
                                                             : DT::load1(xr + (long long)i * H1 + h);
#pragma unroll
                        for (int c = 0; c < VEC; ++c) acc[i * VEC + c] = fmaf(x1, af[c], acc[i * VEC + c]);
                    }
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
        for (int i = 0; i < RS::kRemain; ++i) s_red[wid][kq * N + offset + i] = acc[i];
    }
    __syncthreads();
    for (int t = tid; t < LPR * N; t += NT) {
        const int kq = t / N;
        const int idx = t - kq * N;
        const int i = idx / VEC;
        const int k = kq * VEC + (idx - i * VEC);
        float sum = 0.f;
#pragma unroll
        for (int w = 0; w < NW; ++w) sum += s_red[w][t];
        if (i < nrows) {
            float* dst = &out[(long long)p * out_stride + (long long)(tile.row0 + i) * R + k];
            if (v_final) __hip_atomic_store(dst, sum, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            else *dst = sum;
        }
    }
    if (!v_final) return;

    // In-kernel reduction: the last of the tile's ksplit workgroups to
    // arrive (told by its counter addition, so no workgroup waits) sums the
    // chunks' partials in chunk order, as reduce_partials_kernel would, and
    // writes v.  Partials are stored and read at agent scope (write-through,
    // no L2 write-back), each wave's stores acknowledged before the count;
    // the last arriver returns the counter to zero.
    __shared__ int s_last;
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (tid == 0) {
        int* cnt = &counters[(long long)g * counter_stride];
        const int before = __hip_atomic_fetch_add(cnt, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const bool last = before == ksplit - 1;
        if (last) __hip_atomic_store(cnt, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        s_last = last;
    }
    __syncthreads();
    if (!s_last) return;
    for (int t = tid; t < nrows * R; t += NT) {
        const int i = t / R;
        const int k = t - i * R;
        float* src = &out[(long long)(tile.row0 + i) * R + k];
        float sum = 0.f;
        for (int c0 = 0; c0 < ksplit; c0 += 8) {
            float pv[8];
#pragma unroll
            for (int u = 0; u < 8; ++u)
                pv[u] = c0 + u < ksplit ? __hip_atomic_load(src + (long long)(c0 + u) * out_stride,
                                                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                                        : 0.f;
#pragma unroll
            for (int u = 0; u < 8; ++u)
                if (c0 + u < ksplit) sum += pv[u];
        }
        v_final[(long long)(tile.row0 + i) * R + k] = sum;
    }
}

// ---------------------------------------------------------------------------
// Expand, vectorised.  One wave per workgroup; lane l owns VEC consecutive
// columns j of a CW = 64 * VEC column chunk.  The wave first sums the P
// float32 partials of v for its tile rows (in chunk order) into LDS, then
// walks r in blocks of KB rows of B (KB 16-byte loads in flight per lane),
// and finally updates y with one rounding per element.
// ---------------------------------------------------------------------------
template <typename DT, int R, int RB, int KB>
__global__ __launch_bounds__(kWave) void expand_vec_kernel(
    typename DT::storage* __restrict__ y, const float* __restrict__ vpart, long long v_stride,
    int P, const typename DT::storage* __restrict__ B_stack, const int* __restrict__ seg_indptr,
    const int* __restrict__ adapter_ids, int S, int num_rows, int num_adapters, int H2,
    float scale, int csplit) {
    using st = typename DT::storage;
    constexpr int VEC = DT::kVec;
    constexpr int CW = kWave * VEC;
    static_assert(R % KB == 0, "KB must divide the rank");

    __shared__ int s_scan[tile_scan_ints<kWave>()];
    __shared__ float s_v[RB][R];

    const int g = blockIdx.x / csplit;
    const int c = blockIdx.x - g * csplit;
    Tile tile;
    if (!locate_tile<kWave>(seg_indptr, adapter_ids, S, num_rows, num_adapters, RB, g, s_scan,
                            tile))
        return;

    const int lane = threadIdx.x;
    const int nrows = tile.nrows;
    const int j = c * CW + lane * VEC;
    const bool active = j < H2;
    const st* B = B_stack + (long long)tile.adapter * R * H2 + j;

    // First block of B: issue before waiting on v.
    uint4 bv[KB];
#pragma unroll
    for (int kk = 0; kk < KB; ++kk)
        bv[kk] = active ? load16(B + (long long)kk * H2) : make_uint4(0, 0, 0, 0);

    // v for the tile rows, partials summed in chunk order.
    for (int t = lane; t < RB * R; t += kWave) {
        const int i = t / R;
        const int k = t - i * R;
        float sum = 0.f;
        if (i < nrows) sum = sum_partials(vpart + (long long)(tile.row0 + i) * R + k, v_stride, P);
        s_v[i][k] = sum;
    }
    __syncthreads();

    float acc[RB][VEC];
#pragma unroll
    for (int i = 0; i < RB; ++i)
#pragma unroll
        for (int e = 0; e < VEC; ++e) acc[i][e] = 0.f;

#pragma unroll
    for (int kb = 0; kb < R; kb += KB) {
        if (kb > 0) {
#pragma unroll
            for (int kk = 0; kk < KB; ++kk)
                bv[kk] = active ? load16(B + (long long)(kb + kk) * H2) : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int kk = 0; kk < KB; ++kk) {
            float bf[VEC];
            DT::unpack(bv[kk], bf);
#pragma unroll
            for (int i = 0; i < RB; ++i) {
                if (i < nrows) {
                    const float vv = s_v[i][kb + kk];
#pragma unroll
                    for (int e = 0; e < VEC; ++e) acc[i][e] = fmaf(vv, bf[e], acc[i][e]);
                }
            }
        }
    }

    if (!active) return;
#pragma unroll
    for (int i = 0; i < RB; ++i) {
        if (i < nrows) {
            st* yp = y + (long long)(tile.row0 + i) * H2 + j;
            float yf[VEC];
            DT::unpack(load16(yp), yf);
#pragma unroll
            for (int e = 0; e < VEC; ++e) yf[e] = fmaf(scale, acc[i][e], yf[e]);
            store16(yp, DT::pack(yf));
        }
    }
}

// ---------------------------------------------------------------------------
// General kernels: any rank 1..128, any alignment, scalar element access.
// Same decomposition and the same chunked-partial contract as the
// vectorised kernels; used where those do not apply.
// ---------------------------------------------------------------------------
template <typename DT, int NT, int RB>
__global__ __launch_bounds__(NT) void shrink_generic_kernel(
    float* __restrict__ out, long long out_stride, const typename DT::storage* __restrict__ x,
    const typename DT::storage* __restrict__ A_stack, const int* __restrict__ seg_indptr,
    const int* __restrict__ adapter_ids, int S, int num_rows, int num_adapters, int H1, int r,
    int ksplit, int h_per_split) {
    using st = typename DT::storage;
    __shared__ int s_scan[tile_scan_ints<NT>()];
    __shared__ float s_red[NT * RB];

    const int g = blockIdx.x / ksplit;
    const int p = blockIdx.x - g * ksplit;
    Tile tile;
    if (!locate_tile<NT>(seg_indptr, adapter_ids, S, num_rows, num_adapters, RB, g, s_scan, tile))
        return;

    const int tid = threadIdx.x;
    const int G = NT / r;  // h groups (r <= 128 < NT)
    const int hg = tid / r;
    const int k = tid - hg * r;
    const int h_lo = p * h_per_split;
    const int h_hi = min(H1, h_lo + h_per_split);
    const st* A = A_stack + (long long)tile.adapter * H1 * r;
    const st* xr = x + (long long)tile.row0 * H1;

    float acc[RB];
#pragma unroll
    for (int i = 0; i < RB; ++i) acc[i] = 0.f;
    if (hg < G) {
        for (int h = h_lo + hg; h < h_hi; h += G) {
            const float av = DT::load1(A + (long long)h * r + k);
#pragma unroll
            for (int i = 0; i < RB; ++i)
                if (i < tile.nrows) acc[i] = fmaf(DT::load1(xr + (long long)i * H1 + h), av, acc[i]);
        }
    }
#pragma unroll
    for (int i = 0; i < RB; ++i) s_red[i * NT + tid] = acc[i];
    __syncthreads();
    for (int t = tid; t < RB * r; t += NT) {
        const int i = t / r;
        const int kk = t - i * r;
        float sum = 0.f;
        for (int q = 0; q < G; ++q) sum += s_red[i * NT + q * r + kk];
        if (i < tile.nrows)
            out[(long long)p * out_stride + (long long)(tile.row0 + i) * r + kk] = sum;
    }
}

template <typename DT, int NT, int RB>
__global__ __launch_bounds__(NT) void expand_generic_kernel(
    typename DT::storage* __restrict__ y, const float* __restrict__ vpart, long long v_stride,
    int P, const typename DT::storage* __restrict__ B_stack, const int* __restrict__ seg_indptr,
    const int* __restrict__ adapter_ids, int S, int num_rows, int num_adapters, int r, int H2,
    float scale, int csplit) {
    using st = typename DT::storage;
    __shared__ int s_scan[tile_scan_ints<NT>()];
    __shared__ float s_v[RB * 128];

    const int g = blockIdx.x / csplit;
    const int c = blockIdx.x - g * csplit;
    Tile tile;
    if (!locate_tile<NT>(seg_indptr, adapter_ids, S, num_rows, num_adapters, RB, g, s_scan, tile))
        return;

    const int tid = threadIdx.x;
    for (int t = tid; t < RB * r; t += NT) {
        const int i = t / r;
        const int k = t - i * r;
        float sum = 0.f;
        if (i < tile.nrows) sum = sum_partials(vpart + (long long)(tile.row0 + i) * r + k, v_stride, P);
        s_v[t] = sum;
    }
    __syncthreads();
    const int j = c * NT + tid;
    if (j >= H2) return;
    const st* B = B_stack + (long long)tile.adapter * r * H2 + j;
    float acc[RB];
#pragma unroll
    for (int i = 0; i < RB; ++i) acc[i] = 0.f;
    for (int k = 0; k < r; ++k) {
        const float bv = DT::load1(B + (long long)k * H2);
#pragma unroll
        for (int i = 0; i < RB; ++i) acc[i] = fmaf(s_v[i * r + k], bv, acc[i]);
    }
#pragma unroll
    for (int i = 0; i < RB; ++i) {
        if (i < tile.nrows) {
            st* yp = y + (long long)(tile.row0 + i) * H2 + j;
            *yp = DT::from_float(fmaf(scale, acc[i], DT::load1(yp)));
        }
    }
}

// ---------------------------------------------------------------------------
// Sum of the P chunk partials into v, for covered rows only (sgmv_shrink
// when the reduction over H1 was split).  One thread per (row, k); a row is
// covered when the segment found by binary search over seg_indptr contains
// it and names a valid adapter.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void reduce_partials_kernel(
    float* __restrict__ v, const float* __restrict__ vpart, long long v_stride, int P,
    const int* __restrict__ seg_indptr, const int* __restrict__ adapter_ids, int S, int num_rows,
    int num_adapters, int r) {
    const long long e = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    if (e >= (long long)num_rows * r) return;
    const int row = (int)(e / r);
    // last segment whose start is <= row
    int lo = 0, hi = S;  // answer in [0, S)
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (seg_indptr[mid] <= row) lo = mid; else hi = mid;
    }
    const SegBounds b = seg_bounds(seg_indptr, adapter_ids, lo, num_rows, num_adapters);
    if (!b.ok || row < b.lo || row >= b.hi) return;
    v[e] = sum_partials(vpart + e, v_stride, P);
}

}  // namespace sgmv
