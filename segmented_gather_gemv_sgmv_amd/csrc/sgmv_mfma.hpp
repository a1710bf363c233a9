// sgmv_mfma.hpp -- lora_apply for segments of many rows (prefill shapes):
// 16-row tiles whose two contractions run on the gfx950 matrix cores.
//
// Per tile of up to 16 rows of one segment (adapter a), the shrink
// V = X A_a  ([16 x H1] x [H1 x r]) and the expand Y += s V B_a
// ([16 x r] x [r x H2]) are dense contractions once several rows share an
// adapter, so they use v_mfma_f32_16x16x32_{f16,bf16} with float32
// accumulation (the two SGMV steps of Punica walkthrough,
// omica.com.cn/news/959180, section 2.2).  The work is still bound by HBM
// (x is read once and y read and written once), so the kernel keeps the
// single-launch hand-off of sgmv_fused.hpp: shrink items (tile, H1 chunk)
// publish float32 chunk partials, expand items (tile, column chunk) wait for
// them, and the per-tile counters reset themselves.
//
// Operand layouts of the 16x16x32 MFMA (checked on the device): lane l holds
// A[l % 16][8 (l / 16) + j] and B[8 (l / 16) + j][l % 16], j = 0..7, and
// receives D[4 (l / 16) + i][l % 16], i = 0..3.
//
// Shrink: X is the A operand, loaded straight from global memory (8
// consecutive h of one row = 16 bytes).  A_a is stored [h][r] (r fastest),
// so the B operand (8 consecutive h of one column) is read from an LDS copy
// of the chunk with transposing LDS reads.  The four waves split the
// chunk's h range and their 16 x r results are summed in LDS in a fixed
// order.
//
// Expand: computed as Y^T = B^T V^T so that each lane's result is 4
// consecutive columns of one row (one 8-byte y access).  B^T is read from
// an LDS copy of the B chunk with transposing LDS reads.  V is float32; to
// feed it to a 16-bit MFMA without losing precision it is split as
// v = hi + mid + lo (each 16-bit, each the rounded remainder of the last)
// and the K dimension is [hi | mid | lo | 0] against [B ; B ; B ; B],
// padded to whole MFMA steps of 32.  Three bf16 terms hold 24 significant
// bits, all of a float32 v; three fp16 terms hold more.  For fp16 the
// tile's v is first scaled by a power of two so that max |v| lies in
// [2^12, 2^13) (exact, undone on the result), keeping hi inside the fp16
// range.
#pragma once

#include "sgmv_device.hpp"
#include "sgmv_fused.hpp"

namespace sgmv {

typedef float mf32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 mf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 mbf16x8 __attribute__((ext_vector_type(8)));

template <typename DT>
struct MfmaOps;

template <>
struct MfmaOps<F16> {
    static constexpr bool kScaleV = true;  // keep v inside the fp16 range
    __device__ static __forceinline__ mf32x4 mma(const uint4& a, const uint4& b, mf32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(mf16x8, a),
                                                      __builtin_bit_cast(mf16x8, b), c, 0, 0, 0);
    }
    __device__ static __forceinline__ uint32_t bits(float f) { return F16::f2h(f); }
    __device__ static __forceinline__ float value(uint32_t b) { return F16::h2f(b); }
};

template <>
struct MfmaOps<BF16> {
    static constexpr bool kScaleV = false;  // bf16 has float32's exponent range
    __device__ static __forceinline__ mf32x4 mma(const uint4& a, const uint4& b, mf32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(mbf16x8, a),
                                                       __builtin_bit_cast(mbf16x8, b), c, 0, 0, 0);
    }
    __device__ static __forceinline__ uint32_t bits(float f) { return BF16::f2b(f); }
    __device__ static __forceinline__ float value(uint32_t b) { return BF16::b2f(b); }
};

__device__ __forceinline__ uint2 load8(const void* p) { return *reinterpret_cast<const uint2*>(p); }
__device__ __forceinline__ void store8(void* p, const uint2& v) { *reinterpret_cast<uint2*>(p) = v; }

// One MFMA operand (8 consecutive K of one row or column) gathered from a
// tile in LDS whose rows run along the other index, with two transposing
// LDS reads (ds_read_b64_tr_b16).  Within each group of 16 lanes, that
// instruction gives lane i element i % 4 of the 8-byte pieces addressed by
// lanes i / 4, 4 + i / 4, 8 + i / 4 and 12 + i / 4 of the group (checked on
// the device).  So if lane (grp, m) of the wave passes, for its group, the
// rows k0 .. k0 + 7 of the tile (k0 uniform over the group) as
//     row(c) = base + (k0 + m / 4 + 4 c) * ld + 4 (m % 4),  c = 0, 1,
// it receives tile[k0 + j][m] for j = 0..7, i.e. the 16 columns starting at
// `base` become the operand's 16 lanes.  base and ld must keep every row
// piece 8-byte aligned.
__device__ __forceinline__ uint4 lds_operand_tr(const uint16_t* base, int k0, int ld, int m) {
#if __HIP_DEVICE_COMPILE__
    typedef short v4s __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(3))) v4s lds_v4s;
    typedef __attribute__((address_space(3))) short lds_short;
    const uint16_t* p0 = base + (k0 + (m >> 2)) * ld + 4 * (m & 3);
    const uint16_t* p1 = p0 + 4 * ld;
    const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(lds_short*)(p0));
    const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(lds_short*)(p1));
    const uint2 a = __builtin_bit_cast(uint2, lo);
    const uint2 b = __builtin_bit_cast(uint2, hi);
    return make_uint4(a.x, a.y, b.x, b.y);
#else
    (void)base; (void)k0; (void)ld; (void)m;
    return make_uint4(0, 0, 0, 0);
#endif
}


template <int R, int KC = 16384 / R>
struct MfmaShape {
    static constexpr int kT = 16;                        // rows per tile
    static constexpr int kNT = 256;                      // threads per workgroup
    static constexpr int kNW = kNT / kWave;              // waves
    static constexpr int kKcMax = KC;                    // rows of A per LDS chunk (default 32 KB)
    static_assert(KC % (32 * kNW) == 0, "a chunk is whole K steps of every wave");
    static constexpr int kXSteps = kKcMax / (32 * kNW);  // K steps of 32 per wave and chunk
    // Expand columns per item.  Up to rank 32 the item's whole B chunk
    // (R x kCW) sits in LDS at once; from rank 64 it passes through LDS in
    // slices of kKS = 32 ranks, the next slice loading into registers while
    // the current one is multiplied, so the item keeps 256 columns (a
    // slice then takes the LDS the tile's A chunk takes).
    static constexpr int kCW = R >= 64 ? 256 : ((8192 / R) < 512 ? (8192 / R) : 512);
    static constexpr int kKS = R >= 64 ? 32 : R;         // ranks of B per LDS stage
    static constexpr int kSlices = R / kKS;
    static constexpr int kCBW = kCW / (16 * kNW);        // 16-column blocks per wave
    static constexpr int kBV = kKS * kCW / 8 / kNT;      // 16-byte B vectors per thread and slice
    // Epilogue: y is read and written in row-contiguous 16-byte pieces (kYU
    // pieces of 8 columns per thread; a wave covers 512 columns of a row),
    // and the 16 x kCW tile of y passes through LDS (over the B chunk, which
    // is at least as large) to meet the MFMA result layout.  In LDS, the
    // 8-byte group g of row i sits at position g ^ (i & 15), so that neither
    // the row-piece accesses nor the MFMA-layout ones meet bank conflicts.
    static constexpr int kYU = (2 * kCW + kNT - 1) / kNT;
    // A B slice in LDS: kKS rows of kCW columns, each row padded by 16
    // elements so that the four rows one transposing read touches fall in
    // different banks.
    static constexpr int kLdB = kCW + 16;
    static constexpr int kStageB = kKS * kLdB;  // LDS of a B slice, in 16-bit units
    // K of the expand's v operand: three 16-bit terms of each v, padded to
    // whole MFMA steps of 32 (16-bit units per tile row of s_vh).
    static constexpr int kVK = (3 * R + 31) / 32 * 32;
    static_assert(kStageB >= kT * kCW, "the y tile must fit over the B chunk");
    static_assert(kCW % 64 == 0, "the swizzle needs at least 16 groups per row");
    static_assert(kBV * kNT * 8 == kKS * kCW, "a B slice must split evenly over the threads");
    static_assert(kSlices == 1 || 3 * R == kVK, "sliced ranks need no K padding");
    static_assert(R % 16 == 0 && R <= 128, "MFMA path needs r in {16, 32, 64, 128}");
};

// One H1 chunk [h_lo, h_hi) of the shrink for a tile of nrows <= 16 rows,
// reduced across the workgroup; calls emit(i, k, value) once per (i < nrows,
// k < R) from threads tid < 16 * R.  h_lo and h_hi are multiples of 8 and
// h_hi - h_lo <= KC (rows of A per LDS chunk).  Begins and ends with the
// block synchronised.
// kRedOverA: s_red occupies the same LDS as s_a (the workgroup then waits
// for every wave's last read of the A chunk before the sums are written).
template <typename DT, int R, bool kRedOverA = false, int KC = 16384 / R, typename Emit>
__device__ __forceinline__ void shrink_chunk_mfma(const typename DT::storage* __restrict__ A,
                                                  const typename DT::storage* __restrict__ xr,
                                                  int nrows, int H1, int h_lo, int h_hi,
                                                  uint16_t* s_a, float* s_red, Emit&& emit) {
    using Sh = MfmaShape<R, KC>;
    using Ops = MfmaOps<DT>;
    constexpr int NB = R / 16;
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wid = tid / kWave;
    const int m = lane & 15;   // operand row (A) / column (B) of this lane
    const int grp = lane >> 4; // which 8 of the 32 K values
    const int kc = h_hi - h_lo;
    const int kq = (kc + 32 * Sh::kNW - 1) / (32 * Sh::kNW) * 32;  // h rows per wave

    // x operand for all of this wave's K steps, issued before anything waits.
    uint4 xa[Sh::kXSteps];
#pragma unroll
    for (int s = 0; s < Sh::kXSteps; ++s) {
        const int hl = wid * kq + s * 32 + grp * 8;
        xa[s] = (s * 32 < kq && hl < kc && m < nrows)
                    ? load16(xr + (long long)m * H1 + h_lo + hl)
                    : make_uint4(0, 0, 0, 0);
    }
    // The chunk of A, as stored ([h][r]), into LDS: every load in flight
    // before the first LDS store.
    const typename DT::storage* Ac = A + (long long)h_lo * R;
    constexpr int kAV = Sh::kKcMax * R / 8 / Sh::kNT;  // 16-byte pieces per thread
    static_assert(kAV * Sh::kNT * 8 == Sh::kKcMax * R, "A chunk must split evenly");
    uint4 av[kAV];
#pragma unroll
    for (int u = 0; u < kAV; ++u) {
        const int t = tid + u * Sh::kNT;
        av[u] = t < kc * R / 8 ? load16(Ac + (long long)t * 8) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < kAV; ++u) {
        const int t = tid + u * Sh::kNT;
        if (t < kc * R / 8) store16(s_a + t * 8, av[u]);
    }
    __syncthreads();

    mf32x4 acc[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) acc[nb] = mf32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < Sh::kXSteps; ++s) {
        const int hl = wid * kq + s * 32 + grp * 8;
        if (s * 32 < kq) {  // wave-uniform
            // Rows hl .. hl + 7 of the chunk are all inside it or all past it
            // (both are multiples of 8); past it, LDS holds no data of this
            // chunk, so the operand is zeroed.
            const bool in = hl < kc;
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                uint4 hb = lds_operand_tr(s_a + nb * 16, hl, R, m);
                if (!in) hb = make_uint4(0, 0, 0, 0);
                acc[nb] = Ops::mma(xa[s], hb, acc[nb]);
            }
        }
    }
    // Cross-wave sum in a fixed order.
    if constexpr (kRedOverA) __syncthreads();
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int i = 0; i < 4; ++i) s_red[(wid * 16 + 4 * grp + i) * R + nb * 16 + m] = acc[nb][i];
    __syncthreads();
    for (int t = tid; t < 16 * R; t += Sh::kNT) {
        const int i = t / R;
        const int k = t - i * R;
        float sum = 0.f;
#pragma unroll
        for (int w = 0; w < Sh::kNW; ++w) sum += s_red[(w * 16 + i) * R + k];
        if (i < nrows) emit(i, k, sum);
    }
    __syncthreads();  // s_a and s_red free again
}

// The shrink of [h_lo, h_hi) (multiples of 8, longer than one LDS chunk)
// for a tile of nrows <= 16 rows.  A chain of shrink_chunk_mfma calls
// would wait for each chunk's x before requesting the next; here the x
// operand of a whole stretch of chunks (8 K steps of 32 per wave, 4 at
// r >= 64, where the A chunks and accumulators need the registers) is
// requested before any of it is used, the next chunk of A is requested
// while the current one is multiplied, and each wave's products stay in
// its MFMA accumulators across chunks (in chunk order).  The four waves'
// sums are added in wave order at the end; emit(i, k, value) is called
// once per (i < nrows, k < R) from threads tid < 16 * R.  Begins and ends
// with the block synchronised; s_red may overlap s_a.
template <typename DT, int R, int KC, typename Emit>
__device__ __forceinline__ void shrink_long_mfma(const typename DT::storage* __restrict__ A,
                                                 const typename DT::storage* __restrict__ xr,
                                                 int nrows, int H1, int h_lo, int h_hi,
                                                 uint16_t* s_a, float* s_red, Emit&& emit) {
    using Sh = MfmaShape<R, KC>;
    using Ops = MfmaOps<DT>;
    constexpr int NB = R / 16;
    constexpr int XS = Sh::kXSteps;            // K steps of 32 per wave and chunk
    constexpr int kStretch = R >= 64 ? 4 : 8;  // K steps of x per wave requested together
    constexpr int CPS = XS >= kStretch ? 1 : kStretch / XS;  // chunks per stretch
    constexpr int KQ = KC / Sh::kNW;           // h of a chunk per wave
    constexpr int kAV = KC * R / 8 / Sh::kNT;  // 16-byte pieces of an A chunk per thread
    static_assert(kAV * Sh::kNT * 8 == KC * R, "A chunk must split evenly");
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wid = tid / kWave;
    const int m = lane & 15;
    const int grp = lane >> 4;
    const bool row_ok = m < nrows;
    const typename DT::storage* xm = xr + (long long)m * H1;

    mf32x4 acc[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) acc[nb] = mf32x4{0.f, 0.f, 0.f, 0.f};
    uint4 av[kAV];
    auto load_a = [&](int c_lo) {
        const int n16 = min(KC, h_hi - c_lo) * R / 8;
        const typename DT::storage* Ac = A + (long long)c_lo * R;
#pragma unroll
        for (int u = 0; u < kAV; ++u) {
            const int t = tid + u * Sh::kNT;
            av[u] = t < n16 ? load16(Ac + (long long)t * 8) : make_uint4(0, 0, 0, 0);
        }
    };
    load_a(h_lo);
    for (int s_lo = h_lo; s_lo < h_hi; s_lo += CPS * KC) {
        uint4 xa[CPS][XS];
#pragma unroll
        for (int j = 0; j < CPS; ++j)
#pragma unroll
            for (int s = 0; s < XS; ++s) {
                const int h = s_lo + j * KC + wid * KQ + s * 32 + grp * 8;
                xa[j][s] = (h < h_hi && row_ok) ? load16(xm + h) : make_uint4(0, 0, 0, 0);
            }
#pragma unroll
        for (int j = 0; j < CPS; ++j) {
            const int c_lo = s_lo + j * KC;
            if (c_lo < h_hi) {  // block-uniform
                const int kc = min(KC, h_hi - c_lo);
                __syncthreads();  // every wave is done with the previous chunk
#pragma unroll
                for (int u = 0; u < kAV; ++u) {
                    const int t = tid + u * Sh::kNT;
                    if (t < kc * R / 8) store16(s_a + t * 8, av[u]);
                }
                if (c_lo + KC < h_hi) load_a(c_lo + KC);
                __syncthreads();
#pragma unroll
                for (int s = 0; s < XS; ++s) {
                    // Rows hl .. hl + 7 of the chunk are all inside it or
                    // all past it; past it, LDS holds no data of this chunk.
                    const int hl = wid * KQ + s * 32 + grp * 8;
                    const bool in = hl < kc;
#pragma unroll
                    for (int nb = 0; nb < NB; ++nb) {
                        uint4 hb = lds_operand_tr(s_a + nb * 16, hl, R, m);
                        if (!in) hb = make_uint4(0, 0, 0, 0);
                        acc[nb] = Ops::mma(xa[j][s], hb, acc[nb]);
                    }
                }
            }
        }
    }
    __syncthreads();  // s_red lies over s_a
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int i = 0; i < 4; ++i) s_red[(wid * 16 + 4 * grp + i) * R + nb * 16 + m] = acc[nb][i];
    __syncthreads();
    for (int t = tid; t < 16 * R; t += Sh::kNT) {
        const int i = t / R;
        const int k = t - i * R;
        float sum = 0.f;
#pragma unroll
        for (int w = 0; w < Sh::kNW; ++w) sum += s_red[(w * 16 + i) * R + k];
        if (i < nrows) emit(i, k, sum);
    }
    __syncthreads();  // s_a and s_red free again
}

// The part of an expand item (tile rows x columns [c0, c0 + kCW)) that does
// not depend on v, loaded first: this thread's 16-byte pieces of the first
// B slice and the y values its lane updates.
template <int R>
struct ExpandRegs {
    uint4 bq[MfmaShape<R>::kBV];
    uint4 yv[MfmaShape<R>::kYU];  // piece u: row u / (kCW / 8), columns 8 (u % (kCW / 8)) + [0, 8)
};

// This thread's pieces of B slice sl (ranks sl * kKS + [0, kKS)).
template <typename DT, int R>
__device__ __forceinline__ void expand_load_slice(uint4 (&bq)[MfmaShape<R>::kBV],
                                                  const typename DT::storage* __restrict__ B,
                                                  int sl, int H2, int c0) {
    using Sh = MfmaShape<R>;
    constexpr int CW = Sh::kCW;
    const int tid = threadIdx.x;
#pragma unroll
    for (int u = 0; u < Sh::kBV; ++u) {
        const int t = tid + u * Sh::kNT;
        const int kr = sl * Sh::kKS + t / (CW / 8);
        const int c8 = (t % (CW / 8)) * 8;
        bq[u] = (c0 + c8 < H2) ? load16(B + (long long)kr * H2 + c0 + c8)
                               : make_uint4(0, 0, 0, 0);
    }
}

template <typename DT, int R>
__device__ __forceinline__ void expand_prefetch(ExpandRegs<R>& e,
                                                const typename DT::storage* __restrict__ B,
                                                const typename DT::storage* __restrict__ yr,
                                                int nrows, int H2, int c0) {
    using Sh = MfmaShape<R>;
    constexpr int CW = Sh::kCW;
    const int tid = threadIdx.x;
    expand_load_slice<DT, R>(e.bq, B, 0, H2, c0);
#pragma unroll
    for (int j = 0; j < Sh::kYU; ++j) {
        const int u = tid + j * Sh::kNT;
        const int row = u / (CW / 8);
        const int col = c0 + (u % (CW / 8)) * 8;
        e.yv[j] = (u < 2 * CW && row < nrows && col < H2)
                      ? load16_stream(yr + (long long)row * H2 + col)
                      : make_uint4(0, 0, 0, 0);
    }
}

// Finishes an expand item once s_v (16 x R floats, rows >= nrows zero) is
// complete and visible to the block: y[rows, c0 : c0 + kCW] += scale * V B.
// The B chunk goes to LDS (s_b, kStageB 16-bit units), v is split into
// three 16-bit terms (s_vh, 16 x kVK, range-scaled for fp16), Y^T = B^T V^T
// runs on the MFMA units, and the results return through s_b so that y
// moves in row-contiguous pieces.
template <typename DT, int R>
__device__ __forceinline__ void expand_apply(const ExpandRegs<R>& e, uint16_t* s_b,
                                             const float* s_v, uint16_t* s_vh, float* s_max,
                                             typename DT::storage* __restrict__ yr, int nrows,
                                             int H2, int c0, float scale,
                                             const typename DT::storage* __restrict__ B) {
    using Sh = MfmaShape<R>;
    using Ops = MfmaOps<DT>;
    constexpr int T = Sh::kT;
    constexpr int NT = Sh::kNT;
    constexpr int CW = Sh::kCW;
    constexpr int CBW = Sh::kCBW;
    constexpr int NS = Sh::kSlices;
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wid = tid / kWave;
    const int m = lane & 15;
    const int grp = lane >> 4;
    uint4 bq[Sh::kBV];
#pragma unroll
    for (int u = 0; u < Sh::kBV; ++u) bq[u] = e.bq[u];
    auto stage = [&]() {  // this thread's pieces of the slice in bq -> s_b
#pragma unroll
        for (int u = 0; u < Sh::kBV; ++u) {
            const int t = tid + u * NT;
            store16(s_b + (t / (CW / 8)) * Sh::kLdB + (t % (CW / 8)) * 8, bq[u]);
        }
    };
    stage();
    // The largest |v| of the tile for the fp16 range scaling.
    int shift = 0;
    if constexpr (Ops::kScaleV) {
        float mx = 0.f;
        for (int t = tid; t < T * R; t += NT) mx = fmaxf(mx, fabsf(s_v[t]));
#pragma unroll
        for (int d = 32; d > 0; d >>= 1) mx = fmaxf(mx, __shfl_xor(mx, d));
        if (lane == 0) s_max[wid] = mx;
        __syncthreads();
        mx = fmaxf(fmaxf(s_max[0], s_max[1]), fmaxf(s_max[2], s_max[3]));
        if (mx > 0.f && mx <= 3.0e38f) {
            int ex;
            frexpf(mx, &ex);  // mx = f * 2^ex, f in [0.5, 1)
            shift = min(max(13 - ex, -100), 100);
        }
    }
    constexpr int VK = Sh::kVK;
    for (int t = tid; t < T * R; t += NT) {
        const int i = t / R;
        const int k = t - i * R;
        const float v = ldexpf(s_v[t], shift);
        const uint32_t hi = Ops::bits(v);
        const float r1 = v - Ops::value(hi);
        const uint32_t mid = Ops::bits(r1);
        const uint32_t lo = Ops::bits(r1 - Ops::value(mid));
        s_vh[i * VK + k] = (uint16_t)hi;
        s_vh[i * VK + R + k] = (uint16_t)mid;
        s_vh[i * VK + 2 * R + k] = (uint16_t)lo;
    }
    if constexpr (VK > 3 * R) {  // the padding of the K dimension meets zeros
        for (int t = tid; t < T * (VK - 3 * R); t += NT) {
            const int i = t / (VK - 3 * R);
            s_vh[i * VK + 3 * R + (t - i * (VK - 3 * R))] = 0;
        }
    }
    __syncthreads();

    const float out_scale = ldexpf(scale, -shift);
    mf32x4 acc[CBW];
#pragma unroll
    for (int q = 0; q < CBW; ++q) acc[q] = mf32x4{0.f, 0.f, 0.f, 0.f};
    if constexpr (NS == 1) {
#pragma unroll
        for (int q = 0; q < CBW; ++q) {
            const int cb = wid * CBW + q;
#pragma unroll
            for (int ks = 0; ks < VK / 32; ++ks) {
                // B rows kr .. kr + 7 (every term of v meets B row kr), columns
                // cb * 16 + [0, 16).
                const int kr = (ks * 32 + grp * 8) % R;
                const uint4 ab = lds_operand_tr(s_b + cb * 16, kr, Sh::kLdB, m);
                const uint4 bv =
                    *reinterpret_cast<const uint4*>(s_vh + m * VK + ks * 32 + grp * 8);
                acc[q] = Ops::mma(ab, bv, acc[q]);
            }
        }
    } else {
        // Slice sl holds B rows sl * 32 + [0, 32); each of the three terms
        // of v meets them in one K step.  The next slice is in flight while
        // this one is multiplied.
        expand_load_slice<DT, R>(bq, B, 1, H2, c0);
        for (int sl = 0; sl < NS; ++sl) {
            if (sl > 0) {
                __syncthreads();  // every wave is done with slice sl - 1
                stage();
                __syncthreads();
                if (sl + 1 < NS) expand_load_slice<DT, R>(bq, B, sl + 1, H2, c0);
            }
#pragma unroll
            for (int q = 0; q < CBW; ++q) {
                const int cb = wid * CBW + q;
                const uint4 ab = lds_operand_tr(s_b + cb * 16, grp * 8, Sh::kLdB, m);
#pragma unroll
                for (int term = 0; term < 3; ++term) {
                    const uint4 bv = *reinterpret_cast<const uint4*>(
                        s_vh + m * VK + term * R + sl * Sh::kKS + grp * 8);
                    acc[q] = Ops::mma(ab, bv, acc[q]);
                }
            }
        }
    }
    // The y tile, as loaded (row pieces), into LDS over the B chunk: every
    // wave is done with B once the barrier is passed.
    __syncthreads();
    uint2* s_y = reinterpret_cast<uint2*>(s_b);  // [16][kCW / 4] groups of 4 columns
    constexpr int G = CW / 4;                    // 8-byte groups per row
#pragma unroll
    for (int j = 0; j < Sh::kYU; ++j) {
        const int u = tid + j * NT;
        const int row = u / (CW / 8);
        const int g = (u % (CW / 8)) * 2;
        if (u < 2 * CW) {
            s_y[row * G + (g ^ row)] = make_uint2(e.yv[j].x, e.yv[j].y);
            s_y[row * G + ((g + 1) ^ row)] = make_uint2(e.yv[j].z, e.yv[j].w);
        }
    }
    __syncthreads();
    // Lane (m, grp) owns columns cb * 16 + 4 grp + [0, 4) of row m: one group.
#pragma unroll
    for (int q = 0; q < CBW; ++q) {
        const int g = (wid * CBW + q) * 4 + grp;
        uint2* slot = &s_y[m * G + (g ^ m)];
        const uint2 old = *slot;
        float yf[4];
        DT::unpack2(old.x, yf);
        DT::unpack2(old.y, yf + 2);
#pragma unroll
        for (int i = 0; i < 4; ++i) yf[i] = fmaf(out_scale, acc[q][i], yf[i]);
        *slot = make_uint2(DT::pack2(yf[0], yf[1]), DT::pack2(yf[2], yf[3]));
    }
    __syncthreads();
    // The updated tile back to y, row pieces of 8 columns.
#pragma unroll
    for (int j = 0; j < Sh::kYU; ++j) {
        const int u = tid + j * NT;
        const int row = u / (CW / 8);
        const int g = (u % (CW / 8)) * 2;
        if (u < 2 * CW && row < nrows && c0 + g * 4 < H2) {
            const uint2 a0 = s_y[row * G + (g ^ row)];
            const uint2 a1 = s_y[row * G + ((g + 1) ^ row)];
            store16_stream(yr + (long long)row * H2 + c0 + g * 4,
                           make_uint4(a0.x, a0.y, a1.x, a1.y));
        }
    }
}

template <typename DT, int R>
__global__ __launch_bounds__(256) void lora_mfma_kernel(
    typename DT::storage* __restrict__ y, const typename DT::storage* __restrict__ x,
    const typename DT::storage* __restrict__ A_stack,
    const typename DT::storage* __restrict__ B_stack, const int* __restrict__ seg_indptr,
    const int* __restrict__ adapter_ids, int S, int num_rows, int num_adapters, int H1, int H2,
    float scale, float* __restrict__ partials, int* __restrict__ counters, int ksplit,
    int h_per_split, int csplit, int slots_a, int slots_b, int compact, int n_counters,
    int counter_stride, long long wait_ticks) {
    using st = typename DT::storage;
    using Sh = MfmaShape<R>;
    constexpr int T = Sh::kT;
    constexpr int NT = Sh::kNT;
    constexpr int NW = Sh::kNW;
    constexpr int CW = Sh::kCW;

    __shared__ int s_scan[tile_scan_ints<NT>()];
    // A chunk; later the B chunk [R][CW] and then the expand results
    __shared__ __align__(16) uint16_t s_a[Sh::kKcMax * R > Sh::kStageB ? Sh::kKcMax * R
                                                                       : Sh::kStageB];
    __shared__ float s_red[NW * 16 * R];
    __shared__ float s_v[T * R];
    __shared__ __align__(16) uint16_t s_vh[T * Sh::kVK];  // per row: hi, mid, lo terms of v
    __shared__ float s_max[NW];
    __shared__ int s_flag;

    const int tid = threadIdx.x;
    const long long row_stride = (long long)num_rows * R;
    const int total = ksplit + (csplit << 16);
    const Item it = decode_item(slots_a, slots_b, ksplit, csplit);
    Tile tile;
    const bool have =
        compact ? locate_tile_compact<NT>(seg_indptr, adapter_ids, S, num_rows, num_adapters, T,
                                          it.g, s_scan, tile)
                : locate_tile<NT>(seg_indptr, adapter_ids, S, num_rows, num_adapters, T, it.g,
                                  s_scan, tile);
    if (!have) return;
    const int nrows = tile.nrows;
    const st* A = A_stack + (long long)tile.adapter * H1 * R;
    const st* xr = x + (long long)tile.row0 * H1;
    int* cnt = &counters[it.g * counter_stride];

    if (it.shrink) {
        const int h_lo = it.sub * h_per_split;
        const int h_hi = min(H1, h_lo + h_per_split);
        float* out = partials + (long long)it.sub * row_stride + (long long)tile.row0 * R;
        shrink_chunk_mfma<DT, R>(A, xr, nrows, H1, h_lo, h_hi, s_a, s_red,
                                 [&](int i, int k, float v) { store_partial(&out[i * R + k], v); });
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        __builtin_amdgcn_s_waitcnt(0);  // this wave's partial stores are acknowledged
        __syncthreads();
        if (tid == 0) depart(cnt, 1, total);
        return;
    }

    // ---------------- expand item ----------------
    const int c0 = it.sub * CW;
    ExpandRegs<R> er;
    expand_prefetch<DT, R>(er, B_stack + (long long)tile.adapter * R * H2,
                           y + (long long)tile.row0 * H2, nrows, H2, c0);
    if (tid == 0) s_flag = wait_for_producers(cnt, ksplit, wait_ticks);
    __syncthreads();
    if (s_flag) {
        for (int t = tid; t < T * R; t += NT) {
            const int i = t / R;
            const int k = t - i * R;
            s_v[t] = i < nrows ? sum_partials_coherent(
                                     partials + (long long)(tile.row0 + i) * R + k, row_stride,
                                     ksplit)
                               : 0.f;
        }
    } else {
        // The producers are late: compute every chunk here, summing in the
        // same order as the normal path.
        if (tid == 0)
            __hip_atomic_store(&counters[n_counters - 1], 1, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
        for (int t = tid; t < T * R; t += NT) s_v[t] = 0.f;
        __syncthreads();
        for (int pp = 0; pp < ksplit; ++pp) {
            const int h_lo = pp * h_per_split;
            const int h_hi = min(H1, h_lo + h_per_split);
            shrink_chunk_mfma<DT, R>(A, xr, nrows, H1, h_lo, h_hi, s_a, s_red,
                                     [&](int i, int k, float v) { s_v[i * R + k] += v; });
        }
        // Load B and y again, so that the prefetched registers are not held
        // across this rarely taken path.
        expand_prefetch<DT, R>(er, B_stack + (long long)tile.adapter * R * H2,
                               y + (long long)tile.row0 * H2, nrows, H2, c0);
    }
    __syncthreads();
    // The partials are in LDS now: count out, and reset after the compute.
    int before = 0;
    if (tid == 0) before = depart_begin(cnt, 1 << 16);
    expand_apply<DT, R>(er, s_a, s_v, s_vh, s_max, y + (long long)tile.row0 * H2, nrows, H2, c0,
                        scale, B_stack + (long long)tile.adapter * R * H2);
    if (tid == 0) depart_end(cnt, before, 1 << 16, total);
}

// ---------------------------------------------------------------------------
// The same computation as two launches, for calls large enough that the
// second launch costs little next to the data: every shrink workgroup (tile,
// H1 chunk) stores its float32 chunk partials, and after the launch boundary
// every expand workgroup (tile, column chunk) sums them in chunk order and
// applies them.  No workgroup waits on another, so each streams its data
// with the whole chip busy, instead of holding a slot while it waits.  The
// arithmetic and its order are those of lora_mfma_kernel.
// ---------------------------------------------------------------------------
template <typename DT, int R>
__global__ __launch_bounds__(256) void shrink_mfma_kernel(
    const typename DT::storage* __restrict__ x, const typename DT::storage* __restrict__ A_stack,
    const int* __restrict__ seg_indptr, const int* __restrict__ adapter_ids, int S, int num_rows,
    int num_adapters, int H1, float* __restrict__ partials, int ksplit, int h_per_split,
    int compact, float* __restrict__ v_final = nullptr, int* __restrict__ counters = nullptr,
    int counter_stride = 0) {
    using Sh = MfmaShape<R>;
    constexpr int T = Sh::kT;
    constexpr int NT = Sh::kNT;
    constexpr int NW = Sh::kNW;
    __shared__ int s_scan[tile_scan_ints<NT>()];
    __shared__ __align__(16) uint16_t s_a[Sh::kKcMax * R];
    __shared__ float s_red[NW * 16 * R];
    __shared__ int s_last;

    const int g = (int)(blockIdx.x / (unsigned)ksplit);
    const int p = (int)(blockIdx.x % (unsigned)ksplit);
    Tile tile;
    const bool have =
        compact ? locate_tile_compact<NT>(seg_indptr, adapter_ids, S, num_rows, num_adapters, T, g,
                                          s_scan, tile)
                : locate_tile<NT>(seg_indptr, adapter_ids, S, num_rows, num_adapters, T, g, s_scan,
                                  tile);
    if (!have) return;
    // The workgroup's H1 range, in LDS-sized chunks summed in order: the
    // first chunk stores the partial, later ones add to it (each value is
    // read back by the thread that stored it).
    const int h_lo = p * h_per_split;
    const int h_hi = min(H1, h_lo + h_per_split);
    float* out = partials + (long long)p * num_rows * R + (long long)tile.row0 * R;
    for (int c_lo = h_lo; c_lo < h_hi; c_lo += Sh::kKcMax) {
        const bool first = c_lo == h_lo;
        const bool final_chunk = c_lo + Sh::kKcMax >= h_hi;
        shrink_chunk_mfma<DT, R>(A_stack + (long long)tile.adapter * H1 * R,
                                 x + (long long)tile.row0 * H1, tile.nrows, H1, c_lo,
                                 min(h_hi, c_lo + Sh::kKcMax), s_a, s_red,
                                 [&](int i, int k, float v) {
                                     const float val = first ? v : out[i * R + k] + v;
                                     if (v_final && final_chunk)
                                         __hip_atomic_store(&out[i * R + k], val, __ATOMIC_RELAXED,
                                                            __HIP_MEMORY_SCOPE_AGENT);
                                     else
                                         out[i * R + k] = val;
                                 });
    }
    if (!v_final) return;

    // In-kernel reduction (sgmv_shrink): the last of the tile's ksplit
    // workgroups to arrive sums the ranges' partials in order into v_final,
    // as in shrink_vec_kernel; the partials' final stores are write-through
    // and acknowledged before the count, and the counter returns to zero.
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (threadIdx.x == 0) {
        int* cnt = &counters[(long long)g * counter_stride];
        const int before = __hip_atomic_fetch_add(cnt, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const bool last = before == ksplit - 1;
        if (last) __hip_atomic_store(cnt, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        s_last = last;
    }
    __syncthreads();
    if (!s_last) return;
    const long long stride = (long long)num_rows * R;
    for (int t = threadIdx.x; t < tile.nrows * R; t += NT) {
        const int i = t / R;
        const int k = t - i * R;
        float* src = partials + (long long)(tile.row0 + i) * R + k;
        float sum = 0.f;
        for (int c0 = 0; c0 < ksplit; c0 += 8) {
            float pv[8];
#pragma unroll
            for (int u = 0; u < 8; ++u)
                pv[u] = c0 + u < ksplit ? __hip_atomic_load(src + (c0 + u) * stride,
                                                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                                        : 0.f;
#pragma unroll
            for (int u = 0; u < 8; ++u)
                if (c0 + u < ksplit) sum += pv[u];
        }
        v_final[(long long)(tile.row0 + i) * R + k] = sum;
    }
}

template <typename DT, int R>
__global__ __launch_bounds__(256) void expand_mfma_kernel(
    typename DT::storage* __restrict__ y, const typename DT::storage* __restrict__ B_stack,
    const int* __restrict__ seg_indptr, const int* __restrict__ adapter_ids, int S, int num_rows,
    int num_adapters, int H2, float scale, const float* __restrict__ partials, int ksplit,
    int csplit, int compact) {
    using Sh = MfmaShape<R>;
    constexpr int T = Sh::kT;
    constexpr int NT = Sh::kNT;
    constexpr int NW = Sh::kNW;
    constexpr int CW = Sh::kCW;
    __shared__ int s_scan[tile_scan_ints<NT>()];
    __shared__ __align__(16) uint16_t s_b[Sh::kStageB];  // B chunk, then the results
    __shared__ float s_v[T * R];
    __shared__ __align__(16) uint16_t s_vh[T * Sh::kVK];
    __shared__ float s_max[NW];

    const int g = (int)(blockIdx.x / (unsigned)csplit);
    const int c0 = (int)(blockIdx.x % (unsigned)csplit) * CW;
    Tile tile;
    const bool have =
        compact ? locate_tile_compact<NT>(seg_indptr, adapter_ids, S, num_rows, num_adapters, T, g,
                                          s_scan, tile)
                : locate_tile<NT>(seg_indptr, adapter_ids, S, num_rows, num_adapters, T, g, s_scan,
                                  tile);
    if (!have) return;
    const int nrows = tile.nrows;
    ExpandRegs<R> er;
    expand_prefetch<DT, R>(er, B_stack + (long long)tile.adapter * R * H2,
                           y + (long long)tile.row0 * H2, nrows, H2, c0);
    const long long row_stride = (long long)num_rows * R;
    for (int t = threadIdx.x; t < T * R; t += NT) {
        const int i = t / R;
        const int k = t - i * R;
        s_v[t] = i < nrows
                     ? sum_partials(partials + (long long)(tile.row0 + i) * R + k, row_stride, ksplit)
                     : 0.f;
    }
    __syncthreads();
    expand_apply<DT, R>(er, s_b, s_v, s_vh, s_max, y + (long long)tile.row0 * H2, nrows, H2, c0,
                        scale, B_stack + (long long)tile.adapter * R * H2);
}

}  // namespace sgmv
