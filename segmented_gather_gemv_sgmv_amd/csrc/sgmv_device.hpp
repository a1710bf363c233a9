// sgmv_device.hpp -- device-side building blocks shared by the SGMV kernels:
// element types and their float conversions, 16-byte vector unpacking, the
// wave/block scans, and the segment-tile lookup that turns a workgroup index
// into (segment, first row, row count, adapter).
//
// Written for gfx950 (CDNA4): wave64, 64 KB..160 KB LDS per CU.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sgmv {

constexpr int kWave = 64;

// ---------------------------------------------------------------------------
// Element types.  Each exposes its storage type, its size, the conversion of
// one stored element to float, the unpacking of a 16-byte vector into VEC
// floats, and round-to-nearest-even packing back to storage.
// ---------------------------------------------------------------------------
struct F32 {
    using storage = float;
    static constexpr int kBytes = 4;
    static constexpr int kVec = 4;  // elements per 16-byte vector
    __device__ static __forceinline__ float load1(const storage* p) { return *p; }
    __device__ static __forceinline__ void unpack(const uint4& u, float* f) {
        f[0] = __uint_as_float(u.x);
        f[1] = __uint_as_float(u.y);
        f[2] = __uint_as_float(u.z);
        f[3] = __uint_as_float(u.w);
    }
    __device__ static __forceinline__ uint4 pack(const float* f) {
        return make_uint4(__float_as_uint(f[0]), __float_as_uint(f[1]),
                          __float_as_uint(f[2]), __float_as_uint(f[3]));
    }
    __device__ static __forceinline__ storage from_float(float f) { return f; }
};

struct F16 {
    using storage = uint16_t;  // IEEE binary16 bits
    static constexpr int kBytes = 2;
    static constexpr int kVec = 8;
    __device__ static __forceinline__ float h2f(uint32_t bits16) {
        return (float)__builtin_bit_cast(_Float16, (uint16_t)bits16);
    }
    __device__ static __forceinline__ uint32_t f2h(float f) {
        // v_cvt_f16_f32 rounds to nearest-even under the default mode.
        return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)f);
    }
    __device__ static __forceinline__ float load1(const storage* p) { return h2f(*p); }
    __device__ static __forceinline__ void unpack2(uint32_t w, float* f) {
        f[0] = h2f(w & 0xFFFFu);
        f[1] = h2f(w >> 16);
    }
    __device__ static __forceinline__ void unpack(const uint4& u, float* f) {
        unpack2(u.x, f);
        unpack2(u.y, f + 2);
        unpack2(u.z, f + 4);
        unpack2(u.w, f + 6);
    }
    __device__ static __forceinline__ uint32_t pack2(float lo, float hi) {
        return f2h(lo) | (f2h(hi) << 16);
    }
    __device__ static __forceinline__ uint4 pack(const float* f) {
        return make_uint4(pack2(f[0], f[1]), pack2(f[2], f[3]), pack2(f[4], f[5]),
                          pack2(f[6], f[7]));
    }
    __device__ static __forceinline__ storage from_float(float f) { return (storage)f2h(f); }
};

struct BF16 {
    using storage = uint16_t;  // bfloat16 bits (upper half of a float)
    static constexpr int kBytes = 2;
    static constexpr int kVec = 8;
    __device__ static __forceinline__ float b2f(uint32_t bits16) {
        return __uint_as_float(bits16 << 16);
    }
    __device__ static __forceinline__ uint32_t f2b(float f) {
        // Round to nearest, ties to even; NaN stays a quiet NaN.
        uint32_t u = __float_as_uint(f);
        if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0u;
        u += 0x7FFFu + ((u >> 16) & 1u);
        return u >> 16;
    }
    __device__ static __forceinline__ float load1(const storage* p) { return b2f(*p); }
    __device__ static __forceinline__ void unpack2(uint32_t w, float* f) {
        f[0] = __uint_as_float(w << 16);
        f[1] = __uint_as_float(w & 0xFFFF0000u);
    }
    __device__ static __forceinline__ void unpack(const uint4& u, float* f) {
        unpack2(u.x, f);
        unpack2(u.y, f + 2);
        unpack2(u.z, f + 4);
        unpack2(u.w, f + 6);
    }
    __device__ static __forceinline__ uint32_t pack2(float lo, float hi) {
        return f2b(lo) | (f2b(hi) << 16);
    }
    __device__ static __forceinline__ uint4 pack(const float* f) {
        return make_uint4(pack2(f[0], f[1]), pack2(f[2], f[3]), pack2(f[4], f[5]),
                          pack2(f[6], f[7]));
    }
    __device__ static __forceinline__ storage from_float(float f) { return (storage)f2b(f); }
};

__device__ __forceinline__ uint4 load16(const void* p) {
    return *reinterpret_cast<const uint4*>(p);
}
__device__ __forceinline__ void store16(void* p, const uint4& v) {
    *reinterpret_cast<uint4*>(p) = v;
}

// The same accesses with the nontemporal hint, for y: an expand reads each
// piece of y once and writes it back once, so nothing the caches keep of
// it is used again within the call.  On gfx950 a read-modify-write stream
// that carries the hint on both the load and the store runs markedly
// closer to the HBM rate than one without (measured: 32-row x 1 KB tiles
// of a 4096 x 4096 fp16 matrix, 12.1 us against 17.7 us); 8-byte pieces
// do not gain, and read-only streams (x, the weights) do not either.
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 load16_stream(const void* p) {
    const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void store16_stream(void* p, const uint4& v) {
    const u32x4_t w = {v.x, v.y, v.z, v.w};
    __builtin_nontemporal_store(w, reinterpret_cast<u32x4_t*>(p));
}

// ---------------------------------------------------------------------------
// Scans.
// ---------------------------------------------------------------------------
// Inclusive prefix sum over the 64 lanes of a wave with DPP moves (no LDS
// round trips): row shifts by 1, 2, 4 and 8 scan each row of 16 lanes (a
// lane whose source lies outside its row adds 0), then the last lane of
// row 0 is added to row 1 and that of row 2 to row 3 (row_bcast:15, rows
// 1 and 3 enabled), and the last lane of row 1 to rows 2 and 3
// (row_bcast:31).  Checked against a plain prefix sum on gfx950.
__device__ __forceinline__ int wave_inclusive_scan(int v, int lane) {
    (void)lane;
    v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, false);  // row_shr:1
    v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, false);  // row_shr:2
    v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, false);  // row_shr:4
    v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, false);  // row_shr:8
    v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false);  // row_bcast:15
    v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false);  // row_bcast:31
    return v;
}

// Block-wide inclusive scan of one int per thread.  `lds` holds NT/64 ints.
// Returns the thread's inclusive prefix; `total` receives the block sum.
template <int NT>
__device__ __forceinline__ int block_inclusive_scan(int v, int* lds, int& total) {
    constexpr int NW = NT / kWave;
    const int lane = threadIdx.x & (kWave - 1);
    const int wid = threadIdx.x / kWave;
    v = wave_inclusive_scan(v, lane);
    if (lane == kWave - 1) lds[wid] = v;
    __syncthreads();
    int off = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        const int t = lds[w];
        off += (w < wid) ? t : 0;
        tot += t;
    }
    __syncthreads();
    total = tot;
    return v + off;
}

// ---------------------------------------------------------------------------
// Segment tiles.
//
// A segment of n rows is cut into ceil(n / T) tiles of at most T rows.  A
// launch has S + floor(num_rows / T) tile slots, which bounds the number of
// tiles from above (sum of ceil(n_s / T) <= sum of floor(n_s / T) + S).
// Slot g < S is the first tile of segment g (found with three scalar loads);
// slot g >= S is the (g - S)-th of the remaining tiles, counted segment by
// segment, and is found with a block scan over the segment table.  Slots
// beyond the real tile count find nothing and their workgroups exit.
//
// Segment bounds are clamped to [0, num_rows) and a segment whose adapter
// id is outside [0, num_adapters) has no tiles, so a malformed table never
// makes a kernel touch memory outside the arrays it was given.
// ---------------------------------------------------------------------------
struct Tile {
    int seg;
    int row0;
    int nrows;
    int adapter;
};

struct SegBounds {
    int lo, hi;
    bool ok;
};

__device__ __forceinline__ SegBounds seg_bounds(const int* __restrict__ seg_indptr,
                                                const int* __restrict__ adapter_ids, int s,
                                                int num_rows, int num_adapters) {
    int lo = seg_indptr[s];
    int hi = seg_indptr[s + 1];
    const int a = adapter_ids[s];
    lo = min(max(lo, 0), num_rows);
    hi = min(max(hi, lo), num_rows);
    SegBounds b;
    b.lo = lo;
    b.hi = hi;
    b.ok = (a >= 0) && (a < num_adapters) && (hi > lo);
    return b;
}

// LDS a tile lookup needs: the scan's per-wave totals and what the owning
// thread found (segment, tile index, bounds, adapter), so that nobody has
// to read the table again after the scan.
template <int NT>
constexpr int tile_scan_ints() { return NT / kWave + 8; }

// `lds` must hold tile_scan_ints<NT>() ints.  Every thread of the block must
// call this (it synchronises the block when g >= S).
template <int NT>
__device__ __forceinline__ bool locate_tile(const int* __restrict__ seg_indptr,
                                            const int* __restrict__ adapter_ids, int S,
                                            int num_rows, int num_adapters, int T, int g,
                                            int* lds, Tile& out) {
    if (g < S) {
        const SegBounds b = seg_bounds(seg_indptr, adapter_ids, g, num_rows, num_adapters);
        if (!b.ok) return false;
        out.seg = g;
        out.row0 = b.lo;
        out.nrows = min(T, b.hi - b.lo);
        out.adapter = adapter_ids[g];
        return true;
    }
    const int q = g - S;  // index among the non-first tiles
    int* found = lds + NT / kWave;  // segment, tile index in segment, lo, hi, adapter
    if (threadIdx.x == 0) found[0] = -1;
    __syncthreads();
    int running = 0;  // non-first tiles in the segments already scanned
    for (int base = 0; base < S; base += NT) {
        const int s = base + (int)threadIdx.x;
        int extra = 0;
        if (s < S) {
            const SegBounds b = seg_bounds(seg_indptr, adapter_ids, s, num_rows, num_adapters);
            if (b.ok) extra = (b.hi - b.lo + T - 1) / T - 1;
        }
        int total;
        const int incl = block_inclusive_scan<NT>(extra, lds, total);
        const int excl = running + incl - extra;
        if (extra > 0 && q >= excl && q < excl + extra) {
            const SegBounds b = seg_bounds(seg_indptr, adapter_ids, s, num_rows, num_adapters);
            found[0] = s;
            found[1] = q - excl + 1;
            found[2] = b.lo;
            found[3] = b.hi;
            found[4] = adapter_ids[s];
        }
        running += total;
        if (q < running) break;  // uniform: running and q are block-uniform
    }
    __syncthreads();
    const int s = found[0];
    if (s < 0) return false;
    out.seg = s;
    out.row0 = found[2] + found[1] * T;
    out.nrows = min(T, found[3] - out.row0);
    out.adapter = found[4];
    return true;
}

// Compact mapping: slot g is the g-th tile in segment order (all tiles of
// segment 0, then of segment 1, ...), found with a block scan of the
// per-segment tile counts.  A segment table with S segments over R rows has
// at most m + floor((R - m) / T) tiles, m = min(S, R) (each non-empty
// segment of n rows has 1 + floor((n - 1) / T) tiles), so a launch needs no
// slot that finds nothing.  `lds` must hold tile_scan_ints<NT>() ints.
// Every thread of the block must call this.
template <int NT>
__device__ __forceinline__ bool locate_tile_compact(const int* __restrict__ seg_indptr,
                                                    const int* __restrict__ adapter_ids, int S,
                                                    int num_rows, int num_adapters, int T, int g,
                                                    int* lds, Tile& out) {
    constexpr int NW = NT / kWave;
    const int lane = threadIdx.x & (kWave - 1);
    const int wid = threadIdx.x / kWave;
    int* wave_tot = lds;            // [NW]
    int* found = lds + NW;          // segment, tile index in segment, lo, hi, adapter
    int running = 0;                // tiles in the segments already scanned
    for (int base = 0; base < S; base += NT) {
        const int s = base + (int)threadIdx.x;
        int cnt = 0;
        SegBounds b{0, 0, false};
        if (s < S) {
            b = seg_bounds(seg_indptr, adapter_ids, s, num_rows, num_adapters);
            if (b.ok) cnt = (b.hi - b.lo + T - 1) / T;
        }
        const int incl_w = wave_inclusive_scan(cnt, lane);
        if (lane == kWave - 1) wave_tot[wid] = incl_w;
        __syncthreads();
        int off = 0, total = 0;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            const int t = wave_tot[w];
            off += (w < wid) ? t : 0;
            total += t;
        }
        const int excl = running + off + incl_w - cnt;
        // Exactly one thread owns tile g if it lies in this pass.
        if (cnt > 0 && g >= excl && g < excl + cnt) {
            found[0] = s;
            found[1] = g - excl;
            found[2] = b.lo;
            found[3] = b.hi;
            found[4] = adapter_ids[s];
        }
        running += total;
        __syncthreads();  // found[] visible; wave_tot[] free for the next pass
        if (g < running) break;  // block-uniform
    }
    if (g >= running) return false;  // fewer tiles than g + 1
    out.seg = found[0];
    out.row0 = found[2] + found[1] * T;
    out.nrows = min(T, found[3] - out.row0);
    out.adapter = found[4];
    return true;
}

}  // namespace sgmv
