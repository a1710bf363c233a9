// sgmv_segments.hpp -- segment tables from per-row adapter ids, on the device.
//
// A serving batch usually arrives tagged per row: row i uses adapter
// row_ids[i] (the per-sample LoRA indices of Punica walkthrough,
// omica.com.cn/news/959180, section 3.2), while SGMV wants contiguous
// segments, each naming one adapter (Punica review, nubint.ai, "Proposed
// method").  Two builders, each a single workgroup of 1024 threads (batches
// are thousands of rows at most, so one workgroup keeps the launch cheap):
//
//  * build_segments_kernel: one segment per maximal run of equal ids, in row
//    order.  Needs no permutation: an adapter may name several segments.
//  * group_rows_kernel: a stable grouping by adapter -- perm lists the rows
//    of adapter 0, then adapter 1, ... (each in increasing row order), then
//    the rows whose id is not a valid adapter -- and one segment per adapter
//    present, in increasing id order, over the grouped order.
//
// Both normalise an id outside [0, num_adapters) to "no adapter": such rows
// are in no segment of the grouped table, and form segments with adapter id
// -1 (which lora_apply skips) in the run table.  Entries of the output
// arrays past the real segment count describe empty segments, so a caller
// may pass the table's size -- num_rows for runs, min(num_rows,
// num_adapters) for the grouping -- as the segment count without reading
// the count back.
#pragma once

#include "sgmv_device.hpp"

namespace sgmv {

constexpr int kSegThreads = 1024;
constexpr int kGroupMaxAdapters = 4096;  // adapter bins held in LDS

__device__ __forceinline__ int norm_id(int id, int num_adapters) {
    return (id >= 0 && id < num_adapters) ? id : -1;
}

// Exclusive block scan of one int per thread over kSegThreads threads;
// `total` receives the sum.  `lds` holds kSegThreads / 64 ints.
__device__ __forceinline__ int seg_block_excl_scan(int v, int* lds, int& total) {
    const int incl = block_inclusive_scan<kSegThreads>(v, lds, total);
    return incl - v;
}

__global__ __launch_bounds__(kSegThreads) void build_segments_kernel(
    const int* __restrict__ row_ids, int num_rows, int num_adapters, int* __restrict__ seg_indptr,
    int* __restrict__ adapter_ids, int* __restrict__ num_segments) {
    __shared__ int s_scan[kSegThreads / kWave];
    const int tid = threadIdx.x;
    int running = 0;  // segments started in earlier passes (block-uniform)
    for (int base = 0; base < num_rows; base += kSegThreads) {
        const int i = base + tid;
        const bool in = i < num_rows;
        const int b = in ? norm_id(row_ids[i], num_adapters) : 0;
        const bool start = in && (i == 0 || norm_id(row_ids[i - 1], num_adapters) != b);
        int total;
        const int excl = seg_block_excl_scan(start ? 1 : 0, s_scan, total);
        if (start) {
            seg_indptr[running + excl] = i;
            adapter_ids[running + excl] = b;
        }
        running += total;
    }
    // Empty segments fill the rest: seg_indptr[S .. num_rows] = num_rows.
    for (int k = running + tid; k <= num_rows; k += kSegThreads) {
        seg_indptr[k] = num_rows;
        if (k < num_rows) adapter_ids[k] = -1;
    }
    if (tid == 0) *num_segments = running;
}

// Lanes of a wave that share a bin: for a lane with b >= 0, `rank` is the
// number of lower lanes with the same bin, `cnt` the number of lanes with
// it, and `last` marks the highest such lane.  One round per distinct bin in
// the wave (the loop is wave-uniform).
__device__ __forceinline__ void wave_match(int b, int& rank, int& cnt, bool& last) {
    const int lane = threadIdx.x & (kWave - 1);
    const unsigned long long below = (1ull << lane) - 1ull;
    unsigned long long remaining = __ballot(b >= 0);
    rank = 0;
    cnt = 0;
    last = false;
    while (remaining) {
        const int leader = __ffsll((long long)remaining) - 1;
        const int bl = __shfl(b, leader);
        const unsigned long long m = __ballot(b == bl);
        if (b == bl) {
            rank = __popcll(m & below);
            cnt = __popcll(m);
            last = (63 - __clzll((long long)m)) == lane;
        }
        remaining &= ~m;
    }
}

// Stable grouping.  Bin a < num_adapters holds adapter a's rows, bin
// num_adapters the rows without a valid adapter.
__global__ __launch_bounds__(kSegThreads) void group_rows_kernel(
    const int* __restrict__ row_ids, int num_rows, int num_adapters, int* __restrict__ perm,
    int* __restrict__ seg_indptr, int* __restrict__ adapter_ids, int* __restrict__ num_segments) {
    __shared__ int s_off[kGroupMaxAdapters + 1];  // counts, then first position of each bin
    __shared__ int s_run[kGroupMaxAdapters + 1];  // rows of each bin placed so far
    __shared__ int s_scan[kSegThreads / kWave];
    const int tid = threadIdx.x;
    const int nbins = num_adapters + 1;
    auto bin_of = [&](int i) {
        const int a = norm_id(row_ids[i], num_adapters);
        return a < 0 ? num_adapters : a;
    };

    for (int a = tid; a < nbins; a += kSegThreads) {
        s_off[a] = 0;
        s_run[a] = 0;
    }
    __syncthreads();
    // Counts: one LDS addition per bin per wave, so that long runs of one
    // adapter do not serialise on a single counter.
    for (int base = 0; base < num_rows; base += kSegThreads) {
        const int i = base + tid;
        const int b = i < num_rows ? bin_of(i) : -1;
        int rank, cnt;
        bool last;
        wave_match(b, rank, cnt, last);
        if (last) atomicAdd(&s_off[b], cnt);
    }
    __syncthreads();

    // Counts -> first positions; adapters present -> segments.
    int pos = 0, segs = 0;  // block-uniform running totals
    for (int base = 0; base < nbins; base += kSegThreads) {
        const int a = base + tid;
        const int c = a < nbins ? s_off[a] : 0;
        const int present = (a < num_adapters && c > 0) ? 1 : 0;
        int tot_c, tot_p;
        const int ex_c = seg_block_excl_scan(c, s_scan, tot_c);
        const int ex_p = seg_block_excl_scan(present, s_scan, tot_p);
        if (a < nbins) s_off[a] = pos + ex_c;
        if (present) {
            seg_indptr[segs + ex_p] = pos + ex_c;
            adapter_ids[segs + ex_p] = a;
        }
        pos += tot_c;
        segs += tot_p;
    }
    __syncthreads();
    const int grouped = s_off[num_adapters];  // rows with a valid adapter
    const int smax = min(num_rows, num_adapters);  // table size: at most one segment per adapter
    for (int k = segs + tid; k <= smax; k += kSegThreads) {
        seg_indptr[k] = grouped;
        if (k < smax) adapter_ids[k] = -1;
    }
    if (tid == 0) *num_segments = segs;

    // Rows in order, a pass of kSegThreads at a time.  A row's place in its
    // bin is the bin's rows in earlier passes and earlier waves (s_run) plus
    // the lower lanes of its wave with the same bin; the waves of a pass take
    // their turn in order, so the grouping is stable.
    const int wid = tid / kWave;
    for (int base = 0; base < num_rows; base += kSegThreads) {
        const int i = base + tid;
        const int b = i < num_rows ? bin_of(i) : -1;
        int rank, cnt;
        bool last;
        wave_match(b, rank, cnt, last);
        for (int w = 0; w < kSegThreads / kWave; ++w) {
            if (wid == w && b >= 0) {
                perm[s_off[b] + s_run[b] + rank] = i;
                // every lane has read s_run[b] before its bin's last lane adds
                __builtin_amdgcn_wave_barrier();
                if (last) s_run[b] += cnt;
            }
            __syncthreads();
        }
    }
}

}  // namespace sgmv
