// sgmv_api.hip -- the C ABI of libsgmv.so (declared in include/sgmv.h):
// argument checks, the launch plan (grid sizes and the split of the H1
// reduction, a pure function of the shapes so the workspace size can be
// queried ahead of time), and kernel dispatch on element type and rank.
//
// No call allocates memory, keeps state or synchronises the host: kernels
// are enqueued on the caller's stream and the call returns.
#include <hip/hip_runtime.h>

#include <stdint.h>

#include <algorithm>
#include <atomic>
#include <cstring>
#include <map>
#include <mutex>
#include <tuple>
#include <type_traits>
#include <utility>

#include "sgmv.h"
#include "sgmv_device.hpp"
#include "sgmv_gemv.hpp"
#include "sgmv_fused.hpp"
#include "sgmv_mfma.hpp"
#include "sgmv_segments.hpp"
#include "sgmv_linear.hpp"
#include "sgmv_mixed.hpp"

namespace {

using namespace sgmv;

constexpr int kShrinkThreads = 256;  // threads per shrink workgroup
constexpr int kShrinkRows = 8;       // rows per shrink tile
constexpr int kShrinkPG = 4;         // A loads in flight per lane
constexpr int kExpandRows = 4;       // rows per expand tile
constexpr int kGenericRows = 4;      // rows per tile in the general kernels
constexpr int kGenericThreads = 256;
constexpr int kFusedThreads = 256;   // threads per fused lora_apply workgroup
constexpr int kFusedPG = 4;          // A loads in flight per lane (fused shrink)
constexpr int kFusedItems = 1024;    // items that fit one resident wave (4 per CU)
constexpr long long kFusedMaxChunk = 64 * 1024;  // largest A chunk per shrink item
constexpr int kCompactMaxSegments = 1024;  // beyond: direct + overflow tile mapping
constexpr double kDefaultWaitSeconds = 0.02;  // patience of a fused expand item
constexpr int kTargetWorkgroups = 1024;  // at least four per CU on 256 CUs
constexpr long long kMinChunkBytes = 4096;  // smallest A chunk worth a workgroup
constexpr long long kMaxGrid = 0x7FFFFFFFLL;

int elem_bytes(int dtype) { return dtype == SGMV_F32 ? 4 : 2; }
int vec_width(int dtype) { return dtype == SGMV_F32 ? 4 : 8; }

// Ranks with a vectorised kernel: r a multiple of the vector width with
// r / VEC dividing the wave.
bool vec_rank(int dtype, int r) {
    switch (r) {
        case 4: return dtype == SGMV_F32;
        case 8: case 16: case 32: case 64: case 128: return true;
        default: return false;
    }
}

// Tile slots of a launch whose kernel cuts segments into tiles of `rows`
// rows (see locate_tile): an upper bound on the number of tiles.
long long tile_slots(int num_segments, int num_rows, int rows) {
    return (long long)num_segments + num_rows / rows;
}

struct Plan {
    int ksplit;       // chunks of the H1 reduction
    int h_per_split;  // rows of A per chunk
    int num_segments, num_rows;
    int rows;         // rows per tile of the vectorised shrink
};

// Pure function of the shapes (not of pointers), so that the workspace size
// reported before a call matches what the call uses.
Plan make_plan(int num_rows, int num_segments, int H1, int r, int dtype) {
    Plan p;
    p.num_segments = num_segments;
    p.num_rows = num_rows;
    const bool vec = vec_rank(dtype, r);
    // The split is sized with the vectorised kernel's tile height whichever
    // kernel runs, so that it stays a function of the shapes alone.
    // One-row tiles when no segment needs more on average (decode batches):
    // a tile's registers then hold one row's accumulators, not eight.
    p.rows = num_rows <= num_segments ? 1 : kShrinkRows;
    const long long slots = tile_slots(num_segments, num_rows, vec ? p.rows : kGenericRows);

    // Enough workgroups to fill the chip, but no chunk below kMinChunkBytes.
    const long long a_bytes = (long long)H1 * r * elem_bytes(dtype);
    long long maxk = a_bytes / kMinChunkBytes;
    if (maxk < 1) maxk = 1;
    long long want = (kTargetWorkgroups + slots - 1) / (slots > 0 ? slots : 1);
    long long k = 1;
    while (k < want && k * 2 <= maxk) k *= 2;
    // Chunk boundaries on whole block-wide passes of the vectorised kernel.
    const int unit = vec ? kShrinkThreads / (r / vec_width(dtype)) : 64;
    long long hps = (H1 + k - 1) / k;
    hps = (hps + unit - 1) / unit * unit;
    p.h_per_split = (int)hps;
    p.ksplit = (int)((H1 + hps - 1) / hps);
    return p;
}

// Workspace layout shared by sgmv_shrink and lora_apply:
//   [0, kCounterBytes)   counters of the fused kernel: one per tile slot,
//                        kCounterStride ints apart (one 128-byte line each,
//                        so atomics on different tiles do not contend), and a
//                        sticky timeout flag in the last int.  Zero before
//                        first use; every call leaves the tile counters at
//                        zero.  The offset and size do not depend on the
//                        shapes, so one buffer can serve calls of any shape.
//   [kCounterBytes, ...) float32 chunk partials [ksplit][num_rows][r].
constexpr int kCounterInts = 65536;
constexpr int kCounterStride = 32;
constexpr int kCounterSlots = kCounterInts / kCounterStride - 1;
constexpr size_t kCounterBytes = kCounterInts * sizeof(int);

// Columns of an MFMA expand item (MfmaShape::kCW in sgmv_mfma.hpp).
constexpr int mfma_expand_cols(int r) { return r >= 64 ? 256 : std::min(512, 8192 / r); }
static_assert(mfma_expand_cols(16) == MfmaShape<16>::kCW && mfma_expand_cols(32) == MfmaShape<32>::kCW &&
                  mfma_expand_cols(64) == MfmaShape<64>::kCW &&
                  mfma_expand_cols(128) == MfmaShape<128>::kCW,
              "host and device agree on the expand item width");

// Launch plan of the single-kernel lora_apply (a pure function of shapes).
struct FusedPlan {
    bool ok;            // shapes allow it (alignment is checked per call)
    int rows;           // tile rows: 1 when no segment needs more on average
    int compact;        // compact tile mapping (block scan) vs direct + overflow
    long long slots_a, slots_b;
    int ksplit, h_per_split, csplit;
    long long grid;
};

FusedPlan make_fused_plan(int num_rows, int num_segments, int H1, int H2, int r, int dtype,
                          long long items = kFusedItems) {
    FusedPlan f{};
    if (!vec_rank(dtype, r)) return f;
    const int vec = vec_width(dtype);
    f.rows = num_rows <= num_segments ? 1 : 4;
    f.compact = num_segments <= kCompactMaxSegments;
    if (f.compact) {
        const long long m = num_segments < num_rows ? num_segments : num_rows;
        f.slots_a = m + (num_rows - m) / f.rows;
        f.slots_b = 0;
    } else {
        f.slots_a = num_segments;
        f.slots_b = num_rows / f.rows;
    }
    const long long slots = f.slots_a + f.slots_b;
    const int cw = kFusedThreads * vec;
    f.csplit = (H2 + cw - 1) / cw;
    // Split of the H1 reduction: as fine as fits one resident wave of items,
    // but chunks between kMinChunkBytes and kFusedMaxChunk of A.
    const long long a_bytes = (long long)H1 * r * elem_bytes(dtype);
    long long hi = a_bytes / kMinChunkBytes;
    if (hi < 1) hi = 1;
    long long lo = 1;
    while (lo * kFusedMaxChunk < a_bytes && lo < hi) lo *= 2;
    long long k = 1;
    while (k * 2 <= hi && slots * (k * 2 + f.csplit) <= items) k *= 2;
    if (k < lo) k = lo;
    const int unit = kFusedThreads / (r / vec);
    long long hps = (H1 + k - 1) / k;
    hps = (hps + unit - 1) / unit * unit;
    f.h_per_split = (int)hps;
    f.ksplit = (int)((H1 + hps - 1) / hps);
    f.grid = slots * (f.ksplit + f.csplit);
    f.ok = slots <= kCounterSlots && f.ksplit < (1 << 16) && f.csplit < (1 << 15) &&
           f.grid <= kMaxGrid;
    return f;
}

// Launch plan of the MFMA row-tile kernel (16-row tiles, fp16/bf16, r a
// multiple of 16): chosen when segments hold several rows on average, where
// the two contractions are dense enough for the matrix cores.
constexpr int kMfmaRowsPerSegment = 4;  // use MFMA tiles when R >= 4 S
struct MfmaPlan {
    bool ok;
    int compact;
    long long slots_a, slots_b;
    int ksplit, h_per_split, csplit;
    long long grid;
};

MfmaPlan make_mfma_plan(int num_rows, int num_segments, int H1, int H2, int r, int dtype) {
    MfmaPlan f{};
    if (dtype == SGMV_F32 || (r != 16 && r != 32 && r != 64 && r != 128)) return f;
    if (H1 % 8 != 0 || H2 % 8 != 0) return f;
    constexpr int T = 16;
    f.compact = num_segments <= kCompactMaxSegments;
    if (f.compact) {
        const long long m = num_segments < num_rows ? num_segments : num_rows;
        f.slots_a = m + (num_rows - m) / T;
        f.slots_b = 0;
    } else {
        f.slots_a = num_segments;
        f.slots_b = num_rows / T;
    }
    const long long slots = f.slots_a + f.slots_b;
    const int kc_max = 16384 / r;
    const int cw = mfma_expand_cols(r);
    f.csplit = (H2 + cw - 1) / cw;
    // Fewest chunks that fit the LDS copy of A, more while items still fit
    // one resident wave and chunks keep at least 256 rows of A.
    long long k = (H1 + kc_max - 1) / kc_max;
    while (H1 / (k * 2) >= 256 && slots * (k * 2 + f.csplit) <= kFusedItems) k *= 2;
    long long hps = (H1 + k - 1) / k;
    hps = (hps + 127) / 128 * 128;
    if (hps > kc_max) hps = kc_max;
    f.h_per_split = (int)hps;
    f.ksplit = (int)((H1 + hps - 1) / hps);
    f.grid = slots * (f.ksplit + f.csplit);
    f.ok = slots <= kCounterSlots && f.ksplit < (1 << 16) && f.csplit < (1 << 15) &&
           f.grid <= kMaxGrid;
    return f;
}

// Plan of the two-launch MFMA form (shrink_mfma_kernel, then
// expand_mfma_kernel), taken when the single-kernel form would need more
// than two rounds of resident items: then waiting items hold slots that
// streaming ones could use, and one more launch costs little.
struct MfmaSplitPlan {
    bool ok;
    int compact;
    long long slots;
    int ksplit, h_per_split, csplit;
    long long grid_shrink, grid_expand;
};

MfmaSplitPlan make_mfma_split_plan(const MfmaPlan& mp, int H1, int H2, int r) {
    MfmaSplitPlan sp{};
    if (!mp.ok) return sp;
    sp.compact = mp.compact;
    sp.slots = mp.slots_a + mp.slots_b;
    if (sp.slots * (mp.ksplit + mp.csplit) <= 2LL * kFusedItems) return sp;
    const int kc_max = 16384 / r;
    const int cw = mfma_expand_cols(r);
    sp.csplit = (H2 + cw - 1) / cw;
    // Fewest chunks that fit the LDS copy of A, more while the shrink launch
    // has fewer than kTargetWorkgroups workgroups and chunks keep >= 256 rows.
    long long k = (H1 + kc_max - 1) / kc_max;
    while (sp.slots * k < kTargetWorkgroups && H1 / (k * 2) >= 256) k *= 2;
    long long hps = (H1 + k - 1) / k;
    hps = (hps + 127) / 128 * 128;
    if (hps > kc_max) hps = kc_max;
    // Large ranks have small LDS chunks, and one workgroup (with one
    // float32 partial of the tile's v) per chunk multiplies the partials:
    // at r = 128 and H1 = 4096, 32 chunks write and re-read 16 KB per row,
    // twice the row of x.  Where the partials are heavy (chunks x rank >
    // 256), a workgroup takes as many chunks as keep the launch near one
    // round of workgroups; for small ranks, more workgroups in flight pay
    // more than the partials cost.
    if (k * r > 256 && sp.slots * k > 2LL * kTargetWorkgroups) {
        const long long cpw = (sp.slots * k + kTargetWorkgroups - 1) / kTargetWorkgroups;
        hps = cpw * kc_max;
    }
    sp.h_per_split = (int)hps;
    sp.ksplit = (int)((H1 + hps - 1) / hps);
    sp.grid_shrink = sp.slots * sp.ksplit;
    sp.grid_expand = sp.slots * sp.csplit;
    sp.ok = sp.grid_shrink <= kMaxGrid && sp.grid_expand <= kMaxGrid;
    return sp;
}

// -- per-segment path choice (sgmv_mixed.hpp) -----------------------------------
// Every workgroup of the mixed kernels classifies the segments itself: long
// (>= TH rows: 16-row MFMA tiles), short (2..TH-1 rows: 4-row vector tiles),
// single (one row: one-row vector tiles).  The host only picks the chunk
// sizes of each class and sizes the grid by the largest item count any
// table of this length could need.
constexpr long long kMixedBudget = 1024;  // one resident round: four workgroups per CU
constexpr int kMixedMaxSplit = 16;        // one-launch H1 chunks: one batch of partial loads

struct MixedShape {
    bool ok;               // the mixed kernels serve these shapes
    bool has_long, has_short;
    int TH;                // rows from which a segment is long
    int T[3];              // tile rows: long, short, single
    int cw[3], unit[3], hmax[3];  // columns per expand item, H1 unit, rows per LDS chunk (0: any)
    int e, r;
};

MixedShape mixed_shape(int H1, int H2, int r, int dtype) {
    MixedShape m{};
    if (!vec_rank(dtype, r)) return m;
    const int vec = vec_width(dtype);
    if (H2 % vec != 0) return m;
    const bool mfma_rank = dtype != SGMV_F32 && r >= 16;
    if (mfma_rank && (H1 % 8 != 0 || H2 % 8 != 0)) return m;  // the per-call kernels serve these
    m.e = elem_bytes(dtype);
    m.r = r;
    m.has_long = mfma_rank;
    m.has_short = !mfma_rank;
    m.TH = !m.has_long ? 0x7FFFFFFF : (m.has_short ? 16 : 2);
    const int vunit = kMixedThreads / (r / vec);
    m.T[0] = 16;
    m.cw[0] = mfma_expand_cols(r);
    m.unit[0] = 128;
    m.hmax[0] = std::max(128, 8192 / r);  // MfmaTile's LDS chunk of A
    m.T[1] = 4;
    m.T[2] = 1;
    for (int c = 1; c < 3; ++c) {
        m.cw[c] = kMixedThreads * vec / vec_rank_groups(r, m.T[c]);  // VecTile::kCW
        m.unit[c] = vunit;
        m.hmax[c] = 0;
    }
    m.ok = true;
    return m;
}

// An upper bound, over every table of S segments on R rows, of
// sum over segments of q[class] * (tiles of the segment).  A segment of n
// rows in a class of tile height T has ceil(n / T) <= 1 + (n - 1) / T
// tiles, linear in n within the class's range of lengths, so the count is
// a linear program over how many segments of each length there are, with
// two constraints (at most S segments, at most R rows).  Its optimum uses at
// most two lengths, and within a class only the ends of its range of
// lengths matter; the bound is that optimum over all pairs of such ends.
long long mixed_bound(long long R, long long S, const MixedShape& ms, const long long (&q)[3]) {
    struct End { double n, v; };
    End ends[6];
    int ne = 0;
    auto add = [&](int c, long long n) {
        if (n < 1 || n > R) return;
        ends[ne++] = End{(double)n, (double)q[c] * (1.0 + (double)(n - 1) / (double)ms.T[c])};
    };
    add(2, 1);
    if (ms.has_short) {
        add(1, 2);
        add(1, std::min<long long>(ms.TH - 1, R));
    }
    if (ms.has_long) {
        add(0, ms.TH);
        add(0, R);
    }
    double best = 0.0;
    for (int a = 0; a < ne; ++a) {
        for (int b = a; b < ne; ++b) {
            const End& A = ends[a];
            const End& B = ends[b];
            // one length alone
            best = std::max(best, std::min((double)S, (double)R / A.n) * A.v);
            best = std::max(best, std::min((double)S, (double)R / B.n) * B.v);
            // both, with both constraints tight
            if (B.n != A.n) {
                const End& lo = A.n < B.n ? A : B;
                const End& hi = A.n < B.n ? B : A;
                const double xh = ((double)R - lo.n * (double)S) / (hi.n - lo.n);
                const double xl = (double)S - xh;
                if (xh >= 0.0 && xl >= 0.0) best = std::max(best, xl * lo.v + xh * hi.v);
            }
        }
    }
    return (long long)best + 1;
}

// Chunk sizes of class c for a target of `tb` bytes per shrink item: an item
// of a tall tile reads its rows of A and, for each of its T rows, the same
// stretch of x; a one-row item reads its rows of A (its stretch of x, 1/r
// of that, stays out of the count so that power-of-two targets give
// power-of-two chunks).  One-launch long chunks stay within one LDS chunk
// of A; two-launch ones may span several (summed in order).
void mixed_split_class(const MixedShape& ms, int c, long long tb, int H1, int H2,
                       bool one_launch, MixedSplit& sp) {
    const int unit = ms.unit[c];
    const long long per_row = (long long)(ms.r + (ms.T[c] > 1 ? ms.T[c] : 0)) * ms.e;
    long long hh = tb / per_row / unit * unit;
    if (hh < unit) hh = unit;
    if (ms.hmax[c] > 0 && one_launch && hh > ms.hmax[c]) hh = ms.hmax[c];
    const long long hcap = ((long long)H1 + unit - 1) / unit * unit;
    if (hh > hcap) hh = hcap;
    const long long kk = (H1 + hh - 1) / hh;
    hh = ((H1 + kk - 1) / kk + unit - 1) / unit * unit;
    sp.k[c] = (int)kk;
    sp.h[c] = (int)hh;
    sp.c[c] = (H2 + ms.cw[c] - 1) / ms.cw[c];
}

// Each class's split on its own: the finest byte target whose items, were
// the whole batch of that class (its own worst case), fit `budget` -- with
// at most `max_k` chunks -- or the coarsest target if none does.  `expand`
// counts expand items as well as shrink items.
MixedSplit mixed_split(const MixedShape& ms, int R, int S, int H1, int H2, bool one_launch,
                       long long budget, int max_k) {
    static const long long kTargets[] = {4096, 8192, 16384, 32768, 65536, 131072, 262144};
    const int n_targets = one_launch ? 5 : 7;
    MixedSplit sp{};
    for (int c = 0; c < 3; ++c) {
        if (one_launch && c == 0) {
            // One-launch MFMA items each take a whole LDS chunk of A (the
            // coarsest target, capped by the chunk): on the Zipf decode batch
            // and its one-segment control, half-chunk items (twice the
            // workgroups) measured 3 % and 2 % slower.
            mixed_split_class(ms, 0, kTargets[n_targets - 1], H1, H2, true, sp);
            continue;
        }
        long long unit_q[3] = {0, 0, 0};
        unit_q[c] = 1;
        const long long tiles_c = mixed_bound(R, S, ms, unit_q);
        for (int i = 0; i < n_targets; ++i) {
            mixed_split_class(ms, c, kTargets[i], H1, H2, one_launch, sp);
            const long long per_tile = sp.k[c] + (one_launch ? sp.c[c] : 0);
            if (tiles_c * per_tile <= budget && sp.k[c] <= max_k) break;
        }
    }
    return sp;
}

constexpr long long kSelfMaxA = 32768;  // bytes of one adapter's A (see make_mixed_plan)

struct MixedPlan {
    bool ok;
    bool two;              // two launches (else one)
    MixedSplit one, two_sp;
    long long grid_one, grid_shrink, grid_expand;
    long long tiles;       // bound on the tiles (tile counters)
    int kmax;              // partial chunks the workspace holds (either form)
};

// Pure function of the shapes: each class split on its own (mixed_split),
// one launch when even the worst mix of classes needs at most two resident
// rounds of items and the tiles fit the counters, else two launches, whose
// shrink launch splits each class to fit two rounds of workgroups.
MixedPlan make_mixed_plan(const MixedShape& ms, int R, int S, int H1, int H2) {
    MixedPlan p{};
    if (!ms.ok || S < 1 || R < 1 || S > kMixedMaxSegments) return p;
    const long long ones[3] = {1, 1, 1};
    p.tiles = mixed_bound(R, S, ms, ones);
    p.one = mixed_split(ms, R, S, H1, H2, true, kMixedBudget, kMixedMaxSplit);
    // Small adapters: when an adapter's A is at most kSelfMaxA bytes and no
    // tile has more than two column chunks, the one-launch form has no
    // shrink items; each expand item computes its tile's v itself (at most
    // twice per tile), which costs less than the hand-off's round trips.
    int cmax = p.one.c[2];
    if (ms.has_long) cmax = std::max(cmax, p.one.c[0]);
    if (ms.has_short) cmax = std::max(cmax, p.one.c[1]);
    if ((long long)H1 * ms.r * ms.e <= kSelfMaxA && cmax <= 2) {
        for (int c = 0; c < 3; ++c) p.one.k[c] = 0;
    }
    const long long q[3] = {p.one.k[0] + p.one.c[0], p.one.k[1] + p.one.c[1],
                            p.one.k[2] + p.one.c[2]};
    p.grid_one = mixed_bound(R, S, ms, q);
    p.two = p.grid_one > 2 * kMixedBudget || p.tiles > kCounterSlots;
    p.two_sp = mixed_split(ms, R, S, H1, H2, false, 2 * kMixedBudget, 1 << 15);
    const long long qk[3] = {p.two_sp.k[0], p.two_sp.k[1], p.two_sp.k[2]};
    const long long qc[3] = {p.two_sp.c[0], p.two_sp.c[1], p.two_sp.c[2]};
    p.grid_shrink = mixed_bound(R, S, ms, qk);
    p.grid_expand = mixed_bound(R, S, ms, qc);
    p.kmax = 0;
    bool fits = true;
    for (int c = 0; c < 3; ++c) {
        p.kmax = std::max(p.kmax, std::max(p.one.k[c], p.two_sp.k[c]));
        fits = fits && p.one.k[c] < (1 << 16) && p.one.c[c] < (1 << 15) && p.two_sp.k[c] >= 1;
    }
    p.ok = fits && p.grid_one <= kMaxGrid && p.grid_shrink <= kMaxGrid &&
           p.grid_expand <= kMaxGrid;
    return p;
}

// The two-launch lora_apply's expand item table (sgmv_mixed.hpp, item_count):
// grid_expand 16-byte entries and the count, after the largest partials
// either form of the mixed path writes.
size_t mixed_table_offset(const MixedPlan& xp, long long num_rows, int r) {
    const size_t part = (size_t)xp.kmax * (size_t)num_rows * (size_t)r * sizeof(float);
    return kCounterBytes + ((part + 255) & ~(size_t)255);
}

size_t mixed_table_end(const MixedPlan& xp, long long num_rows, int r) {
    return mixed_table_offset(xp, num_rows, r) + (size_t)(xp.grid_expand + 1) * 16;
}

// Calls f(DT{}, integral_constant<R>{}, LongP{}, ShortP{}, SingleP{}) for the
// mixed kernels of the dtype and rank (the classes as mixed_shape defines them).
template <typename F>
void with_mixed(int dtype, int r, F&& f) {
    auto by_rank = [&](auto dt) {
        using DT = decltype(dt);
        auto go = [&](auto rank) {
            constexpr int R = decltype(rank)::value;
            using G = VecTile<DT, R, 1>;
            if constexpr (!std::is_same<DT, F32>::value && R >= 16)
                f(dt, rank, MfmaTile<DT, R>{}, NoTile<DT>{}, G{});
            else
                f(dt, rank, NoTile<DT>{}, ShortTile<DT, R>{}, G{});
        };
        switch (r) {
            case 4:
                if constexpr (DT::kVec == 4) go(std::integral_constant<int, 4>{});
                break;
            case 8: go(std::integral_constant<int, 8>{}); break;
            case 16: go(std::integral_constant<int, 16>{}); break;
            case 32: go(std::integral_constant<int, 32>{}); break;
            case 64: go(std::integral_constant<int, 64>{}); break;
            default: go(std::integral_constant<int, 128>{}); break;
        }
    };
    switch (dtype) {
        case SGMV_F32: by_rank(F32{}); break;
        case SGMV_F16: by_rank(F16{}); break;
        default: by_rank(BF16{}); break;
    }
}

// Whether the mixed kernels take a call (shapes; alignment is the caller's).
bool mixed_takes(const MixedShape& ms, int S) { return ms.ok && S <= kMixedMaxSegments; }

// Calls f(DT{}, integral_constant<R>) for the MFMA tile kernels' dtypes
// (fp16, bf16) and ranks (16, 32, 64, 128); the caller has checked both.
template <typename F>
void with_mfma_rank(int dtype, int r, F&& f) {
    auto by_rank = [&](auto dt) {
        switch (r) {
            case 16: f(dt, std::integral_constant<int, 16>{}); break;
            case 32: f(dt, std::integral_constant<int, 32>{}); break;
            case 64: f(dt, std::integral_constant<int, 64>{}); break;
            default: f(dt, std::integral_constant<int, 128>{}); break;
        }
    };
    if (dtype == SGMV_F16) by_rank(F16{});
    else by_rank(BF16{});
}

bool use_mfma(int num_rows, int num_segments) {
    return (long long)num_rows >= (long long)kMfmaRowsPerSegment * num_segments;
}

size_t partial_bytes(const Plan& p, int num_rows, int r) {
    return (size_t)p.ksplit * (size_t)num_rows * (size_t)r * sizeof(float);
}

size_t round256(size_t n) { return (n + 255) / 256 * 256; }


// Process-wide patience of the fused kernel's expand workgroups (seconds),
// stored as the bits of a double so that it can be read without a lock.
std::atomic<unsigned long long> g_wait_bits{0};

double fused_wait_seconds() {
    const unsigned long long b = g_wait_bits.load(std::memory_order_relaxed);
    if (b == 0) return kDefaultWaitSeconds;
    double d;
    memcpy(&d, &b, sizeof d);
    return d;
}

// Ticks of the constant-rate wall clock (wall_clock64) per second, per device.
long long wall_ticks_per_second() {
    static long long cache[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 100000000LL;
    if (cache[dev] == 0) {
        int khz = 0;
        if (hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess ||
            khz <= 0) {
            (void)hipGetLastError();  // do not leave our failed query to the caller
            khz = 100000;
        }
        cache[dev] = (long long)khz * 1000LL;
    }
    return cache[dev];
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

int check_common(int num_segments, int num_rows, int num_adapters, int r, int dtype) {
    if (dtype != SGMV_F32 && dtype != SGMV_F16 && dtype != SGMV_BF16) return SGMV_ERR_BAD_DTYPE;
    if (num_segments < 0 || num_rows < 0 || num_adapters < 0) return SGMV_ERR_BAD_SHAPE;
    if (r < 1 || r > SGMV_MAX_RANK) return SGMV_ERR_BAD_SHAPE;
    return SGMV_OK;
}

// Launch bookkeeping: every launch goes through hipLaunchKernel, whose
// return value describes that launch alone (hipGetLastError could also
// report an older, unrelated error of the caller's).  The first failure of a
// call is kept until launch_status() reads it; the last one stays readable
// through sgmv_last_hip_error().
thread_local hipError_t t_pending = hipSuccess;
thread_local hipError_t t_last = hipSuccess;

template <typename Tuple, size_t... I>
void arg_pointers(Tuple& t, void** out, std::index_sequence<I...>) {
    ((out[I] = (void*)&std::get<I>(t)), ...);
}

template <typename... KArgs, typename... Args>
void launch(void (*kernel)(KArgs...), dim3 grid, dim3 block, hipStream_t st, Args&&... args) {
    static_assert(sizeof...(KArgs) == sizeof...(Args), "argument count mismatch");
    std::tuple<std::decay_t<KArgs>...> vals(static_cast<std::decay_t<KArgs>>(args)...);
    void* ptrs[sizeof...(KArgs) > 0 ? sizeof...(KArgs) : 1];
    arg_pointers(vals, ptrs, std::index_sequence_for<KArgs...>{});
    const hipError_t e = hipLaunchKernel((const void*)kernel, grid, block, ptrs, 0, st);
    if (e != hipSuccess && t_pending == hipSuccess) t_pending = e;
}

int launch_status() {
    const hipError_t e = t_pending;
    t_pending = hipSuccess;
    if (e == hipSuccess) return SGMV_OK;
    t_last = e;
    return SGMV_ERR_HIP;
}

// Whether a call's shrink fits the mixed two-launch form's shrink half, as a
// pure function of the shapes (so that workspace sizes can be queried): ok,
// and k, the largest number of H1 ranges of a class (k > 1: k partial
// planes of [rows][r] floats, reduced into v by each tile's last workgroup
// on the tile counters).
struct MixedShrinkFit {
    bool ok = false;
    int k = 0;
    MixedShape ms{};
    MixedPlan xp{};
};

MixedShrinkFit mixed_shrink_fit(int M, int S, int H1, int r, int dtype) {
    MixedShrinkFit f;
    f.ms = mixed_shape(H1, 8, r, dtype);
    if (!mixed_takes(f.ms, S)) return f;
    f.xp = make_mixed_plan(f.ms, M, S, H1, 8);
    f.k = std::max(std::max(f.xp.two_sp.k[0], f.xp.two_sp.k[1]), f.xp.two_sp.k[2]);
    f.ok = f.xp.ok && (f.k == 1 || f.xp.tiles <= kCounterSlots);
    return f;
}

bool mixed_shrink_aligned(const MixedShrinkFit& f, const void* x, const void* A_stack) {
    return aligned16(A_stack) && (!f.ms.has_long || aligned16(x));
}

// v [rows][r] from the shrink half (partial planes at `part` and the tile
// counters at `counters` when k > 1).
void launch_mixed_shrink(const MixedShrinkFit& f, float* v, float* part, int* counters,
                         const void* x, const void* A_stack, const int32_t* seg_indptr,
                         const int32_t* adapter_ids, int S, int M, int num_adapters, int H1,
                         int r, int dtype, hipStream_t st) {
    const bool in_kernel = f.k > 1;
    with_mixed(dtype, r, [&](auto dt, auto rank, auto lp, auto sp_, auto gp) {
        using DT = decltype(dt);
        using T = typename DT::storage;
        constexpr int R = decltype(rank)::value;
        using LP = decltype(lp);
        using SP = decltype(sp_);
        using GP = decltype(gp);
        launch(&shrink_mixed_kernel<DT, R, LP, SP, GP>, dim3((unsigned)f.xp.grid_shrink),
               dim3(kMixedThreads), st, (const T*)x, (const T*)A_stack, seg_indptr, adapter_ids,
               S, M, num_adapters, H1, in_kernel ? part : v, f.xp.two_sp,
               in_kernel ? v : (float*)nullptr, in_kernel ? counters : (int*)nullptr,
               kCounterStride, (int4*)nullptr, 0);
    });
}


// -- shrink dispatch ---------------------------------------------------------
template <typename DT, int R>
void launch_shrink_vec(float* out, long long out_stride, const void* x, const void* A,
                       const int32_t* seg, const int32_t* ids, int S, int rows, int nad, int H1,
                       const Plan& p, hipStream_t st, float* v_final, int* counters) {
    using T = typename DT::storage;
    const unsigned grid = (unsigned)(tile_slots(S, rows, p.rows) * p.ksplit);
    if (p.rows == 1)
        launch(&shrink_vec_kernel<DT, R, kShrinkThreads, 1, kShrinkPG>, dim3(grid),
               dim3(kShrinkThreads), st, out, out_stride, (const T*)x, (const T*)A, seg, ids, S,
               rows, nad, H1, p.ksplit, p.h_per_split, v_final, counters, kCounterStride);
    else
        launch(&shrink_vec_kernel<DT, R, kShrinkThreads, kShrinkRows, kShrinkPG>, dim3(grid),
               dim3(kShrinkThreads), st, out, out_stride, (const T*)x, (const T*)A, seg, ids, S,
               rows, nad, H1, p.ksplit, p.h_per_split, v_final, counters, kCounterStride);
}

template <typename DT>
void launch_shrink_generic(float* out, long long out_stride, const void* x, const void* A,
                           const int32_t* seg, const int32_t* ids, int S, int rows, int nad,
                           int H1, int r, const Plan& p, hipStream_t st) {
    using T = typename DT::storage;
    const unsigned grid = (unsigned)(tile_slots(S, rows, kGenericRows) * p.ksplit);
    launch(&shrink_generic_kernel<DT, kGenericThreads, kGenericRows>, dim3(grid),
                       dim3(kGenericThreads), st, out, out_stride, (const T*)x, (const T*)A,
                       seg, ids, S, rows, nad, H1, r, p.ksplit, p.h_per_split);
}

// Returns true when the launched kernel also reduced the partials into
// v_final (vectorised kernel, v_final and counters given).
template <typename DT>
bool dispatch_shrink(float* out, long long out_stride, const void* x, const void* A,
                     const int32_t* seg, const int32_t* ids, int S, int rows, int nad, int H1,
                     int r, const Plan& p, hipStream_t st, float* v_final = nullptr,
                     int* counters = nullptr) {
    const bool vec = vec_rank(std::is_same<DT, F32>::value ? SGMV_F32 : SGMV_F16, r) &&
                     aligned16(A);
    auto go = [&](auto rank) {
        constexpr int R = decltype(rank)::value;
        launch_shrink_vec<DT, R>(out, out_stride, x, A, seg, ids, S, rows, nad, H1, p, st,
                                 v_final, counters);
        return v_final != nullptr;
    };
    if (vec) {
        switch (r) {
            case 4:
                if constexpr (DT::kVec == 4) return go(std::integral_constant<int, 4>{});
                break;
            case 8: return go(std::integral_constant<int, 8>{});
            case 16: return go(std::integral_constant<int, 16>{});
            case 32: return go(std::integral_constant<int, 32>{});
            case 64: return go(std::integral_constant<int, 64>{});
            case 128: return go(std::integral_constant<int, 128>{});
            default: break;
        }
    }
    launch_shrink_generic<DT>(out, out_stride, x, A, seg, ids, S, rows, nad, H1, r, p, st);
    return false;
}

// -- expand dispatch ---------------------------------------------------------
template <typename DT, int R>
void launch_expand_vec(void* y, const float* vpart, long long v_stride, int P, const void* B,
                       const int32_t* seg, const int32_t* ids, int S, int rows, int nad, int H2,
                       float scale, const Plan& p, hipStream_t st) {
    using T = typename DT::storage;
    constexpr int KB = R < 16 ? R : 16;
    const int cw = kWave * DT::kVec;
    const int csplit = (H2 + cw - 1) / cw;
    const unsigned grid = (unsigned)(tile_slots(S, rows, kExpandRows) * csplit);
    launch(&expand_vec_kernel<DT, R, kExpandRows, KB>, dim3(grid), dim3(kWave), st, (T*)y, vpart, v_stride, P, (const T*)B, seg, ids, S, rows, nad, H2,
                       scale, csplit);
}

template <typename DT>
void launch_expand_generic(void* y, const float* vpart, long long v_stride, int P, const void* B,
                           const int32_t* seg, const int32_t* ids, int S, int rows, int nad,
                           int r, int H2, float scale, const Plan& p, hipStream_t st) {
    using T = typename DT::storage;
    const int csplit = (H2 + kGenericThreads - 1) / kGenericThreads;
    const unsigned grid = (unsigned)(tile_slots(S, rows, kGenericRows) * csplit);
    launch(&expand_generic_kernel<DT, kGenericThreads, kGenericRows>, dim3(grid),
                       dim3(kGenericThreads), st, (T*)y, vpart, v_stride, P, (const T*)B, seg,
                       ids, S, rows, nad, r, H2, scale, csplit);
}

template <typename DT>
void dispatch_expand(void* y, const float* vpart, long long v_stride, int P, const void* B,
                     const int32_t* seg, const int32_t* ids, int S, int rows, int nad, int r,
                     int H2, float scale, const Plan& p, hipStream_t st) {
    const bool vec = vec_rank(std::is_same<DT, F32>::value ? SGMV_F32 : SGMV_F16, r) &&
                     aligned16(B) && aligned16(y) && (H2 % DT::kVec == 0);
    if (vec) {
        switch (r) {
            case 4:
                if constexpr (DT::kVec == 4) {
                    launch_expand_vec<DT, 4>(y, vpart, v_stride, P, B, seg, ids, S, rows, nad, H2, scale, p, st);
                    return;
                }
                break;
            case 8: launch_expand_vec<DT, 8>(y, vpart, v_stride, P, B, seg, ids, S, rows, nad, H2, scale, p, st); return;
            case 16: launch_expand_vec<DT, 16>(y, vpart, v_stride, P, B, seg, ids, S, rows, nad, H2, scale, p, st); return;
            case 32: launch_expand_vec<DT, 32>(y, vpart, v_stride, P, B, seg, ids, S, rows, nad, H2, scale, p, st); return;
            case 64: launch_expand_vec<DT, 64>(y, vpart, v_stride, P, B, seg, ids, S, rows, nad, H2, scale, p, st); return;
            case 128: launch_expand_vec<DT, 128>(y, vpart, v_stride, P, B, seg, ids, S, rows, nad, H2, scale, p, st); return;
            default: break;
        }
    }
    launch_expand_generic<DT>(y, vpart, v_stride, P, B, seg, ids, S, rows, nad, r, H2, scale, p, st);
}

template <typename F>
void with_dtype(int dtype, F&& f) {
    switch (dtype) {
        case SGMV_F32: f(F32{}); break;
        case SGMV_F16: f(F16{}); break;
        default: f(BF16{}); break;
    }
}

// The expand launch needs the row capacity of the partial buffer to fit the
// grid; both launches index at most num_rows rows.
// Whichever kernel a call ends up on, its grid must fit one launch.  The
// general kernels have the shortest tiles and so the most slots.
bool grid_fits(const Plan& p, int H2) {
    const long long slots = tile_slots(p.num_segments, p.num_rows, 1);  // the most tiles
    const long long csplit = (H2 + kGenericThreads - 1) / kGenericThreads;
    const long long csplit_vec = (H2 + kWave * 4 - 1) / (kWave * 4);
    return slots * p.ksplit <= kMaxGrid && slots * csplit <= kMaxGrid &&
           slots * csplit_vec <= kMaxGrid;
}

// -- adapted linear layer ------------------------------------------------------
// Skinny tiles for decode-sized batches (64 rows: the whole batch, x shared
// by the four waves through LDS, four chunks of loads in flight to stream
// W), square tiles for many rows (each operand read once per 128 rows or
// columns of output).
using LinSkinny = LinearShape<1, 4, 4, 1, 4>;
using LinSquare = LinearShape<2, 2, 4, 4, 2>;
constexpr int kLinTargetWorkgroups = 256;  // split K until the grid has this many
// 256 x 256 tiles (linear_wide_kernel) once they give at least half a tile
// per compute unit, and the segments average at least this many rows (the
// correction runs once per segment a tile overlaps).
constexpr long long kLinWideMinTiles = 128;
constexpr long long kLinWideMinRows = 32;
using LinWide = WideShape<4, 1>;

struct LinearPlan {
    int cfg;  // 0 skinny tiles, 1 square tiles, 2 wide tiles, -1 the element-wise kernel
    int BM, BN;
    long long tiles_m, tiles_n, tiles;
    int ksplit, cps;  // K ranges per tile and chunks of 64 per range
    Plan shrink;      // the per-call shrink launch (its ksplit = v's partials)
    int mix_planes;   // planes the mixed shrink needs (v and its partials), 0 if it does not fit
};

// Pure function of the shapes, so that the workspace size can be queried.
LinearPlan make_linear_plan(int M, int S, int H1, int H2, int r, int dtype) {
    LinearPlan lp{};
    lp.shrink = make_plan(M, S, H1, r, dtype);
    {
        const MixedShrinkFit f = mixed_shrink_fit(M, S, H1, r, dtype);
        lp.mix_planes = f.ok ? (f.k > 1 ? 1 + f.k : 1) : 0;
    }
    lp.cfg = -1;
    lp.ksplit = 1;
    if (dtype == SGMV_F32 || H1 % 8 != 0 || H2 % 8 != 0) return lp;
    lp.cfg = M <= LinSkinny::kBM ? 0 : 1;
    if (lp.cfg == 1) {
        const long long tw =
            (long long)((M + kWideBM - 1) / kWideBM) * ((H2 + kWideBN - 1) / kWideBN);
        if (tw >= kLinWideMinTiles && (long long)S * kLinWideMinRows <= M) {
            lp.cfg = 2;
            lp.BM = kWideBM;
            lp.BN = kWideBN;
            lp.tiles_m = (M + kWideBM - 1) / kWideBM;
            lp.tiles_n = (H2 + kWideBN - 1) / kWideBN;
            lp.tiles = lp.tiles_m * lp.tiles_n;
            lp.cps = (H1 + kLinBK - 1) / kLinBK;
            lp.ksplit = 1;
            return lp;
        }
    }
    lp.BM = lp.cfg == 0 ? LinSkinny::kBM : LinSquare::kBM;
    lp.BN = lp.cfg == 0 ? LinSkinny::kBN : LinSquare::kBN;
    lp.tiles_m = (M + lp.BM - 1) / lp.BM;
    lp.tiles_n = (H2 + lp.BN - 1) / lp.BN;
    lp.tiles = lp.tiles_m * lp.tiles_n;
    const int nk = (H1 + kLinBK - 1) / kLinBK;
    long long k = 1;
    if (lp.tiles < kLinTargetWorkgroups && lp.tiles <= kCounterSlots) {
        k = (kLinTargetWorkgroups + lp.tiles - 1) / lp.tiles;
        const long long kmax = nk / 2 > 1 ? nk / 2 : 1;  // at least two chunks per range
        if (k > kmax) k = kmax;
    }
    lp.cps = (int)((nk + k - 1) / k);
    lp.ksplit = (nk + lp.cps - 1) / lp.cps;
    return lp;
}

size_t linear_v_bytes(const LinearPlan& lp, int M, int r) {
    // the per-call shrink's chunk partials, or (folded) one per K range, or
    // the mixed shrink's v and partials
    const size_t planes = (size_t)std::max<long long>(
        std::max<long long>(lp.shrink.ksplit, lp.ksplit), lp.mix_planes);
    return round256(planes * (size_t)M * (size_t)r * sizeof(float));
}

size_t linear_part_bytes(const LinearPlan& lp) {
    if (lp.cfg < 0 || lp.ksplit <= 1) return 0;
    return (size_t)lp.tiles * (size_t)lp.ksplit * (size_t)lp.BM * (size_t)lp.BN * sizeof(float);
}

template <typename DT, typename SH, bool kFold = false>
void launch_linear_tiled(void* y, const void* x, const void* W, const void* bias, const void* B,
                         const float* vpart, long long vstride, int vsplit, const int32_t* seg,
                         const int32_t* ids, int S, int M, int nad, int H1, int H2, int r,
                         float scale, float* part, int* counters, const LinearPlan& lp,
                         hipStream_t st, const void* A = nullptr, long long wait = -1) {
    using T = typename DT::storage;
    // folded: one shrink workgroup per row and K range ahead of the tiles
    const int n_shrink = kFold ? M * (int)lp.ksplit : 0;
    const unsigned grid = (unsigned)(n_shrink + lp.tiles * lp.ksplit);
    launch(&linear_lora_kernel<DT, SH, kFold>, dim3(grid), dim3(kLinThreads), st, (T*)y,
           (const T*)x, (const T*)W, (const T*)bias, (const T*)B, vpart, vstride, vsplit, seg, ids,
           S, M, nad, H1, H2, r, scale, part, counters, kCounterStride, lp.ksplit, lp.cps,
           (int)lp.tiles_n, (int)lp.tiles, (const T*)A,
           kFold ? counters + lp.tiles * kCounterStride : (int*)nullptr,
           kFold ? counters + kCounterInts - 1 : (int*)nullptr, wait, n_shrink);
}

// Whether lora_linear folds its shrink into the tile launch: decode tiles
// (one row block), an MFMA rank, a rank share that the correction takes in
// one pass, room for the extra counter, and counts that fit its halves
// (shrink workgroups in the low 16 bits, tile workgroups in the rest).
bool linear_folds(const LinearPlan& lp, int M, int S, int r, int dtype) {
    if (lp.cfg != 0 || S < 1 || dtype == SGMV_F32) return false;
    if (r != 16 && r != 32 && r != 64 && r != 128) return false;
    if ((r + lp.ksplit - 1) / lp.ksplit > kLinRG) return false;
    if (lp.tiles + 1 > kCounterSlots) return false;
    return (long long)M * lp.ksplit < (1 << 16) && lp.tiles * lp.ksplit < (1 << 15);
}

// -- scratch of lora_apply_noalloc ------------------------------------------
// A file-scope device array: each GPU the library runs on holds its own copy
// from the moment the library's code is loaded there until the process ends.
// In host code `scratch` names a host-side stand-in, not device memory, so
// host code never passes it to a kernel or a copy: the device address comes
// from hipGetSymbolAddress, once per device, and is kept in g_scratch_ptr.
static __device__ __align__(256) unsigned char scratch[SGMV_NOALLOC_SCRATCH_BYTES];
static_assert(SGMV_NOALLOC_SCRATCH_BYTES > kCounterBytes, "scratch must hold the counters");

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};
bool g_scratch_cleared[kMaxDevices] = {};

__global__ __launch_bounds__(256) void zero_ints_kernel(int* __restrict__ p, int n) {
    const int i = (int)(blockIdx.x * blockDim.x + threadIdx.x);
    if (i < n) p[i] = 0;
}

// The current device's scratch address (looked up on its first use), with
// the counter region cleared by a kernel on `st` at the first call on the
// device that is not being captured (static storage is zero already; this
// makes no assumption about it).  Allocates nothing.
int device_scratch(hipStream_t st, void** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) {
        t_last = e;
        return SGMV_ERR_HIP;
    }
    if (dev < 0 || dev >= kMaxDevices) return SGMV_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p) {
            t_last = e != hipSuccess ? e : hipErrorInvalidSymbol;
            return SGMV_ERR_HIP;
        }
        g_scratch_ptr[dev] = p;
    }
    if (!g_scratch_cleared[dev]) {
        hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
        e = hipStreamIsCapturing(st, &cs);
        if (e != hipSuccess) {
            t_last = e;
            return SGMV_ERR_HIP;
        }
        if (cs == hipStreamCaptureStatusNone) {
            launch(&zero_ints_kernel, dim3((kCounterInts + 255) / 256), dim3(256), st,
                   (int*)g_scratch_ptr[dev], kCounterInts);
            const int rc = launch_status();
            if (rc != SGMV_OK) return rc;
            g_scratch_cleared[dev] = true;
        }
    }
    *out = g_scratch_ptr[dev];
    return SGMV_OK;
}

}  // namespace

extern "C" {

int sgmv_abi_version(void) { return SGMV_ABI_VERSION; }

const char* sgmv_last_hip_error(void) { return hipGetErrorString(t_last); }

const char* sgmv_status_string(int status) {
    switch (status) {
        case SGMV_OK: return "ok";
        case SGMV_ERR_NULL_PTR: return "a required pointer is NULL";
        case SGMV_ERR_BAD_SHAPE: return "invalid size or rank";
        case SGMV_ERR_BAD_DTYPE: return "unknown dtype";
        case SGMV_ERR_UNSUPPORTED: return "sizes exceed what the kernels index";
        case SGMV_ERR_WORKSPACE: return "workspace missing or too small";
        case SGMV_ERR_HIP: return "HIP launch error";
        case SGMV_ERR_BAD_SEGMENTS: return "malformed segment table";
        case SGMV_ERR_SCRATCH:
            return "the call needs more scratch than lora_apply_noalloc holds "
                   "(SGMV_NOALLOC_SCRATCH_BYTES); use lora_apply with a workspace";
        default: return "unknown status";
    }
}

size_t sgmv_shrink_workspace_bytes(int32_t num_rows, int32_t num_segments, int32_t H1, int32_t r,
                                   int32_t dtype) {
    if (check_common(num_segments, num_rows, 0, r, dtype) != SGMV_OK || H1 < 1) return 0;
    const Plan p = make_plan(num_rows, num_segments, H1, r, dtype);
    size_t need = p.ksplit > 1 ? kCounterBytes + partial_bytes(p, num_rows, r) : 0;
    const MixedShape ms = mixed_shape(H1, 8, r, dtype);
    if (mixed_takes(ms, num_segments)) {
        const MixedPlan xp = make_mixed_plan(ms, num_rows, num_segments, H1, 8);
        const int k = std::max(std::max(xp.two_sp.k[0], xp.two_sp.k[1]), xp.two_sp.k[2]);
        if (xp.ok && k > 1 && xp.tiles <= kCounterSlots)
            need = std::max(need, kCounterBytes + (size_t)k * (size_t)num_rows * (size_t)r *
                                                      sizeof(float));
    }
    return need;
}

size_t lora_apply_workspace_bytes(int32_t num_rows, int32_t num_segments, int32_t H1, int32_t H2,
                                  int32_t r, int32_t dtype) {
    if (check_common(num_segments, num_rows, 0, r, dtype) != SGMV_OK || H1 < 1 || H2 < 1) return 0;
    const Plan p = make_plan(num_rows, num_segments, H1, r, dtype);
    const FusedPlan f = make_fused_plan(num_rows, num_segments, H1, H2, r, dtype);
    const MfmaPlan mp = make_mfma_plan(num_rows, num_segments, H1, H2, r, dtype);
    int k = p.ksplit;
    if (f.ok && f.ksplit > k) k = f.ksplit;
    if (mp.ok && mp.ksplit > k) k = mp.ksplit;
    const MfmaSplitPlan sp = make_mfma_split_plan(mp, H1, H2, r);
    if (sp.ok && sp.ksplit > k) k = sp.ksplit;
    const MixedShape ms = mixed_shape(H1, H2, r, dtype);
    size_t table = 0;
    if (mixed_takes(ms, num_segments)) {
        const MixedPlan xp = make_mixed_plan(ms, num_rows, num_segments, H1, H2);
        if (xp.ok && xp.kmax > k) k = xp.kmax;
        if (xp.ok && xp.two) table = mixed_table_end(xp, num_rows, r);
    }
    return std::max(table, kCounterBytes + (size_t)k * (size_t)num_rows * (size_t)r * sizeof(float));
}

int sgmv_shrink(float* v, const void* x, const void* A_stack, const int32_t* seg_indptr,
                const int32_t* adapter_ids, int32_t num_segments, int32_t num_rows,
                int32_t num_adapters, int32_t H1, int32_t r, int32_t dtype, void* workspace,
                size_t workspace_bytes, void* stream) {
    int rc = check_common(num_segments, num_rows, num_adapters, r, dtype);
    if (rc != SGMV_OK) return rc;
    if (H1 < 1) return SGMV_ERR_BAD_SHAPE;
    if (num_rows == 0 || num_segments == 0) return SGMV_OK;
    if (!v || !x || !A_stack || !seg_indptr || !adapter_ids) return SGMV_ERR_NULL_PTR;
    const Plan p = make_plan(num_rows, num_segments, H1, r, dtype);
    if (!grid_fits(p, 1)) return SGMV_ERR_UNSUPPORTED;
    const size_t need = p.ksplit > 1 ? kCounterBytes + partial_bytes(p, num_rows, r) : 0;
    if (need > 0 && (!workspace || workspace_bytes < need)) return SGMV_ERR_WORKSPACE;
    hipStream_t st = (hipStream_t)stream;
    // The path chosen per segment (sgmv_mixed.hpp), the shrink half of the
    // two-launch form.  With a split H1, each tile's last workgroup reduces
    // the partials into v in-kernel (tile counters at the start of the
    // workspace); calls whose tiles could outnumber the counters keep the
    // per-call kernels.
    {
        const MixedShrinkFit f = mixed_shrink_fit(num_rows, num_segments, H1, r, dtype);
        if (f.ok && mixed_shrink_aligned(f, x, A_stack)) {
            const size_t need_m = f.k > 1 ? kCounterBytes + (size_t)f.k * (size_t)num_rows *
                                                                (size_t)r * sizeof(float)
                                          : 0;
            if (need_m > 0 && (!workspace || workspace_bytes < need_m)) return SGMV_ERR_WORKSPACE;
            launch_mixed_shrink(f, v, f.k > 1 ? (float*)((char*)workspace + kCounterBytes) : v,
                                (int*)workspace, x, A_stack, seg_indptr, adapter_ids,
                                num_segments, num_rows, num_adapters, H1, r, dtype, st);
            return launch_status();
        }
    }
    float* out = p.ksplit > 1 ? (float*)((char*)workspace + kCounterBytes) : v;
    const long long stride = (long long)num_rows * r;
    // Row-heavy calls: 16-row MFMA tiles over the same H1 ranges (each
    // workgroup sums its range's LDS-sized chunks in order), so the
    // workspace is the same as for the vector kernel.
    const MfmaPlan mp = make_mfma_plan(num_rows, num_segments, H1, 8, r, dtype);
    const long long mslots = mp.slots_a + mp.slots_b;
    bool reduced = false;
    if (mslots > 0 && aligned16(x) && aligned16(A_stack) && use_mfma(num_rows, num_segments) &&
        mslots * p.ksplit <= kMaxGrid) {
        // A split is reduced in-kernel when the tiles fit the counters.
        const bool in_kernel = p.ksplit > 1 && mslots <= kCounterSlots;
        with_mfma_rank(dtype, r, [&](auto dt, auto rank) {
            using DT = decltype(dt);
            using T = typename DT::storage;
            constexpr int R = decltype(rank)::value;
            launch(&shrink_mfma_kernel<DT, R>, dim3((unsigned)(mslots * p.ksplit)), dim3(256), st,
                   (const T*)x, (const T*)A_stack, seg_indptr, adapter_ids, num_segments,
                   num_rows, num_adapters, H1, out, p.ksplit, p.h_per_split, mp.compact,
                   in_kernel ? v : nullptr, in_kernel ? (int*)workspace : nullptr,
                   kCounterStride);
        });
        reduced = in_kernel;
    } else {
        // With a split, the tile's last workgroup reduces the partials into v
        // (tile counters at the start of the workspace) when the tiles fit
        // the counters; otherwise (or after the general kernel) a reduction
        // launch follows.  The plan splits only below 512 tile slots, so for
        // the vectorised kernel the tiles always fit.
        const bool in_kernel =
            p.ksplit > 1 && tile_slots(num_segments, num_rows, p.rows) <= kCounterSlots;
        with_dtype(dtype, [&](auto dt) {
            using DT = decltype(dt);
            reduced = dispatch_shrink<DT>(out, stride, x, A_stack, seg_indptr, adapter_ids,
                                          num_segments, num_rows, num_adapters, H1, r, p, st,
                                          in_kernel ? v : nullptr,
                                          in_kernel ? (int*)workspace : nullptr);
        });
    }
    if ((rc = launch_status()) != SGMV_OK) return rc;
    if (p.ksplit > 1 && !reduced) {
        const long long n = stride;
        const unsigned grid = (unsigned)((n + 255) / 256);
        launch(&reduce_partials_kernel, dim3(grid), dim3(256), st, v, out, stride,
                           p.ksplit, seg_indptr, adapter_ids, num_segments, num_rows,
                           num_adapters, r);
        rc = launch_status();
    }
    return rc;
}

int sgmv_expand(void* y, const float* v, const void* B_stack, const int32_t* seg_indptr,
                const int32_t* adapter_ids, int32_t num_segments, int32_t num_rows,
                int32_t num_adapters, int32_t r, int32_t H2, float scale, int32_t dtype,
                void* stream) {
    int rc = check_common(num_segments, num_rows, num_adapters, r, dtype);
    if (rc != SGMV_OK) return rc;
    if (H2 < 1) return SGMV_ERR_BAD_SHAPE;
    if (num_rows == 0 || num_segments == 0) return SGMV_OK;
    if (!y || !v || !B_stack || !seg_indptr || !adapter_ids) return SGMV_ERR_NULL_PTR;
    const Plan p = make_plan(num_rows, num_segments, 1, r, dtype);
    if (!grid_fits(p, H2)) return SGMV_ERR_UNSUPPORTED;
    hipStream_t st = (hipStream_t)stream;
    // The path chosen per segment (sgmv_mixed.hpp), the expand half of the
    // two-launch form, v read as the single partial of every row.
    {
        const MixedShape ms = mixed_shape(8, H2, r, dtype);
        if (mixed_takes(ms, num_segments) && aligned16(B_stack) && aligned16(y)) {
            const MixedPlan xp = make_mixed_plan(ms, num_rows, num_segments, 8, H2);
            if (xp.ok) {
                with_mixed(dtype, r, [&](auto dt, auto rank, auto lp, auto sp_, auto gp) {
                    using DT = decltype(dt);
                    using T = typename DT::storage;
                    constexpr int R = decltype(rank)::value;
                    using LP = decltype(lp);
                    using SP = decltype(sp_);
                    (void)gp;
                    launch(&expand_mixed_kernel<DT, R, LP, SP, SplitSingle<DT, R>>, dim3((unsigned)xp.grid_expand),
                           dim3(kMixedThreads), st, (T*)y, (const T*)B_stack, seg_indptr,
                           adapter_ids, num_segments, num_rows, num_adapters, H2, scale, v,
                           xp.two_sp, 1, 1, 1, (const int4*)nullptr, 0);
                });
                return launch_status();
            }
        }
    }
    // Row-heavy calls: 16-row MFMA tiles, v read as the single "partial".
    const MfmaPlan mp = make_mfma_plan(num_rows, num_segments, 8, H2, r, dtype);
    const long long mslots = mp.slots_a + mp.slots_b;
    if (mslots > 0 && aligned16(y) && aligned16(B_stack) && use_mfma(num_rows, num_segments) &&
        mslots * mp.csplit <= kMaxGrid) {
        with_mfma_rank(dtype, r, [&](auto dt, auto rank) {
            using DT = decltype(dt);
            using T = typename DT::storage;
            constexpr int R = decltype(rank)::value;
            launch(&expand_mfma_kernel<DT, R>, dim3((unsigned)(mslots * mp.csplit)), dim3(256), st,
                   (T*)y, (const T*)B_stack, seg_indptr, adapter_ids, num_segments, num_rows,
                   num_adapters, H2, scale, v, 1, mp.csplit, mp.compact);
        });
        return launch_status();
    }
    with_dtype(dtype, [&](auto dt) {
        using DT = decltype(dt);
        dispatch_expand<DT>(y, v, 0, 1, B_stack, seg_indptr, adapter_ids, num_segments, num_rows,
                            num_adapters, r, H2, scale, p, st);
    });
    return launch_status();
}

int lora_apply(void* y, const void* x, const void* A_stack, const void* B_stack,
               const int32_t* seg_indptr, const int32_t* adapter_ids, int32_t num_segments,
               int32_t num_rows, int32_t num_adapters, int32_t H1, int32_t H2, int32_t r,
               float scale, int32_t dtype, void* workspace, size_t workspace_bytes,
               void* stream) {
    int rc = check_common(num_segments, num_rows, num_adapters, r, dtype);
    if (rc != SGMV_OK) return rc;
    if (H1 < 1 || H2 < 1) return SGMV_ERR_BAD_SHAPE;
    if (num_rows == 0 || num_segments == 0) return SGMV_OK;
    if (!y || !x || !A_stack || !B_stack || !seg_indptr || !adapter_ids) return SGMV_ERR_NULL_PTR;
    const Plan p = make_plan(num_rows, num_segments, H1, r, dtype);
    if (!grid_fits(p, H2)) return SGMV_ERR_UNSUPPORTED;
    const size_t need = lora_apply_workspace_bytes(num_rows, num_segments, H1, H2, r, dtype);
    if (!workspace || workspace_bytes < need) return SGMV_ERR_WORKSPACE;
    hipStream_t st = (hipStream_t)stream;
    int* counters = (int*)workspace;
    float* part = (float*)((char*)workspace + kCounterBytes);
    const long long stride = (long long)num_rows * r;
    const int vec = vec_width(dtype);
    const bool aligned = aligned16(A_stack) && aligned16(B_stack) && aligned16(y);
    const double wait_s = fused_wait_seconds();
    const long long wait =
        wait_s < 1e-300 ? -1 : (long long)(wait_s * (double)wall_ticks_per_second());
    // The path chosen per segment (sgmv_mixed.hpp): one launch, or a shrink
    // launch and an expand launch for calls beyond two resident rounds.
    {
        const MixedShape ms = mixed_shape(H1, H2, r, dtype);
        if (mixed_takes(ms, num_segments) && aligned && (!ms.has_long || aligned16(x))) {
            const MixedPlan xp = make_mixed_plan(ms, num_rows, num_segments, H1, H2);
            if (xp.ok) {
                with_mixed(dtype, r, [&](auto dt, auto rank, auto lp, auto sp_, auto gp) {
                    using DT = decltype(dt);
                    using T = typename DT::storage;
                    constexpr int R = decltype(rank)::value;
                    using LP = decltype(lp);
                    using SP = decltype(sp_);
                    using GP = decltype(gp);
                    if (!xp.two) {
                        // as many rows as segments: guess one row per
                        // segment; one segment: guess it covers every row
                        const int guess =
                            num_rows == num_segments ? 1 : (num_segments == 1 ? 2 : 0);
                        launch(&lora_mixed_kernel<DT, R, LP, SP, GP>, dim3((unsigned)xp.grid_one),
                               dim3(kMixedThreads), st, (T*)y, (const T*)x, (const T*)A_stack,
                               (const T*)B_stack, seg_indptr, adapter_ids, num_segments, num_rows,
                               num_adapters, H1, H2, scale, part, counters, xp.one, kCounterInts,
                               kCounterStride, wait, guess);
                        return;
                    }
                    // the shrink launch writes the expand launch's items
                    int4* items = (int4*)((char*)workspace + mixed_table_offset(xp, num_rows, r));
                    const int n_items = (int)xp.grid_expand;
                    launch(&shrink_mixed_kernel<DT, R, LP, SP, GP>, dim3((unsigned)xp.grid_shrink),
                           dim3(kMixedThreads), st, (const T*)x, (const T*)A_stack, seg_indptr,
                           adapter_ids, num_segments, num_rows, num_adapters, H1, part,
                           xp.two_sp, (float*)nullptr, (int*)nullptr, 0, items, n_items);
                    if (t_pending != hipSuccess) return;  // no expand over unwritten partials
                    launch(&expand_mixed_kernel<DT, R, LP, SP, SplitSingle<DT, R>>, dim3((unsigned)xp.grid_expand),
                           dim3(kMixedThreads), st, (T*)y, (const T*)B_stack, seg_indptr,
                           adapter_ids, num_segments, num_rows, num_adapters, H2, scale,
                           (const float*)part, xp.two_sp, xp.two_sp.k[0], xp.two_sp.k[1],
                           xp.two_sp.k[2], (const int4*)items, n_items);
                });
                return launch_status();
            }
        }
    }
    const MfmaPlan mp = make_mfma_plan(num_rows, num_segments, H1, H2, r, dtype);
    if (mp.ok && aligned && aligned16(x) && use_mfma(num_rows, num_segments)) {
        const MfmaSplitPlan sp = make_mfma_split_plan(mp, H1, H2, r);
        auto go = [&](auto dt, auto rank) {
            using DT = decltype(dt);
            using T = typename DT::storage;
            constexpr int R = decltype(rank)::value;
            if (sp.ok) {
                launch(&shrink_mfma_kernel<DT, R>, dim3((unsigned)sp.grid_shrink), dim3(256), st,
                       (const T*)x, (const T*)A_stack, seg_indptr, adapter_ids, num_segments,
                       num_rows, num_adapters, H1, part, sp.ksplit, sp.h_per_split, sp.compact,
                       (float*)nullptr, (int*)nullptr, 0);
                if (t_pending != hipSuccess) return;  // no expand over partials never written
                launch(&expand_mfma_kernel<DT, R>, dim3((unsigned)sp.grid_expand), dim3(256), st,
                       (T*)y, (const T*)B_stack, seg_indptr, adapter_ids, num_segments, num_rows,
                       num_adapters, H2, scale, (const float*)part, sp.ksplit, sp.csplit,
                       sp.compact);
                return;
            }
            launch(&lora_mfma_kernel<DT, R>, dim3((unsigned)mp.grid), dim3(256), st, (T*)y,
                   (const T*)x, (const T*)A_stack, (const T*)B_stack, seg_indptr, adapter_ids,
                   num_segments, num_rows, num_adapters, H1, H2, scale, part, counters,
                   mp.ksplit, mp.h_per_split, mp.csplit, (int)mp.slots_a, (int)mp.slots_b,
                   mp.compact, kCounterInts, kCounterStride, wait);
        };
        auto by_rank = [&](auto dt) {
            switch (r) {
                case 16: go(dt, std::integral_constant<int, 16>{}); break;
                case 32: go(dt, std::integral_constant<int, 32>{}); break;
                case 64: go(dt, std::integral_constant<int, 64>{}); break;
                default: go(dt, std::integral_constant<int, 128>{}); break;
            }
        };
        if (dtype == SGMV_F16) by_rank(F16{});
        else by_rank(BF16{});
        return launch_status();
    }
    const FusedPlan f = make_fused_plan(num_rows, num_segments, H1, H2, r, dtype);
    const bool fused = f.ok && aligned && (H2 % vec == 0);
    if (fused) {
        with_dtype(dtype, [&](auto dt) {
            using DT = decltype(dt);
            using T = typename DT::storage;
            auto go = [&](auto rank, auto rows) {
                constexpr int R = decltype(rank)::value;
                constexpr int RB = decltype(rows)::value;
                constexpr int KB = R < 16 ? R : 16;
                launch(&lora_fused_kernel<DT, R, kFusedThreads, RB, kFusedPG, KB>,
                       dim3((unsigned)f.grid), dim3(kFusedThreads), st, (T*)y, (const T*)x,
                       (const T*)A_stack, (const T*)B_stack, seg_indptr, adapter_ids,
                       num_segments, num_rows, num_adapters, H1, H2, scale, part, counters,
                       f.ksplit, f.h_per_split, f.csplit, (int)f.slots_a, (int)f.slots_b,
                       f.compact, kCounterInts, kCounterStride, wait);
            };
            auto by_rows = [&](auto rank) {
                if (f.rows == 1) go(rank, std::integral_constant<int, 1>{});
                else go(rank, std::integral_constant<int, 4>{});
            };
            switch (r) {
                case 4:
                    if constexpr (DT::kVec == 4) by_rows(std::integral_constant<int, 4>{});
                    break;
                case 8: by_rows(std::integral_constant<int, 8>{}); break;
                case 16: by_rows(std::integral_constant<int, 16>{}); break;
                case 32: by_rows(std::integral_constant<int, 32>{}); break;
                case 64: by_rows(std::integral_constant<int, 64>{}); break;
                default: by_rows(std::integral_constant<int, 128>{}); break;
            }
        });
        return launch_status();
    }
    with_dtype(dtype, [&](auto dt) {
        using DT = decltype(dt);
        dispatch_shrink<DT>(part, stride, x, A_stack, seg_indptr, adapter_ids, num_segments,
                            num_rows, num_adapters, H1, r, p, st);
    });
    if ((rc = launch_status()) != SGMV_OK) return rc;
    with_dtype(dtype, [&](auto dt) {
        using DT = decltype(dt);
        dispatch_expand<DT>(y, part, stride, p.ksplit, B_stack, seg_indptr, adapter_ids,
                            num_segments, num_rows, num_adapters, r, H2, scale, p, st);
    });
    return launch_status();
}

int lora_apply_noalloc(void* y, const void* x, const void* A_stack, const void* B_stack,
                       const int32_t* seg_indptr, const int32_t* adapter_ids,
                       int32_t num_segments, int32_t num_rows, int32_t num_adapters, int32_t H1,
                       int32_t H2, int32_t r, float scale, int32_t dtype, void* stream) {
    // lora_apply's checks, in its order, before the scratch is touched.
    int rc = check_common(num_segments, num_rows, num_adapters, r, dtype);
    if (rc != SGMV_OK) return rc;
    if (H1 < 1 || H2 < 1) return SGMV_ERR_BAD_SHAPE;
    if (num_rows == 0 || num_segments == 0) return SGMV_OK;
    if (!y || !x || !A_stack || !B_stack || !seg_indptr || !adapter_ids) return SGMV_ERR_NULL_PTR;
    const size_t need = lora_apply_workspace_bytes(num_rows, num_segments, H1, H2, r, dtype);
    if (need > (size_t)SGMV_NOALLOC_SCRATCH_BYTES) return SGMV_ERR_SCRATCH;
    void* ws = nullptr;
    if ((rc = device_scratch((hipStream_t)stream, &ws)) != SGMV_OK) return rc;
    return lora_apply(y, x, A_stack, B_stack, seg_indptr, adapter_ids, num_segments, num_rows,
                      num_adapters, H1, H2, r, scale, dtype, ws,
                      (size_t)SGMV_NOALLOC_SCRATCH_BYTES, stream);
}

// -- several add-ons in one launch ------------------------------------------

static_assert(kMaxProblems == SGMV_MAX_PROBLEMS, "problem limit mismatch");
static_assert(sizeof(sgmv_lora_problem) == 48, "sgmv_lora_problem layout");

namespace {

// Plans of the problems of one lora_apply_multi call, or ok = false when the
// single-launch form does not apply (then each problem runs on its own).
struct MultiPlan {
    bool ok;
    FusedPlan f[kMaxProblems];
    size_t partial_off[kMaxProblems + 1];  // in floats, after the counter region
};

MultiPlan make_multi_plan(const sgmv_lora_problem* pr, int P, int num_rows, int num_segments,
                          int r, int dtype) {
    MultiPlan m{};
    if (P < 1 || P > kMaxProblems || num_segments > kCompactMaxSegments) return m;
    // Two resident rounds of items in all: smaller items per problem than one
    // round would allow, whose loads are in flight together (measured best
    // for 2 and 4 decode projections; equal for 8).
    const long long budget = 2 * kFusedItems / P > 64 ? 2 * kFusedItems / P : 64;
    long long slots_total = 0;
    m.partial_off[0] = 0;
    for (int p = 0; p < P; ++p) {
        m.f[p] = make_fused_plan(num_rows, num_segments, pr[p].H1, pr[p].H2, r, dtype, budget);
        if (!m.f[p].ok || m.f[p].rows != m.f[0].rows) return m;
        slots_total += m.f[p].slots_a;
        m.partial_off[p + 1] =
            m.partial_off[p] + (size_t)m.f[p].ksplit * (size_t)num_rows * (size_t)r;
    }
    long long items = 0;
    for (int p = 0; p < P; ++p) items += m.f[p].grid;
    m.ok = slots_total <= kCounterSlots && items <= kMaxGrid;
    return m;
}

bool problem_fits_fused(const sgmv_lora_problem& q, int dtype) {
    return aligned16(q.A_stack) && aligned16(q.B_stack) && aligned16(q.y) &&
           q.H2 % vec_width(dtype) == 0;
}

}  // namespace

size_t lora_apply_multi_workspace_bytes(const sgmv_lora_problem* problems, int32_t num_problems,
                                        int32_t num_rows, int32_t num_segments, int32_t r,
                                        int32_t dtype) {
    if (!problems || num_problems < 1 || num_problems > SGMV_MAX_PROBLEMS) return 0;
    if (check_common(num_segments, num_rows, 0, r, dtype) != SGMV_OK) return 0;
    size_t need = 0;
    for (int p = 0; p < num_problems; ++p) {
        const size_t one = lora_apply_workspace_bytes(num_rows, num_segments, problems[p].H1,
                                                      problems[p].H2, r, dtype);
        if (one == 0) return 0;
        if (one > need) need = one;
    }
    const MultiPlan m = make_multi_plan(problems, num_problems, num_rows, num_segments, r, dtype);
    if (m.ok) {
        const size_t multi = kCounterBytes + m.partial_off[num_problems] * sizeof(float);
        if (multi > need) need = multi;
    }
    return need;
}

int lora_apply_multi(const sgmv_lora_problem* problems, int32_t num_problems,
                     const int32_t* seg_indptr, const int32_t* adapter_ids, int32_t num_segments,
                     int32_t num_rows, int32_t num_adapters, int32_t r, int32_t dtype,
                     void* workspace, size_t workspace_bytes, void* stream) {
    if (!problems) return SGMV_ERR_NULL_PTR;
    if (num_problems < 1 || num_problems > SGMV_MAX_PROBLEMS) return SGMV_ERR_BAD_SHAPE;
    int rc = check_common(num_segments, num_rows, num_adapters, r, dtype);
    if (rc != SGMV_OK) return rc;
    for (int p = 0; p < num_problems; ++p) {
        const sgmv_lora_problem& q = problems[p];
        if (q.H1 < 1 || q.H2 < 1) return SGMV_ERR_BAD_SHAPE;
        if (num_rows > 0 && num_segments > 0 && (!q.y || !q.x || !q.A_stack || !q.B_stack))
            return SGMV_ERR_NULL_PTR;
    }
    if (num_rows == 0 || num_segments == 0) return SGMV_OK;
    if (!seg_indptr || !adapter_ids) return SGMV_ERR_NULL_PTR;
    const size_t need = lora_apply_multi_workspace_bytes(problems, num_problems, num_rows,
                                                         num_segments, r, dtype);
    if (need == 0) return SGMV_ERR_UNSUPPORTED;
    if (!workspace || workspace_bytes < need) return SGMV_ERR_WORKSPACE;

    const MultiPlan m = make_multi_plan(problems, num_problems, num_rows, num_segments, r, dtype);
    bool one_launch = m.ok;
    for (int p = 0; p < num_problems && one_launch; ++p)
        one_launch = problem_fits_fused(problems[p], dtype) &&
                     !use_mfma(num_rows, num_segments);
    if (!one_launch) {
        // One call per problem, in order, each with the whole workspace.
        for (int p = 0; p < num_problems; ++p) {
            const sgmv_lora_problem& q = problems[p];
            rc = lora_apply(q.y, q.x, q.A_stack, q.B_stack, seg_indptr, adapter_ids, num_segments,
                            num_rows, num_adapters, q.H1, q.H2, r, q.scale, dtype, workspace,
                            workspace_bytes, stream);
            if (rc != SGMV_OK) return rc;
        }
        return SGMV_OK;
    }

    hipStream_t st = (hipStream_t)stream;
    int* counters = (int*)workspace;
    float* part = (float*)((char*)workspace + kCounterBytes);
    const double wait_s = fused_wait_seconds();
    const long long wait =
        wait_s < 1e-300 ? -1 : (long long)(wait_s * (double)wall_ticks_per_second());
    const FusedPlan& f0 = m.f[0];
    with_dtype(dtype, [&](auto dt) {
        using DT = decltype(dt);
        using T = typename DT::storage;
        MultiProblems<T> P{};
        P.num = num_problems;
        long long next_counter = 0, next_item = 0;
        for (int p = 0; p < num_problems; ++p) {
            const sgmv_lora_problem& q = problems[p];
            const FusedPlan& f = m.f[p];
            P.y[p] = (T*)q.y;
            P.x[p] = (const T*)q.x;
            P.A[p] = (const T*)q.A_stack;
            P.B[p] = (const T*)q.B_stack;
            P.partials[p] = part + m.partial_off[p];
            P.counters[p] = counters + next_counter * kCounterStride;
            next_counter += f.slots_a;
            P.H1[p] = q.H1;
            P.H2[p] = q.H2;
            P.ksplit[p] = f.ksplit;
            P.h_per_split[p] = f.h_per_split;
            P.csplit[p] = f.csplit;
            P.scale[p] = q.scale;
            P.sbase[p] = next_item;
            next_item += f.slots_a * f.ksplit;
        }
        P.sbase[num_problems] = next_item;
        for (int p = 0; p < num_problems; ++p) {
            P.ebase[p] = next_item;
            next_item += m.f[p].slots_a * m.f[p].csplit;
        }
        P.ebase[num_problems] = next_item;
        auto go = [&](auto rank, auto rows) {
            constexpr int R = decltype(rank)::value;
            constexpr int RB = decltype(rows)::value;
            constexpr int KB = R < 16 ? R : 16;
            launch(&lora_fused_multi_kernel<DT, R, kFusedThreads, RB, kFusedPG, KB>,
                   dim3((unsigned)next_item), dim3(kFusedThreads), st, P, seg_indptr,
                   adapter_ids, num_segments, num_rows, num_adapters, f0.compact,
                   &counters[kCounterInts - 1], kCounterStride, wait);
        };
        auto by_rows = [&](auto rank) {
            if (f0.rows == 1) go(rank, std::integral_constant<int, 1>{});
            else go(rank, std::integral_constant<int, 4>{});
        };
        switch (r) {
            case 4:
                if constexpr (DT::kVec == 4) by_rows(std::integral_constant<int, 4>{});
                break;
            case 8: by_rows(std::integral_constant<int, 8>{}); break;
            case 16: by_rows(std::integral_constant<int, 16>{}); break;
            case 32: by_rows(std::integral_constant<int, 32>{}); break;
            case 64: by_rows(std::integral_constant<int, 64>{}); break;
            default: by_rows(std::integral_constant<int, 128>{}); break;
        }
    });
    return launch_status();
}

int sgmv_load_adapter(void* A_stack, void* B_stack, int32_t slot, int32_t count,
                      int32_t num_adapters, const void* h_A, const void* h_B, int32_t H1,
                      int32_t H2, int32_t r, int32_t dtype, void* stream) {
    if (dtype != SGMV_F32 && dtype != SGMV_F16 && dtype != SGMV_BF16) return SGMV_ERR_BAD_DTYPE;
    if (H1 < 1 || H2 < 1 || r < 1 || r > SGMV_MAX_RANK || num_adapters < 1 || slot < 0 ||
        count < 1 || (long long)slot + count > num_adapters)
        return SGMV_ERR_BAD_SHAPE;
    if (!A_stack || !B_stack || !h_A || !h_B) return SGMV_ERR_NULL_PTR;
    const size_t e = (size_t)elem_bytes(dtype);
    const size_t a_bytes = (size_t)H1 * (size_t)r * e;  // one adapter
    const size_t b_bytes = (size_t)r * (size_t)H2 * e;
    hipStream_t st = (hipStream_t)stream;
    hipError_t err = hipMemcpyAsync((char*)A_stack + (size_t)slot * a_bytes, h_A,
                                    a_bytes * (size_t)count, hipMemcpyHostToDevice, st);
    if (err == hipSuccess)
        err = hipMemcpyAsync((char*)B_stack + (size_t)slot * b_bytes, h_B,
                             b_bytes * (size_t)count, hipMemcpyHostToDevice, st);
    if (err != hipSuccess) {
        t_last = err;
        return SGMV_ERR_HIP;
    }
    return SGMV_OK;
}

size_t lora_linear_workspace_bytes(int32_t num_rows, int32_t num_segments, int32_t H1, int32_t H2,
                                   int32_t r, int32_t dtype) {
    if (check_common(num_segments, num_rows, 0, r, dtype) != SGMV_OK || H1 < 1 || H2 < 1) return 0;
    const LinearPlan lp = make_linear_plan(num_rows, num_segments, H1, H2, r, dtype);
    return kCounterBytes + linear_v_bytes(lp, num_rows, r) + linear_part_bytes(lp);
}

int lora_linear(void* y, const void* x, const void* W, const void* bias, const void* A_stack,
                const void* B_stack, const int32_t* seg_indptr, const int32_t* adapter_ids,
                int32_t num_segments, int32_t num_rows, int32_t num_adapters, int32_t H1,
                int32_t H2, int32_t r, float scale, int32_t dtype, void* workspace,
                size_t workspace_bytes, void* stream) {
    int rc = check_common(num_segments, num_rows, num_adapters, r, dtype);
    if (rc != SGMV_OK) return rc;
    if (H1 < 1 || H2 < 1) return SGMV_ERR_BAD_SHAPE;
    if (num_rows == 0) return SGMV_OK;
    if (!y || !x || !W) return SGMV_ERR_NULL_PTR;
    if (num_segments > 0 && (!A_stack || !B_stack || !seg_indptr || !adapter_ids))
        return SGMV_ERR_NULL_PTR;
    const LinearPlan lp = make_linear_plan(num_rows, num_segments, H1, H2, r, dtype);
    if (num_segments > 0 && !grid_fits(lp.shrink, 1)) return SGMV_ERR_UNSUPPORTED;
    if (lp.cfg >= 0 ? lp.tiles * lp.ksplit > kMaxGrid
                    : ((long long)num_rows * H2 + 255) / 256 > kMaxGrid)
        return SGMV_ERR_UNSUPPORTED;
    const size_t need = lora_linear_workspace_bytes(num_rows, num_segments, H1, H2, r, dtype);
    if (!workspace || workspace_bytes < need) return SGMV_ERR_WORKSPACE;
    hipStream_t st = (hipStream_t)stream;
    int* counters = (int*)workspace;
    float* vpart = (float*)((char*)workspace + kCounterBytes);
    float* part = (float*)((char*)vpart + linear_v_bytes(lp, num_rows, r));
    const long long vstride = (long long)num_rows * r;
    const bool tiled = lp.cfg >= 0 && aligned16(x) && aligned16(W) && aligned16(y) &&
                       aligned16(B_stack) && aligned16(bias);
    // Decode tiles fold the shrink into their own launch (linear_lora_kernel).
    const bool fold =
        tiled && aligned16(A_stack) && linear_folds(lp, num_rows, num_segments, r, dtype);
    int vsplit = fold ? lp.ksplit : lp.shrink.ksplit;
    const double wait_s = fused_wait_seconds();
    const long long wait =
        wait_s < 1e-300 ? -1 : (long long)(wait_s * (double)wall_ticks_per_second());
    // The shrink: the mixed two-launch form's shrink half when it fits (v
    // finished in plane 0, its partials after it; the tile counters it uses
    // return to zero), else the per-call kernels' chunk partials.
    const MixedShrinkFit mf = num_segments > 0 && !fold && lp.mix_planes > 0
                                  ? mixed_shrink_fit(num_rows, num_segments, H1, r, dtype)
                                  : MixedShrinkFit{};
    if (mf.ok && mixed_shrink_aligned(mf, x, A_stack)) {
        launch_mixed_shrink(mf, vpart, vpart + vstride, counters, x, A_stack, seg_indptr,
                            adapter_ids, num_segments, num_rows, num_adapters, H1, r, dtype, st);
        if ((rc = launch_status()) != SGMV_OK) return rc;
        vsplit = 1;
    } else if (num_segments > 0 && !fold) {
        with_dtype(dtype, [&](auto dt) {
            using DT = decltype(dt);
            dispatch_shrink<DT>(vpart, vstride, x, A_stack, seg_indptr, adapter_ids, num_segments,
                                num_rows, num_adapters, H1, r, lp.shrink, st);
        });
        if ((rc = launch_status()) != SGMV_OK) return rc;
    }
    with_dtype(dtype, [&](auto dt) {
        using DT = decltype(dt);
        using T = typename DT::storage;
        if constexpr (!std::is_same<DT, F32>::value) {
            if (fold) {
                launch_linear_tiled<DT, LinSkinny, true>(
                    y, x, W, bias, B_stack, vpart, vstride, vsplit, seg_indptr, adapter_ids,
                    num_segments, num_rows, num_adapters, H1, H2, r, scale, part, counters, lp,
                    st, A_stack, wait);
                return;
            }
            if (tiled) {
                if (lp.cfg == 2) {
                    // direct global-to-LDS stages when K is whole steps of 4 x 32
                    auto k = H1 % 128 == 0 ? &linear_wide_kernel<DT, LinWide, true>
                                           : &linear_wide_kernel<DT, LinWide, false>;
                    launch(k, dim3((unsigned)lp.tiles), dim3(LinWide::kNT), st, (T*)y,
                           (const T*)x, (const T*)W, (const T*)bias, (const T*)B_stack,
                           (const float*)vpart, vstride, vsplit, seg_indptr, adapter_ids,
                           num_segments, num_rows, num_adapters, H1, H2, r, scale,
                           (int)lp.tiles_n, (int)lp.tiles);
                }
                else if (lp.cfg == 0)
                    launch_linear_tiled<DT, LinSkinny>(y, x, W, bias, B_stack, vpart, vstride,
                                                       vsplit, seg_indptr, adapter_ids,
                                                       num_segments, num_rows, num_adapters, H1,
                                                       H2, r, scale, part, counters, lp, st);
                else
                    launch_linear_tiled<DT, LinSquare>(y, x, W, bias, B_stack, vpart, vstride,
                                                       vsplit, seg_indptr, adapter_ids,
                                                       num_segments, num_rows, num_adapters, H1,
                                                       H2, r, scale, part, counters, lp, st);
                return;
            }
        }
        const unsigned grid = (unsigned)(((long long)num_rows * H2 + 255) / 256);
        launch(&linear_lora_generic_kernel<DT>, dim3(grid), dim3(256), st, (T*)y, (const T*)x,
               (const T*)W, (const T*)bias, (const T*)B_stack, (const float*)vpart, vstride,
               vsplit, seg_indptr, adapter_ids, num_segments, num_rows, num_adapters, H1, H2, r,
               scale);
    });
    return launch_status();
}

int sgmv_set_fused_wait(double seconds) {
    if (!(seconds >= 0.0) || seconds > 10.0) return SGMV_ERR_BAD_SHAPE;
    unsigned long long b;
    if (seconds == 0.0) {
        // 0 must stay distinguishable from "unset": store the smallest
        // positive double, which rounds to zero ticks.
        const double tiny = 5e-324;
        memcpy(&b, &tiny, sizeof b);
    } else {
        memcpy(&b, &seconds, sizeof b);
    }
    g_wait_bits.store(b, std::memory_order_relaxed);
    return SGMV_OK;
}

int sgmv_build_segments(const int32_t* row_ids, int32_t num_rows, int32_t num_adapters,
                        int32_t* seg_indptr, int32_t* adapter_ids, int32_t* num_segments,
                        void* stream) {
    if (num_rows < 0 || num_adapters < 0) return SGMV_ERR_BAD_SHAPE;
    if (!seg_indptr || !num_segments || (num_rows > 0 && (!row_ids || !adapter_ids)))
        return SGMV_ERR_NULL_PTR;
    launch(&build_segments_kernel, dim3(1), dim3(kSegThreads), (hipStream_t)stream, row_ids,
           num_rows, num_adapters, seg_indptr, adapter_ids, num_segments);
    return launch_status();
}

int sgmv_group_rows(const int32_t* row_ids, int32_t num_rows, int32_t num_adapters,
                    int32_t* perm, int32_t* seg_indptr, int32_t* adapter_ids,
                    int32_t* num_segments, void* stream) {
    if (num_rows < 0 || num_adapters < 0) return SGMV_ERR_BAD_SHAPE;
    if (num_adapters > kGroupMaxAdapters) return SGMV_ERR_UNSUPPORTED;
    if (!seg_indptr || !num_segments || (num_rows > 0 && (!row_ids || !perm)) ||
        (num_rows > 0 && num_adapters > 0 && !adapter_ids))
        return SGMV_ERR_NULL_PTR;
    launch(&group_rows_kernel, dim3(1), dim3(kSegThreads), (hipStream_t)stream, row_ids, num_rows,
           num_adapters, perm, seg_indptr, adapter_ids, num_segments);
    return launch_status();
}

int sgmv_validate_segments(const int32_t* h_seg_indptr, const int32_t* h_adapter_ids,
                           int32_t num_segments, int32_t num_rows, int32_t num_adapters) {
    if (num_segments < 0 || num_rows < 0 || num_adapters < 0) return SGMV_ERR_BAD_SHAPE;
    if (!h_seg_indptr) return SGMV_ERR_NULL_PTR;
    if (num_segments > 0 && !h_adapter_ids) return SGMV_ERR_NULL_PTR;
    if (h_seg_indptr[0] < 0) return SGMV_ERR_BAD_SEGMENTS;
    for (int32_t s = 0; s < num_segments; ++s) {
        if (h_seg_indptr[s + 1] < h_seg_indptr[s]) return SGMV_ERR_BAD_SEGMENTS;
        if (h_adapter_ids[s] < 0 || h_adapter_ids[s] >= num_adapters) return SGMV_ERR_BAD_SEGMENTS;
    }
    if (h_seg_indptr[num_segments] > num_rows) return SGMV_ERR_BAD_SEGMENTS;
    return SGMV_OK;
}

}  // extern "C"
