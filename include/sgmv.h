/*
 * sgmv.h -- C ABI of libsgmv.so, SGMV (segmented gather matrix-vector
 * multiplication) for multi-LoRA serving on AMD Instinct MI355X (gfx950).
 *
 * The operation.  A LoRA-adapted linear layer outputs the base product plus
 * a low-rank correction, y = xW + xAB, with A of shape [H1, r] and B of shape
 * [r, H2] (Punica walkthrough, omica.com.cn/news/959180, section 2.1).  A
 * batch mixes requests for many adapters; the correction for request i,
 * x_i A_i B_i, is computed in two steps: the shrink v_i = x_i A_i, a gather of
 * the request's A out of one back-to-back stack of all adapters' A matrices
 * followed by a vector-matrix product, and the expand v_i B_i over the
 * likewise stacked B matrices (same page, section 2.2; aivaro.ru answer 959,
 * section 3.2).  Requests for the same adapter form contiguous row segments
 * (segmented inputs and outputs: Punica review on nubint.ai, "Proposed
 * method").  This library adds the correction, times a scale s, to y:
 *
 *     for every segment t, every row i in [seg_indptr[t], seg_indptr[t+1]):
 *         a = adapter_ids[t]
 *         v[i, :] = x[i, :] @ A_stack[a]                  (shrink, H1 -> r)
 *         y[i, :] = y[i, :] + s * v[i, :] @ B_stack[a]    (expand, r -> H2)
 *
 * Layout (all row-major, dense, no padding):
 *     x        [num_rows, H1]              dtype
 *     y        [num_rows, H2]              dtype, updated in place
 *     A_stack  [num_adapters, H1, r]       dtype, adapter a at a*H1*r
 *     B_stack  [num_adapters, r, H2]       dtype, adapter a at a*r*H2
 *     v        [num_rows, r]               float32 (the shrink output)
 *     seg_indptr  int32 [num_segments + 1], non-decreasing, CSR row pointer
 *     adapter_ids int32 [num_segments]
 * x, A_stack, B_stack and y share one dtype; every sum is accumulated in
 * float32 and y is rounded once (nearest-even) to its dtype.
 *
 * Pointers.  Every array argument is a DEVICE pointer owned by the caller
 * (the host-side validator is the one exception and says so).  The library
 * keeps no state between calls, allocates no memory and never synchronises
 * the host with the device (sgmv_set_fused_wait() is the one process-wide
 * setting): each call only enqueues kernels on `stream`
 * (a hipStream_t; NULL means the default stream) and returns.
 *
 * Segment table.  Rows outside every segment are left untouched; empty
 * segments do nothing; an adapter may name several segments; segments must
 * not overlap.  The table is read on the device and is not validated on the
 * host (that would need a device-to-host copy).  For memory safety the
 * kernels clamp segment bounds to [0, num_rows) and skip a segment whose
 * adapter id lies outside [0, num_adapters); what a malformed table computes
 * is otherwise unspecified.  sgmv_validate_segments() checks a host copy.
 *
 * Workspace.  sgmv_shrink and lora_apply take caller-owned device scratch
 * (size from the *_workspace_bytes queries, a pure function of the shapes).
 * Its first 256 KiB hold synchronisation counters: they must be zero before
 * the buffer is first used (hipMemset once at allocation), and every call
 * leaves them zero again, so one buffer serves any sequence of calls of any
 * shapes, including calls captured in a HIP graph.  (The last 4 bytes of
 * that region are a sticky flag, set to 1 if a workgroup ever stopped
 * waiting and recomputed its input itself; results are the same either way.)
 * The rest holds float32 partial sums and may contain anything.  Two calls
 * that may run at the same time (e.g. on different streams) must not share
 * a workspace.
 *
 * Aliasing.  y must not overlap x, v, the stacks or the workspace.
 *
 * Errors.  Calls return SGMV_OK after enqueueing, or a status describing the
 * first problem found by the host-side checks (made before anything is
 * enqueued) or by the HIP launch.  Device faults surface at the caller's
 * next synchronisation, as usual for HIP.  num_rows == 0 or
 * num_segments == 0 is a valid no-op.
 *
 * Rank.  r is a runtime argument (any 1 <= r <= SGMV_MAX_RANK, no
 * recompilation: aivaro.ru answer 959, section 3.2).  Ranks 8, 16, 32, 64
 * and 128 (and 4 for float32) with 16-byte aligned arrays take the
 * vectorised kernels; anything else takes a slower general kernel that
 * computes the same thing.
 */
#ifndef SGMV_H
#define SGMV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SGMV_ABI_VERSION 1
#define SGMV_MAX_RANK 128

typedef enum {
    SGMV_F32 = 0,
    SGMV_F16 = 1,
    SGMV_BF16 = 2
} sgmv_dtype_t;

typedef enum {
    SGMV_OK = 0,
    SGMV_ERR_NULL_PTR = 1,     /* a required pointer is NULL                    */
    SGMV_ERR_BAD_SHAPE = 2,    /* negative size, r outside [1, SGMV_MAX_RANK]   */
    SGMV_ERR_BAD_DTYPE = 3,    /* dtype is not one of sgmv_dtype_t              */
    SGMV_ERR_UNSUPPORTED = 4,  /* sizes beyond what the kernels index (>2^31)   */
    SGMV_ERR_WORKSPACE = 5,    /* workspace NULL or smaller than required       */
    SGMV_ERR_HIP = 6,          /* a HIP launch reported an error                */
    SGMV_ERR_BAD_SEGMENTS = 7, /* (validator only) malformed segment table      */
    SGMV_ERR_SCRATCH = 8       /* lora_apply_noalloc: the call needs more than  */
                               /* SGMV_NOALLOC_SCRATCH_BYTES of scratch         */
} sgmv_status_t;

/* Version of this ABI (SGMV_ABI_VERSION of the library that was loaded). */
int sgmv_abi_version(void);

/* Human-readable name of a status code (static string, never NULL). */
const char* sgmv_status_string(int status);

/* Text of the last HIP error behind an SGMV_ERR_HIP returned to the calling
 * thread ("no error" if there was none; static string, never NULL). */
const char* sgmv_last_hip_error(void);

/*
 * Shrink: v[i, :] = x[i, :] @ A_stack[adapter_ids[t]] for every row i of
 * every segment t (overwrite; float32).  Rows of v outside every segment
 * keep their contents.  The reduction over H1 is split across workgroups and
 * combined in a fixed order, so repeated calls give identical bits.
 *
 * workspace: device scratch of at least sgmv_shrink_workspace_bytes(...)
 * bytes (see "Workspace" above).  May be NULL only when that size is 0.
 */
size_t sgmv_shrink_workspace_bytes(int32_t num_rows, int32_t num_segments,
                                   int32_t H1, int32_t r, int32_t dtype);
int sgmv_shrink(float* v, const void* x, const void* A_stack,
                const int32_t* seg_indptr, const int32_t* adapter_ids,
                int32_t num_segments, int32_t num_rows, int32_t num_adapters,
                int32_t H1, int32_t r, int32_t dtype,
                void* workspace, size_t workspace_bytes, void* stream);

/*
 * Expand: y[i, :] = round(y[i, :] + scale * (v[i, :] @ B_stack[adapter_ids[t]]))
 * for every row i of every segment t; v is float32 [num_rows, r], the sum
 * over r is taken in float32 and y is rounded once to its dtype.
 */
int sgmv_expand(void* y, const float* v, const void* B_stack,
                const int32_t* seg_indptr, const int32_t* adapter_ids,
                int32_t num_segments, int32_t num_rows, int32_t num_adapters,
                int32_t r, int32_t H2, float scale, int32_t dtype, void* stream);

/*
 * Fused add-on: y[i, :] = round(y[i, :] + scale * (x[i, :] @ A_a) @ B_a),
 * a = adapter_ids of row i's segment.  The intermediate v stays in float32
 * and never leaves the workspace.
 *
 * Decode- and prefill-shaped calls with a vectorised rank run as a single
 * kernel in which the expand workgroups wait, with bounded patience, for the
 * shrink workgroups of their rows; the result does not depend on how long
 * they wait.
 *
 * workspace: device scratch of at least lora_apply_workspace_bytes(...)
 * bytes (see "Workspace" above).
 */
size_t lora_apply_workspace_bytes(int32_t num_rows, int32_t num_segments,
                                  int32_t H1, int32_t H2, int32_t r, int32_t dtype);
int lora_apply(void* y, const void* x, const void* A_stack, const void* B_stack,
               const int32_t* seg_indptr, const int32_t* adapter_ids,
               int32_t num_segments, int32_t num_rows, int32_t num_adapters,
               int32_t H1, int32_t H2, int32_t r, float scale, int32_t dtype,
               void* workspace, size_t workspace_bytes, void* stream);

/*
 * lora_apply for callers that cannot allocate memory -- code being captured
 * into a HIP graph, tight serving loops, harnesses that forbid hipMalloc:
 * the same computation, kernels and results as lora_apply (bit for bit),
 * with no workspace argument.  Its scratch is a static device array inside
 * the library, SGMV_NOALLOC_SCRATCH_BYTES per GPU, held from the first call
 * on a GPU until the process ends.  The call allocates nothing: no hipMalloc,
 * no hipFree, no allocating library routine.
 *
 * Limit: a call whose lora_apply_workspace_bytes(...) exceeds
 * SGMV_NOALLOC_SCRATCH_BYTES returns SGMV_ERR_SCRATCH before enqueueing
 * anything (use lora_apply with a workspace of that size instead).
 *
 * The scratch is shared by every call on one GPU and keeps what the last
 * call left there: calls that may overlap on one GPU (different streams,
 * different host threads without ordering) race and must not be made.
 * Its synchronisation counters are zero when the library is loaded (static
 * storage) and every call leaves them zero; the first call on a GPU made
 * outside a graph capture also clears them with a small kernel on `stream`.
 * The current device must be the GPU that `stream` belongs to.  Arguments,
 * layout and the other errors are those of lora_apply.
 */
#define SGMV_NOALLOC_SCRATCH_BYTES (16u << 20)
int lora_apply_noalloc(void* y, const void* x, const void* A_stack, const void* B_stack,
                       const int32_t* seg_indptr, const int32_t* adapter_ids,
                       int32_t num_segments, int32_t num_rows, int32_t num_adapters,
                       int32_t H1, int32_t H2, int32_t r, float scale, int32_t dtype,
                       void* stream);

/*
 * Several LoRA add-ons over one batch -- e.g. the q, k, v and o projections
 * of a decoder layer -- in one call: for every problem p,
 *   problems[p].y[i, :] = round(y + scale_p * (x_p[i, :] @ A_p[a]) @ B_p[a])
 * with the shared segment table, num_rows, num_adapters, r and dtype, and
 * each problem's own arrays, H1, H2 and scale.  This amortises the launch
 * and the shrink-to-expand hand-off, which dominate a decode-sized call
 * (the pages stress kernel-launch overhead: Punica walkthrough,
 * omica.com.cn/news/959180, section 2.2).  Results equal those of one
 * lora_apply per problem.
 *
 * problems: HOST array of num_problems (1..SGMV_MAX_PROBLEMS) descriptors;
 * the pointers in them are device pointers, as for lora_apply, and the
 * problems must not overlap each other's y.  Decode-shaped calls (vector
 * ranks, aligned pointers, at most 1024 segments, segments of few rows) run
 * as one launch; any other call runs as one lora_apply per problem, in order.
 *
 * workspace: at least lora_apply_multi_workspace_bytes(...) bytes, with the
 * conventions of "Workspace" above.  Returns as lora_apply.
 */
#define SGMV_MAX_PROBLEMS 8
typedef struct {
    void* y;               /* [num_rows, H2], updated in place */
    const void* x;         /* [num_rows, H1] */
    const void* A_stack;   /* [num_adapters, H1, r] */
    const void* B_stack;   /* [num_adapters, r, H2] */
    int32_t H1;
    int32_t H2;
    float scale;
} sgmv_lora_problem;

size_t lora_apply_multi_workspace_bytes(const sgmv_lora_problem* problems,
                                        int32_t num_problems, int32_t num_rows,
                                        int32_t num_segments, int32_t r, int32_t dtype);
int lora_apply_multi(const sgmv_lora_problem* problems, int32_t num_problems,
                     const int32_t* seg_indptr, const int32_t* adapter_ids,
                     int32_t num_segments, int32_t num_rows, int32_t num_adapters,
                     int32_t r, int32_t dtype, void* workspace, size_t workspace_bytes,
                     void* stream);

/*
 * Adapted linear layer with the base product fused in:
 *   y[i, :] = round(x[i, :] @ W^T + bias + scale * (x[i, :] @ A_a) @ B_a)
 * for every row i, a = adapter_ids of row i's segment; rows outside every
 * segment (or in a segment whose adapter id is outside [0, num_adapters))
 * get round(x[i, :] @ W^T + bias).  This is the layer y = xW + xAB of Punica
 * walkthrough (omica.com.cn/news/959180, section 2.1) computed as one fused
 * kernel over the output, the correction added to each base tile before it
 * is stored (aivaro.ru answer 959, section 3.2: fusing the LoRA transform
 * into the base linear layer saves memory traffic), so y is written once
 * and never read.
 *
 * y: [num_rows, H2], overwritten.  x: [num_rows, H1].  W: [H2, H1], the row
 * of weights of each output feature (the usual layout of a linear layer's
 * weight; the page's W is its transpose).  bias: [H2] or NULL.  The stacks
 * and the segment table are those of lora_apply; with num_segments == 0
 * they may be NULL and the call computes the base layer alone.  All sums
 * are taken in float32 and y is rounded once.
 *
 * fp16/bf16 with H1 and H2 multiples of 8 and 16-byte aligned x, W, y,
 * bias and B_stack run on the matrix cores; any other call (float32
 * included) takes a slow element-wise kernel with the same definition.
 * Decode batches on the matrix cores (at most 64 rows, r in {16, 32, 64,
 * 128}, 16-byte aligned A_stack) take one launch: each workgroup of the
 * layer also computes a share of x @ A_a, publishes it, and waits for the
 * others' before adding its correction (the single-launch hand-off of
 * lora_apply, with the same patience, sgmv_set_fused_wait(); a workgroup
 * that stops waiting recomputes its share with the same arithmetic, so
 * the bits do not depend on it).  Other calls enqueue two launches: the
 * shrink of the add-on (skipped when num_segments == 0), then the layer.
 *
 * workspace: at least lora_linear_workspace_bytes(...) bytes, with the
 * conventions of "Workspace" above.  Returns as lora_apply; num_rows == 0
 * is a no-op.
 */
size_t lora_linear_workspace_bytes(int32_t num_rows, int32_t num_segments, int32_t H1,
                                   int32_t H2, int32_t r, int32_t dtype);
int lora_linear(void* y, const void* x, const void* W, const void* bias,
                const void* A_stack, const void* B_stack,
                const int32_t* seg_indptr, const int32_t* adapter_ids,
                int32_t num_segments, int32_t num_rows, int32_t num_adapters,
                int32_t H1, int32_t H2, int32_t r, float scale, int32_t dtype,
                void* workspace, size_t workspace_bytes, void* stream);

/*
 * On-demand adapter loading: copies `count` adapters from HOST memory into
 * slots [slot, slot + count) of the device stacks -- h_A [count, H1, r]
 * into A_stack[slot ..] and h_B [count, r, H2] into B_stack[slot ..], all
 * row-major in the stacks' dtype -- with two asynchronous copies on
 * `stream`, so that the next lora_apply on that stream sees them.  Adapters
 * not yet resident are brought in this way when a request needs them
 * (Punica review, nubint.ai, "Proposed method": the
 * system loads LoRA models on demand and keeps only the base model
 * resident).  For the copy to overlap other work the host buffers must be
 * pinned (hipHostMalloc); pageable buffers are staged by the runtime.  The
 * host buffers must stay valid until the copies have completed.  Returns
 * SGMV_OK, SGMV_ERR_NULL_PTR, SGMV_ERR_BAD_SHAPE (slots outside
 * [0, num_adapters), count < 1, bad sizes), SGMV_ERR_BAD_DTYPE or
 * SGMV_ERR_HIP.
 */
int sgmv_load_adapter(void* A_stack, void* B_stack, int32_t slot, int32_t count,
                      int32_t num_adapters, const void* h_A, const void* h_B, int32_t H1,
                      int32_t H2, int32_t r, int32_t dtype, void* stream);

/*
 * Process-wide patience, in seconds (0 <= seconds <= 10; default 0.02), of
 * the single-kernel lora_apply's expand workgroups waiting for their shrink
 * workgroups (and of the one-launch lora_linear's workgroups waiting for
 * each other's shares of x @ A_a).  A workgroup that stops waiting computes its input itself with
 * the same arithmetic in the same order, so results never depend on this
 * setting; 0 makes every expand workgroup do so without waiting (that is
 * how the path is tested).  This is the library's only state.  Returns SGMV_OK or
 * SGMV_ERR_BAD_SHAPE for a value out of range.
 */
int sgmv_set_fused_wait(double seconds);

/*
 * Host-side check of a segment table held in HOST memory: seg_indptr
 * non-decreasing from >= 0, seg_indptr[num_segments] <= num_rows, every
 * adapter id in [0, num_adapters).  Returns SGMV_OK or SGMV_ERR_BAD_SEGMENTS
 * (SGMV_ERR_NULL_PTR / SGMV_ERR_BAD_SHAPE for bad arguments).
 */
int sgmv_validate_segments(const int32_t* h_seg_indptr, const int32_t* h_adapter_ids,
                           int32_t num_segments, int32_t num_rows, int32_t num_adapters);

/*
 * Segment tables built on the device from per-row adapter ids (the
 * per-sample LoRA indices of Punica walkthrough, omica.com.cn/news/959180,
 * section 3.2; SGMV itself wants the batch "segmented" by adapter, Punica
 * review, nubint.ai, "Proposed method").
 *
 * row_ids [num_rows] int32: the adapter of each row; an id outside
 * [0, num_adapters) means "no adapter" (the row is left untouched by a
 * lora_apply over the resulting table).
 *
 * Outputs, all DEVICE arrays owned by the caller:
 *   seg_indptr [num_rows + 1], adapter_ids [num_rows]: a segment table of
 *     num_rows segments whose first *num_segments are the real ones; the
 *     rest are empty (seg_indptr = the end of the last real segment,
 *     adapter id -1).  So the table can be handed to lora_apply with
 *     num_segments = num_rows and no device-to-host read.
 *   num_segments [1]: the real segment count.
 *
 * sgmv_build_segments: one segment per maximal run of equal (normalised)
 * ids, in row order; no reordering of rows is needed.  Rows without an
 * adapter form segments with adapter id -1.
 *
 * sgmv_group_rows: also writes perm [num_rows], a stable grouping of the
 * rows: the rows of adapter 0 in increasing row order, then those of
 * adapter 1, ..., then the rows without an adapter.  Row j of the grouped
 * batch is row perm[j] of the original one.  The segment table describes
 * the grouped batch, with one segment per adapter present, in increasing
 * id order; the rows without an adapter come after the last segment.  Its
 * size is M = min(num_rows, num_adapters) segments instead of num_rows
 * (seg_indptr [M + 1], adapter_ids [M] are written), since there is at most
 * one segment per adapter; pass M to lora_apply.  num_adapters must be at
 * most 4096 (SGMV_ERR_UNSUPPORTED beyond).
 *
 * Both run as one workgroup on `stream` and return SGMV_OK after
 * enqueueing, SGMV_ERR_NULL_PTR / SGMV_ERR_BAD_SHAPE for bad arguments, or
 * SGMV_ERR_HIP.  num_rows == 0 writes seg_indptr[0] = 0 and a zero count.
 */
int sgmv_build_segments(const int32_t* row_ids, int32_t num_rows, int32_t num_adapters,
                        int32_t* seg_indptr, int32_t* adapter_ids, int32_t* num_segments,
                        void* stream);
int sgmv_group_rows(const int32_t* row_ids, int32_t num_rows, int32_t num_adapters,
                    int32_t* perm, int32_t* seg_indptr, int32_t* adapter_ids,
                    int32_t* num_segments, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SGMV_H */
