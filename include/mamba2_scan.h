/*
 * mamba2_scan.h -- C ABI of the Mamba2 temporal scan (forward and backward)
 * for AMD Instinct MI355X (gfx950).
 *
 * The operation (foxhunt "Custom Kernel Optimization Implementation Plan",
 * Task 1 "Mamba2 Forward" and Task 2 "Mamba2 Backward"; design spec
 * "cuBLAS Projections + Batch-Parallel Scans", Design section 1):
 *
 *   a = H W_A,  b = H W_B   over the B*K history rows H = h_history[B][K][SH2]
 *   c = h_s2 W_C            over the B current trunk rows h_s2[B][SH2]
 *   x_0 = 0,  x_{t+1} = sigmoid(a_t) * x_t + b_t   for t = 0 .. K-1
 *   context[b][s] = c[b][s] * x_K[b][s]
 *
 * and, for the scalar L = sum_{b,s} d_context[b][s] * context[b][s],
 *
 *   dW_A = H^T d_a,  dW_B = H^T d_b,  dW_C = h_s2^T d_c
 *
 * where d_a, d_b, d_c are dL/da, dL/db, dL/dc (reverse scan).
 *
 * Conventions for every entry point:
 *   - All tensors are fp32, row-major and contiguous.  Element (b, t, j) of
 *     h_history is at (b*K + t)*SH2 + j; W_X[j][s] is at j*STATE_D + s;
 *     context and d_context [b][s] at b*STATE_D + s.  Row t = K-1 is the
 *     newest history step.
 *   - Every pointer is device memory owned by the caller.  The library
 *     allocates nothing, keeps no state between calls and never synchronises:
 *     work is enqueued on `stream` (a hipStream_t; NULL = the null stream).
 *   - Supported shapes: B >= 1, K >= 1, STATE_D in {16, 32, 64},
 *     SH2 a multiple of 64 with 64 <= SH2 <= 512.
 *   - h_history, h_s2, W_A, W_B, W_C, saved and workspace must be 16-byte
 *     aligned; the other pointers 4-byte aligned.
 *   - Every argument check runs before any work is enqueued.  On a nonzero
 *     return nothing has been written, except after MAMBA2_SCAN_EHIP.
 *   - Outputs are overwritten, never accumulated into.
 *   - Calls on different streams may run concurrently if their output and
 *     scratch buffers do not overlap.
 */
#ifndef MAMBA2_SCAN_H
#define MAMBA2_SCAN_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
#define MAMBA2_SCAN_OK            0
#define MAMBA2_SCAN_EBADDIM      -1 /* a dimension <= 0, or sizes overflow    */
#define MAMBA2_SCAN_EUNSUPPORTED -2 /* STATE_D or SH2 outside the list above  */
#define MAMBA2_SCAN_ENULL        -3 /* a required pointer is NULL             */
#define MAMBA2_SCAN_ESIZE        -4 /* saved or workspace buffer too small    */
#define MAMBA2_SCAN_EALIGN       -5 /* a pointer is not aligned as required   */
#define MAMBA2_SCAN_EHIP         -6 /* the HIP runtime refused a launch       */
#define MAMBA2_SCAN_ESCRATCH     -7 /* more scratch than the fixed buffer     */

/*
 * Bytes of the `saved` buffer that mamba2_scan_fwd fills and mamba2_scan_bwd
 * reads for these dimensions (the plan's Task 2 reuses the forward's
 * projections instead of recomputing them).  Its contents are private to the
 * library.  Returns 0 if the dimensions are invalid or unsupported.
 */
size_t mamba2_scan_saved_bytes(int B, int K, int SH2, int STATE_D);

/*
 * Bytes of the scratch workspace mamba2_scan_bwd needs: the split-K partial
 * sums of the weight gradients, one slice per backward work-group.  The
 * number of slices depends only on the dimensions, so the reduction order,
 * and with it every bit of dW, is the same on every call.  Returns 0 if the
 * dimensions are invalid or unsupported.
 */
size_t mamba2_scan_bwd_workspace_bytes(int B, int K, int SH2, int STATE_D);

/*
 * Forward (plan Task 1; design spec forward steps 1-2).
 *   h_history [B][K][SH2], h_s2 [B][SH2], W_A/W_B/W_C [SH2][STATE_D]  (in)
 *   context   [B][STATE_D]                                            (out)
 *   saved     saved_bytes >= mamba2_scan_saved_bytes(...)             (out)
 * `saved` receives what the backward needs (per-step gate terms and x_K);
 * pass it unchanged to mamba2_scan_bwd with the same inputs.
 */
int mamba2_scan_fwd(int B, int K, int SH2, int STATE_D,
                    const float* h_history, const float* h_s2,
                    const float* W_A, const float* W_B, const float* W_C,
                    float* context, void* saved, size_t saved_bytes,
                    void* stream);

/*
 * Backward (plan Task 2; design spec backward steps 1-3).
 *   h_history, h_s2       the same buffers the forward read           (in)
 *   saved                 the forward's `saved` for those inputs      (in,
 *                         required: NULL returns MAMBA2_SCAN_ENULL)
 *   d_context [B][STATE_D] upstream gradient dL/dcontext              (in)
 *   dW_A, dW_B, dW_C [SH2][STATE_D]                                   (out)
 *   d_a, d_b [B][K][STATE_D], d_c [B][STATE_D]  optional (out); NULL skips
 *   workspace             workspace_bytes >= mamba2_scan_bwd_workspace_bytes
 * Equivalent to mamba2_scan_bwd_partials followed by mamba2_scan_bwd_reduce
 * on the same stream.  The weight gradients are bitwise reproducible.
 * With STATE_D > 16 supports K * SH2 <= 2^26 (a 16-sample block's rows are
 * addressed with 32-bit offsets; MAMBA2_SCAN_EUNSUPPORTED beyond, before
 * any other check); STATE_D = 16 has no such limit.
 *
 * Why `saved` is required: the two pages differ on where the backward gets
 * the projections.  The plan's Task 2 step 4 reuses the forward's A/B
 * projections, which the forward saves.  The spec's backward step 1 replays
 * them from h_history.  Both give the same results.  This library takes the
 * plan's reading.  The forward stores per-step gate coefficients (8.5 MiB at
 * B=8192, K=8, SH2=256, STATE_D=16), and the backward reads them instead of
 * projecting H a second time.  That second projection would add a whole
 * contraction to a kernel that already streams H through its matrix cores.
 * No replay form is offered, so `saved` cannot be NULL.
 */
int mamba2_scan_bwd(int B, int K, int SH2, int STATE_D,
                    const float* h_history, const float* h_s2,
                    const void* saved, size_t saved_bytes,
                    const float* d_context,
                    float* dW_A, float* dW_B, float* dW_C,
                    float* d_a, float* d_b, float* d_c,
                    void* workspace, size_t workspace_bytes,
                    void* stream);

/*
 * mamba2_scan_bwd without a workspace, for callers that cannot allocate
 * device memory: code under stream capture, tight serving loops, harnesses
 * that forbid it.  The split-K slices go to a fixed 4 MiB buffer inside the
 * library, one per device, which every supported shape fits.  A shape that
 * needed more would return MAMBA2_SCAN_ESCRATCH.  The call allocates nothing.
 * Its first call on a device looks up that device's buffer, so the device
 * must be current.  Every call on a device shares its buffer, so calls that
 * overlap in time on one device (different streams, or concurrent host
 * threads enqueuing on them) race.  Results match mamba2_scan_bwd bit for
 * bit.  The other arguments are as for mamba2_scan_bwd.
 */
int mamba2_scan_bwd_noalloc(int B, int K, int SH2, int STATE_D,
                            const float* h_history, const float* h_s2,
                            const void* saved, size_t saved_bytes,
                            const float* d_context,
                            float* dW_A, float* dW_B, float* dW_C,
                            float* d_a, float* d_b, float* d_c,
                            void* stream);

/*
 * First phase of the backward: the reverse scan and the split-K products
 * H^T [d_a | d_b] and h_s2^T d_c, one partial slice per work-group, written
 * to `workspace`.  Arguments as for mamba2_scan_bwd.
 */
int mamba2_scan_bwd_partials(int B, int K, int SH2, int STATE_D,
                             const float* h_history, const float* h_s2,
                             const void* saved, size_t saved_bytes,
                             const float* d_context,
                             float* d_a, float* d_b, float* d_c,
                             void* workspace, size_t workspace_bytes,
                             void* stream);

/*
 * Second phase: sums the partial slices of `workspace` in a fixed order and
 * overwrites dW_A, dW_B, dW_C [SH2][STATE_D].
 */
int mamba2_scan_bwd_reduce(int B, int K, int SH2, int STATE_D,
                           const void* workspace, size_t workspace_bytes,
                           float* dW_A, float* dW_B, float* dW_C,
                           void* stream);

/*
 * Input gradients, one step past the pages' backward (the implementation
 * plan's Task 2 ends at the weight gradients; its Task 1 step 2 defines the
 * projections these differentiate):
 *   d_h_history[b][t][j] = sum_s d_a[b][t][s] W_A[j][s] + d_b[b][t][s] W_B[j][s]
 *   d_h_s2[b][j]         = sum_s d_c[b][s] W_C[j][s]
 * with d_a, d_b, d_c the same terms mamba2_scan_bwd forms from `saved` and
 * d_context.  Reads W_A, W_B, W_C [SH2][STATE_D], `saved` (filled by
 * mamba2_scan_fwd with the same B, K, SH2, STATE_D) and d_context
 * [B][STATE_D]; never reads h_history or h_s2.  Overwrites
 * d_h_history [B][K][SH2] and d_h_s2 [B][SH2] (row-major, caller-owned
 * device memory, 16-byte aligned); either may be NULL to skip it, not both.
 * Independent of mamba2_scan_bwd: the two may run in either order or on
 * different streams once the forward has finished.
 * Supports K * SH2 <= 2^26 (MAMBA2_SCAN_EUNSUPPORTED beyond).
 * Returns MAMBA2_SCAN_ENULL for a NULL input or both outputs NULL,
 * MAMBA2_SCAN_ESIZE if saved_bytes is short, MAMBA2_SCAN_EALIGN for a
 * misaligned pointer (saved, d_h_history, d_h_s2: 16 bytes; the rest: 4).
 */
int mamba2_scan_bwd_input(int B, int K, int SH2, int STATE_D,
                          const float* W_A, const float* W_B, const float* W_C,
                          const void* saved, size_t saved_bytes,
                          const float* d_context,
                          float* d_h_history, float* d_h_s2,
                          void* stream);

/*
 * The backward and the input gradients together: dW_A, dW_B, dW_C as
 * mamba2_scan_bwd and d_h_history [B][K][SH2], d_h_s2 [B][SH2] as
 * mamba2_scan_bwd_input.  Training the trunk through the scan needs both.
 * Every output is bitwise reproducible and agrees with those two calls to
 * fp32 rounding.  The one-pass form contracts with bf16 MFMAs on exact
 * three-term splits of both operands, as the forward does.  With fp32 trunk
 * inputs it sums its split-K partials over 8 waves per work-group instead
 * of 12, another fixed order.  When STATE_D = 16 it makes one
 * pass over the history instead of two: the backward's work-groups, which
 * form each 16-sample block's d_a, d_b (per step) and d_c (readout) for one
 * 64-feature column block, also multiply them into W_A, W_B, W_C for that
 * block's 64 input-gradient features (the chain rule through the plan's
 * Task 1 step 2 projections).  Other widths run the two calls in sequence.
 *   W_A, W_B, W_C   the forward's weights [SH2][STATE_D], 16-byte aligned (in)
 *   d_h_history, d_h_s2  (out, overwritten, 16-byte aligned); either may be
 *                   NULL to skip it, not both
 * The other arguments are as for mamba2_scan_bwd (no debug outputs).
 * Supports K * SH2 <= 2^26 (MAMBA2_SCAN_EUNSUPPORTED beyond).
 */
int mamba2_scan_bwd_full(int B, int K, int SH2, int STATE_D,
                         const float* h_history, const float* h_s2,
                         const void* saved, size_t saved_bytes,
                         const float* d_context,
                         const float* W_A, const float* W_B, const float* W_C,
                         float* dW_A, float* dW_B, float* dW_C,
                         float* d_h_history, float* d_h_s2,
                         void* workspace, size_t workspace_bytes,
                         void* stream);

/*
 * The step after the path, with the stability multiplier (implementation
 * plan, Task 1 step 3).  As mamba2_scan_fwd, except:
 *   - the gate is m * sigmoid(a) with m = *stability (a device scalar, such
 *     as the trainer's isv_signals + 11), or 1 when stability is NULL;
 *   - when h_enriched [B][SH2] is not NULL it is overwritten with
 *       h_enriched[b][j] = h_s2[b][j] + w_j * (sum_s context[b][s]) / STATE_D,
 *     w = temporal_weight [SH2] (all ones when NULL).
 * `saved` then feeds mamba2_scan_bwd, mamba2_scan_bwd_blend or
 * mamba2_scan_bwd_input as usual (the multiplier is folded into it).
 * Alignment: h_enriched and temporal_weight 16 bytes, stability 4 bytes;
 * the other arguments as for mamba2_scan_fwd.
 */
int mamba2_scan_fwd_blend(int B, int K, int SH2, int STATE_D,
                          const float* h_history, const float* h_s2,
                          const float* W_A, const float* W_B, const float* W_C,
                          const float* stability, const float* temporal_weight,
                          float* context, float* h_enriched,
                          void* saved, size_t saved_bytes,
                          void* stream);

/* Bytes of the workspace mamba2_scan_bwd_blend needs; 0 for unsupported dims. */
size_t mamba2_scan_bwd_blend_workspace_bytes(int B, int K, int SH2, int STATE_D);

/*
 * Backward of the blend, then of the scan.  The loss is
 * L = sum_{b,j} d_h_enriched[b][j] * h_enriched[b][j]; by the chain rule
 *   d_context[b][s] = (sum_j d_h_enriched[b][j] * w_j) / STATE_D for every s,
 *   d_temporal_weight[j] = sum_b d_h_enriched[b][j] * (sum_s context[b][s]) / STATE_D,
 * then dW_A, dW_B, dW_C exactly as mamba2_scan_bwd with that d_context.
 * (The gradient reaching h_s2 through the residual is d_h_enriched itself;
 * mamba2_scan_bwd_input with the d_context written here adds the W_C path.)
 * `saved` comes from mamba2_scan_fwd_blend or mamba2_scan_fwd with the same
 * dimensions, temporal_weight the one the forward used (NULL = ones).
 * d_context [B][STATE_D] is written (and read back by the scan's backward);
 * d_temporal_weight [SH2] is overwritten, or skipped when NULL.  workspace:
 * mamba2_scan_bwd_blend_workspace_bytes() bytes, 16-byte aligned.
 * Deterministic: bitwise reproducible for given dimensions.
 * Returns MAMBA2_SCAN_ENULL for a NULL required pointer, MAMBA2_SCAN_ESIZE
 * for a short saved or workspace, MAMBA2_SCAN_EALIGN for a misaligned one
 * (d_h_enriched, temporal_weight: 16 bytes).
 */
int mamba2_scan_bwd_blend(int B, int K, int SH2, int STATE_D,
                          const float* h_history, const float* h_s2,
                          const void* saved, size_t saved_bytes,
                          const float* temporal_weight, const float* d_h_enriched,
                          float* d_context, float* dW_A, float* dW_B, float* dW_C,
                          float* d_temporal_weight,
                          void* workspace, size_t workspace_bytes,
                          void* stream);

/*
 * Reduced-precision trunk inputs: h_history and h_s2 hold bfloat16 values
 * (their 16-bit patterns, the top half of the fp32 with the same value),
 * halving the bytes of the dominant reads.  The xtrain page "Phase T7:
 * Performance -- Design Document", section "Follow-up" item 4 (bf16 mixed
 * precision with an fp32 master copy), defers this idea: bf16 matmuls change
 * the numerics and would need their own, wider tolerance.  Here only the
 * storage is bf16.  The bf16 values meet bf16
 * matrix instructions whose other operand (the weights in the forward,
 * d_a/d_b/d_c in the backward) is split exactly into three bf16 terms, so
 * every product is exact in fp32 and every sum accumulates in fp32: results
 * agree with the fp32 entry point of the same name, fed the same values,
 * to fp32 rounding.  Every other argument is as for mamba2_scan_fwd,
 * mamba2_scan_bwd_partials and mamba2_scan_bwd.  The same `saved`,
 * workspace and second phase (mamba2_scan_bwd_reduce) serve both.
 * h_history and h_s2 must be 16-byte aligned.
 */
int mamba2_scan_fwd_bf16(int B, int K, int SH2, int STATE_D,
                         const void* h_history, const void* h_s2,
                         const float* W_A, const float* W_B, const float* W_C,
                         float* context, void* saved, size_t saved_bytes,
                         void* stream);
int mamba2_scan_bwd_partials_bf16(int B, int K, int SH2, int STATE_D,
                                  const void* h_history, const void* h_s2,
                                  const void* saved, size_t saved_bytes,
                                  const float* d_context,
                                  float* d_a, float* d_b, float* d_c,
                                  void* workspace, size_t workspace_bytes,
                                  void* stream);
int mamba2_scan_bwd_full_bf16(int B, int K, int SH2, int STATE_D,
                              const void* h_history, const void* h_s2,
                              const void* saved, size_t saved_bytes,
                              const float* d_context,
                              const float* W_A, const float* W_B, const float* W_C,
                              float* dW_A, float* dW_B, float* dW_C,
                              float* d_h_history, float* d_h_s2,
                              void* workspace, size_t workspace_bytes,
                              void* stream);
int mamba2_scan_bwd_bf16(int B, int K, int SH2, int STATE_D,
                         const void* h_history, const void* h_s2,
                         const void* saved, size_t saved_bytes,
                         const float* d_context,
                         float* dW_A, float* dW_B, float* dW_C,
                         float* d_a, float* d_b, float* d_c,
                         void* workspace, size_t workspace_bytes,
                         void* stream);

/* Static text for a status code. */
const char* mamba2_scan_strerror(int status);

/*
 * Launch plan of a forward call (pure host code: touches no device and
 * enqueues nothing).  It names each kernel launch that mamba2_scan_fwd,
 * mamba2_scan_fwd_bf16 or mamba2_scan_fwd_blend enqueues for these
 * dimensions, in order.  A profiler can match them to its per-kernel rows,
 * as the design spec's "nsys Breakdown" table does for the pages' kernels.
 * A test can use it to check that every launch form the dispatcher can
 * choose is run against a reference.
 *
 * A history too long for its few samples to fill the GPU is cut into
 * chunks.  The chunks run in parallel: a summary pass, then the carry
 * across chunks, then the replay pass.  Otherwise one full pass does
 * everything.  The plan does not depend on the trunk precision.
 *
 * Fills launches[0 .. min(n, max_launches) - 1] and returns n (1 or 3), or
 * a negative status for invalid or unsupported dimensions.  `launches` may
 * be NULL when max_launches is 0.
 */
#define MAMBA2_SCAN_KERNEL_FWD    0 /* projections, gated scan, saved terms  */
#define MAMBA2_SCAN_KERNEL_CARRY  1 /* carry of the state across chunks      */
#define MAMBA2_SCAN_PASS_FULL     0 /* whole history: context + saved terms  */
#define MAMBA2_SCAN_PASS_SUMMARY  1 /* per chunk: gate product, end state    */
#define MAMBA2_SCAN_PASS_CARRY    2 /* each chunk's start state              */
#define MAMBA2_SCAN_PASS_REPLAY   3 /* per chunk from its start state        */
typedef struct {
  int kernel;        /* MAMBA2_SCAN_KERNEL_*                                 */
  int sample_blocks; /* 16-sample blocks per work-group (0 for the carry)    */
  int pass;          /* MAMBA2_SCAN_PASS_*                                   */
  int chunks;        /* history chunks run in parallel (1: not chunked)      */
  int chunk_steps;   /* steps per chunk (the last chunk takes the rest)      */
  int grid;          /* work-groups                                          */
  int threads;       /* threads per work-group                               */
} mamba2_scan_launch;
int mamba2_scan_fwd_plan(int B, int K, int SH2, int STATE_D,
                         mamba2_scan_launch* launches, int max_launches);

#ifdef __cplusplus
}
#endif

#endif /* MAMBA2_SCAN_H */
