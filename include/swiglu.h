/*
 * swiglu.h -- C ABI of the MI355X (gfx950) fused SwiGLU MLP library.
 *
 * Operation (problem statement of "Tile-Level Activation Overlap for
 * Efficient LLM Inference"; MLP block of "Anatomie d'un transformeur sur
 * GPU", §1.1 skeleton and §1.2 projection table):
 *
 *     out = silu(x . Wgate) (.) (x . Wup),     silu(z) = z * sigmoid(z)
 *     y   = out . Wdown                         (mlp_forward only)
 *
 * with x: M x d, Wgate and Wup: d x dff, Wdown: dff x d, out: M x dff,
 * y: M x d.  All matrices are row-major and dense.
 *
 * Conventions shared by every entry point
 *   - Pointers named x, w*, out, y and workspace are DEVICE pointers on the
 *     current HIP device; the caller allocates and owns them.  The library
 *     keeps no pointer after a call returns and holds no mutable global
 *     state, so calls are thread-safe (two exceptions: the graph handles at
 *     the end of this header keep the pointers they were captured with, and
 *     swiglu_up_noalloc works in a fixed array that its calls on one GPU
 *     share).
 *   - dtype is SWIGLU_BF16 (bf16 storage, fp32 accumulation, bf16 output)
 *     or SWIGLU_F32 (fp32 storage and arithmetic): x, the weights and the
 *     output share that dtype.  Or SWIGLU_BF16_FP8W / SWIGLU_BF16_MXFP4W: x,
 *     out and y in bf16, weights stored as 8-bit or 4-bit floats (see
 *     below), fp32 accumulation.
 *   - Calls only enqueue kernels on `stream` (the graph-creation calls
 *     excepted): no allocation, no copy, no
 *     synchronisation (the decode-path conventions of "Où part le temps d'un
 *     token": fixed buffers, no per-call allocation, no host waits).  A
 *     return of SWIGLU_OK means the arguments were valid and the launches
 *     were accepted; faults during execution surface at the caller's next
 *     synchronisation.  Launch errors are read with hipGetLastError, so
 *     SWIGLU_ERR_HIP also reports (and clears) an error that an earlier HIP
 *     call of the calling thread left pending.
 *   - Results are deterministic: the same inputs, shapes and device give
 *     bitwise identical outputs on every call (no atomics in any sum).
 *   - Errors are returned as negative status codes; nothing throws.  When
 *     M == 0 every call is a no-op returning SWIGLU_OK, and pointers may be
 *     NULL.
 *   - Requirements: d and dff multiples of 8 (bf16) or 4 (fp32); device
 *     pointers 16-byte aligned; 1 <= d, dff <= 2^20; 0 <= M <= 2^18.
 *     Otherwise SWIGLU_ERR_UNSUPPORTED / SWIGLU_ERR_MISALIGNED.
 *   - out, y and the workspace must not overlap any input.
 */
#ifndef SWIGLU_H
#define SWIGLU_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum swiglu_dtype {
    SWIGLU_F32 = 0,
    SWIGLU_BF16 = 1,
    /*
     * FP8 weights for decode: "Tile-Level Activation Overlap for Efficient
     * LLM Inference" (section on the problem) notes that quantised weights
     * make the memory-bound part weigh more; streaming one byte per weight
     * halves the decode path's traffic.  The pack calls take bf16 Wgate,
     * Wup and Wdown and quantise each output column: scale = (largest
     * magnitude in the column) / 448 in fp32, codes = OCP E4M3 (no
     * infinities; largest value 448) nearest to w / scale (an fp32
     * division), ties to the even code, saturating; an all-zero column
     * gets scale 0.  A NaN weight does not count toward the scale and takes
     * E4M3's NaN code 0x7F (code 0 if the column's scale is 0, like every
     * code of such a column); an infinite one makes the scale infinite.
     * The kernels widen the codes exactly to bf16, multiply
     * on the matrix unit with fp32 accumulation and apply the column scale
     * to the finished sum.  Served by the skinny path only (any M; it is
     * built for M <= 64): SWIGLU_PATH_WIDE and WIDE_PHASED return
     * SWIGLU_ERR_UNSUPPORTED.  The packed buffers hold the codes (one byte
     * per weight, padded like bf16) followed by the fp32 column scales.
     */
    SWIGLU_BF16_FP8W = 2,
    /*
     * MXFP4 weights for decode, the same idea at four bits: OCP Microscaling
     * (v1.0) MXFP4, E2M1 codes with one power-of-two (E8M0) scale per 32
     * consecutive rows of a column.  The pack calls take bf16 weights: the
     * block's shared exponent is floor(log2(largest magnitude)) - 2,
     * clamped to [-126, 127] (0 for an all-zero block), and each code is
     * the E2M1 value (0, 0.5, 1, 1.5, 2, 3, 4, 6) nearest to w / 2^s, ties
     * to the even code, saturating at 6.  E2M1 has no infinity or NaN: such
     * weights are coded +-6 with their sign bit, a NaN does not count toward
     * the largest magnitude and an infinite one sets s = 127 (the block
     * becomes useless, but nothing is undefined; the MX block-NaN scale is
     * not used).  The kernels widen codes and scale
     * exactly to bf16 (gfx950's scaled FP4 conversion), multiply on the
     * matrix unit with fp32 accumulation.  Skinny path only, like
     * SWIGLU_BF16_FP8W; K is padded to 128 and the packed buffers hold half
     * a byte per weight plus one scale byte per 32 weights.
     */
    SWIGLU_BF16_MXFP4W = 3
} swiglu_dtype_t;

typedef enum swiglu_status {
    SWIGLU_OK = 0,
    SWIGLU_ERR_INVALID_ARG = -1,   /* NULL pointer, negative M, d or dff <= 0 */
    SWIGLU_ERR_UNSUPPORTED = -2,   /* unknown dtype, unsupported shape or path */
    SWIGLU_ERR_MISALIGNED = -3,    /* a device pointer is not 16-byte aligned */
    SWIGLU_ERR_WORKSPACE = -4,     /* workspace smaller than required */
    SWIGLU_ERR_HIP = -5,           /* a HIP launch or attribute call failed */
    SWIGLU_ERR_SCRATCH = -6        /* swiglu_up_noalloc: needs more than its fixed array */
} swiglu_status_t;

/* Path selection for the *_ex entry points. */
typedef enum swiglu_path {
    SWIGLU_PATH_AUTO = 0,      /* dispatcher: few rows -> skinny, many rows -> wide */
    SWIGLU_PATH_SKINNY = 1,    /* split-over-weights kernels (any M, any dtype) */
    SWIGLU_PATH_WIDE = 2,      /* bf16 MFMA GEMM over a four-stage LDS ring of operand
                                  tiles, the two waves of each SIMD in ping-pong */
    /* bf16 MFMA GEMM, two-pass schedule: per output tile a K loop over the
     * gate columns, silu in registers, then a K loop over the up columns
     * (Kernel-1 of "Tile-Level Activation Overlap for Efficient LLM
     * Inference", section on its two kernel designs).  Results are
     * bit-identical to SWIGLU_PATH_WIDE; the dispatcher never picks it
     * because it is slower on MI355X at every measured shape.  In
     * mlp_forward_ex it applies to the gate/up product; the down product
     * then takes SWIGLU_PATH_WIDE. */
    SWIGLU_PATH_WIDE_PHASED = 3,
    /* mlp_forward_ex / mlp_block_forward_ex only, bf16 only: the down
     * projection fused into the gate/up kernel, the fusion of the launches
     * that "Où part le temps d'un token" proposes in its section on what
     * remains.  Each workgroup owns a slice of d_ff and up to 64 rows: it
     * forms that slice of h = silu(x.Wg)*(x.Wu) in LDS (rounded to bf16, as
     * on the other paths), multiplies it by the matching rows of Wdown and
     * writes the slice's fp32 share of y to the workspace; a second kernel
     * adds the slices in ascending order (deterministic, no atomics) and
     * applies the epilogue.  h never reaches memory; the workspace holds
     * slices x M x d fp32 values instead.  Other calls return
     * SWIGLU_ERR_UNSUPPORTED. */
    SWIGLU_PATH_FUSED_DOWN = 4
} swiglu_path_t;

/* Human-readable name of a status code (static string, never NULL). */
const char *swiglu_status_string(int status);

/* Library ABI version (incremented on any incompatible change). */
int swiglu_version(void);

/*
 * Size in bytes of the fused gate/up buffer written by swiglu_pack_weights,
 * or 0 for invalid arguments.  The buffer is opaque: gate and up column
 * blocks interleaved (the fused K x 2N weight of Kernel-2 in "Tile-Level
 * Activation Overlap for Efficient LLM Inference"), padded with zeros.
 */
size_t swiglu_packed_bytes(int64_t d, int64_t dff, int dtype);

/* Size in bytes of the packed down weight written by swiglu_pack_down. */
size_t swiglu_down_packed_bytes(int64_t d, int64_t dff, int dtype);

/*
 * Workspace bytes for swiglu_up (with_down = 0) or mlp_forward
 * (with_down = 1) with these sizes on the automatic path (0 if none); the
 * _ex variant gives the size for a forced path.  Returns 0 for invalid
 * arguments as well, which the calls then reject.
 *
 * With this much workspace the many-rows (MFMA) path first copies x into
 * the workspace in the layout of its A operand fragments (row blocks of 16,
 * K chunks of 32; about M x d x 2 bytes), and mlp_forward keeps h in that
 * layout, which makes the matrix product faster.  A smaller workspace that
 * still holds the row-major plan (nothing for swiglu_up on that path; h as
 * M x padded-dff row-major for mlp_forward) runs the same kernels on x in
 * place, with bit-identical results.  Below that the call returns
 * SWIGLU_ERR_WORKSPACE.  The skinny path needs only its split-K partials.
 */
size_t swiglu_workspace_bytes(int64_t M, int64_t d, int64_t dff, int dtype, int with_down);
size_t swiglu_workspace_bytes_ex(int64_t M, int64_t d, int64_t dff, int dtype, int with_down,
                                 int path);

/* The path SWIGLU_PATH_AUTO takes for these sizes (SKINNY or WIDE), or a
 * negative status for invalid arguments. */
int swiglu_select_path(int64_t M, int64_t d, int64_t dff, int dtype);

/*
 * Packs Wgate and Wup (each d x dff, row-major, device) into Wpacked (device,
 * swiglu_packed_bytes(d, dff, dtype) bytes).  Done once per weight set; the
 * packed buffer then serves every M and both paths.  Pure permutation with
 * zero padding: no rounding (SWIGLU_BF16_FP8W: Wgate and Wup are bf16 and
 * are quantised as described with that dtype).  Wpacked must not overlap
 * Wgate or Wup.
 */
int swiglu_pack_weights(const void *Wgate, const void *Wup, void *Wpacked,
                        int64_t d, int64_t dff, int dtype, hipStream_t stream);

/*
 * Packs Wdown (dff x d, row-major, device) into Wdpacked (device,
 * swiglu_down_packed_bytes(d, dff, dtype) bytes) for mlp_forward.
 */
int swiglu_pack_down(const void *Wdown, void *Wdpacked, int64_t d, int64_t dff, int dtype,
                     hipStream_t stream);

/*
 * out (M x dff) = silu(x . Wgate) (.) (x . Wup), with x M x d and Wpacked
 * from swiglu_pack_weights: the SwiGLU product of the problem statement of
 * "Tile-Level Activation Overlap for Efficient LLM Inference" (gate and up
 * projections of the MLP, "Anatomie d'un transformeur sur GPU" §1.2).
 * Accumulation in fp32; silu and the product in
 * fp32; one rounding to the output dtype at the store.  workspace (device,
 * may be NULL when swiglu_workspace_bytes returns 0) holds split-K partial
 * sums on the skinny path and the packed copy of x on the many-rows path
 * (see swiglu_workspace_bytes).
 */
int swiglu_up(const void *x, const void *Wpacked, void *out,
              int64_t M, int64_t d, int64_t dff, int dtype,
              void *workspace, size_t workspace_bytes, hipStream_t stream);

/* swiglu_up (the same product, "Tile-Level Activation Overlap for Efficient
 * LLM Inference", problem statement) with a forced path (swiglu_path_t);
 * WIDE or WIDE_PHASED with fp32, and FUSED_DOWN, return
 * SWIGLU_ERR_UNSUPPORTED. */
int swiglu_up_ex(const void *x, const void *Wpacked, void *out,
                 int64_t M, int64_t d, int64_t dff, int dtype,
                 void *workspace, size_t workspace_bytes, hipStream_t stream, int path);

/*
 * swiglu_up for callers that cannot allocate device memory: code under HIP
 * graph capture, serving loops and harnesses that forbid hipMalloc.  Same
 * arguments, computation, dispatcher (SWIGLU_PATH_AUTO) and status codes as
 * swiglu_up, without the workspace arguments: the workspace is a fixed
 * array of SWIGLU_SCRATCH_BYTES (32 MiB) inside the library, one copy per
 * GPU, held until the process ends.  It holds the split-K partial sums of
 * the few-rows path (at most 16 MiB for any shape within the limits) and,
 * when it fits, the packed copy of x for the many-rows path (M x d x 2
 * bytes, rows padded to 16 and d to 64; otherwise x is read in place, with
 * bit-identical results).  A call whose plan would need more returns
 * SWIGLU_ERR_SCRATCH before any launch.  The call allocates nothing and
 * calls no allocating routine; the first call on each device looks up the
 * array's device address (hipGetSymbolAddress, no allocation), so make one
 * call per device before capturing one into a graph.  Results are bitwise
 * those of swiglu_up with the workspace it reports.
 *
 * Every call on a GPU shares that GPU's array: calls that may run at the
 * same time on one GPU (other streams, other threads, or graph replays in
 * flight together) race on it and must be serialised by the caller: issue
 * them on one stream and, when several host threads make them, one call at
 * a time (a call enqueues up to two kernels, the split product and its
 * second pass, which another call's kernels must not come between).  No
 * part of the array has to start at zero: each call writes every byte it
 * reads.
 */
#define SWIGLU_SCRATCH_BYTES ((size_t)32 << 20)

int swiglu_up_noalloc(const void *x, const void *Wpacked, void *out,
                      int64_t M, int64_t d, int64_t dff, int dtype, hipStream_t stream);

/*
 * y (M x d) = (silu(x . Wgate) (.) (x . Wup)) . Wdown: the MLP of the layer
 * skeleton ("Anatomie d'un transformeur sur GPU" §1.1: Wgate and Wup into
 * SwiGLU, then Wdown), with Wpacked from swiglu_pack_weights and Wdpacked from
 * swiglu_pack_down.  The intermediate h (M x dff) is kept in the workspace
 * in the storage dtype (bf16 or fp32), then multiplied by Wdown with fp32
 * accumulation.
 */
int mlp_forward(const void *x, const void *Wpacked, const void *Wdpacked, void *y,
                int64_t M, int64_t d, int64_t dff, int dtype,
                void *workspace, size_t workspace_bytes, hipStream_t stream);

/* mlp_forward (the MLP of "Anatomie d'un transformeur sur GPU" §1.1) with a
 * forced path for both products. */
int mlp_forward_ex(const void *x, const void *Wpacked, const void *Wdpacked, void *y,
                   int64_t M, int64_t d, int64_t dff, int dtype,
                   void *workspace, size_t workspace_bytes, hipStream_t stream, int path);

/*
 * The MLP half of a pre-normalised transformer layer in one call:
 *
 *     n   = rmsnorm(r) = r / sqrt(mean(r^2) + eps) * gamma      (per row)
 *     out = r + (silu(n . Wgate) (.) (n . Wup)) . Wdown (+ bias)
 *
 * "Anatomie d'un transformeur sur GPU", §1.1 layer skeleton (RMSNorm, the
 * SwiGLU MLP, then the residual add) and §1.6 (its kernels 7 to 11, five
 * launches in a classic implementation); the optional bias is the product
 * plus bias of the "Affine" operation of "Où part le temps d'un token"
 * (section "Deux opérations de trop"), added in the epilogue that finishes
 * the down product.  The pages do not write RMSNorm out: this is the usual
 * RMS form with a per-feature gain and a caller-given eps >= 0.
 *
 * r (M x d), gamma (d), bias (d, or NULL) and out (M x d) are device
 * arrays in the activation type of dtype (bf16 for SWIGLU_BF16,
 * SWIGLU_BF16_FP8W and SWIGLU_BF16_MXFP4W, fp32 for SWIGLU_F32); Wpacked
 * and Wdpacked as for
 * mlp_forward.  n is rounded once to the activation type; the products
 * accumulate in fp32; bias and residual are added in fp32 before the one
 * rounding of out.  out may equal r (the residual stream updated in place);
 * otherwise it must not overlap any input.  The workspace (device,
 * mlp_block_workspace_bytes[_ex] bytes) holds n, h and any split-K
 * partials.  r, gamma, out and the workspace must be 16-byte aligned, bias
 * element-aligned.  Errors as for mlp_forward; eps negative, infinite or
 * NaN is SWIGLU_ERR_INVALID_ARG.  The _ex variant forces the path of both
 * products as mlp_forward_ex does.
 */
size_t mlp_block_workspace_bytes(int64_t M, int64_t d, int64_t dff, int dtype);
size_t mlp_block_workspace_bytes_ex(int64_t M, int64_t d, int64_t dff, int dtype, int path);

int mlp_block_forward(const void *r, const void *gamma, float eps, const void *Wpacked,
                      const void *Wdpacked, const void *bias, void *out,
                      int64_t M, int64_t d, int64_t dff, int dtype,
                      void *workspace, size_t workspace_bytes, hipStream_t stream);

int mlp_block_forward_ex(const void *r, const void *gamma, float eps, const void *Wpacked,
                         const void *Wdpacked, const void *bias, void *out,
                         int64_t M, int64_t d, int64_t dff, int dtype,
                         void *workspace, size_t workspace_bytes, hipStream_t stream, int path);

/*
 * Recorded calls (HIP graphs).  A per-kernel fixed cost (launch, ramp-up,
 * drain) dominates short calls; replaying a recorded sequence of launches
 * from one host call is one of the two remedies that "Où part le temps d'un
 * token" names in its section on what remains (the launches), fusion being
 * the other.  As that section notes, a recording replays the same kernels
 * on the same buffers with the same sizes: every pointer and size given to
 * a *_graph_create call is fixed in the graph.  To reuse it, overwrite x
 * (and the weights, if they change) in place and launch again; out/y are
 * rewritten by each launch.
 *
 * swiglu_up_graph_create / mlp_forward_graph_create / mlp_block_graph_create
 * validate their arguments exactly as swiglu_up_ex / mlp_forward_ex /
 * mlp_block_forward_ex do (same status codes; nothing is created on
 * error), then record that one call on a
 * private stream of the current device and instantiate it.  They allocate
 * host and HIP objects, so they belong to set-up, not to the per-call path.
 * On success *graph receives a handle owned by the caller; the buffers must
 * outlive it.  M == 0 records an empty graph.
 *
 * swiglu_graph_launch enqueues one replay on `stream` (any stream of the
 * device the graph was created on); replays on one stream run in order,
 * and replays that share a workspace must not run concurrently.  Returns
 * SWIGLU_ERR_INVALID_ARG for a NULL handle, SWIGLU_ERR_HIP if the launch is
 * refused.  swiglu_graph_destroy releases the handle (NULL is a no-op); it
 * must not be called while a replay may still be running.
 */
typedef struct swiglu_graph_s *swiglu_graph_t;

int swiglu_up_graph_create(const void *x, const void *Wpacked, void *out,
                           int64_t M, int64_t d, int64_t dff, int dtype,
                           void *workspace, size_t workspace_bytes, int path,
                           swiglu_graph_t *graph);

int mlp_forward_graph_create(const void *x, const void *Wpacked, const void *Wdpacked, void *y,
                             int64_t M, int64_t d, int64_t dff, int dtype,
                             void *workspace, size_t workspace_bytes, int path,
                             swiglu_graph_t *graph);

int mlp_block_graph_create(const void *r, const void *gamma, float eps, const void *Wpacked,
                           const void *Wdpacked, const void *bias, void *out,
                           int64_t M, int64_t d, int64_t dff, int dtype,
                           void *workspace, size_t workspace_bytes, int path,
                           swiglu_graph_t *graph);

int swiglu_graph_launch(swiglu_graph_t graph, hipStream_t stream);

int swiglu_graph_destroy(swiglu_graph_t graph);

#ifdef __cplusplus
}
#endif

#endif /* SWIGLU_H */
