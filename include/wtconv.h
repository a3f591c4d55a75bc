/*
 * wtconv.h -- C ABI of libwtconv, the WTConv layer (wavelet convolution) for
 * AMD Instinct MI355X (gfx950), forward and backward.
 *
 * The layer, per channel c of an NCHW activation x (source: "Fast and
 * Memory-Efficient Wavelet Convolutions via I/O-Aware Reformulation", arXiv
 * 2608.10805; its English abstract describes WTConv as a drop-in replacement
 * for a depthwise convolution, and the technical summary's Methodology section
 * describes the analysis, the per-level convolutions with learned per-channel
 * scales, and the synthesis cascade):
 *
 *   y = s0[c] * (W0[c] (*) x + b0[c])
 *     + sum over levels l = 1..L of the Haar synthesis, from level l back to full
 *       resolution, of Z_l^b = s_l[4c+b] * (W_l[4c+b] (*) A_l^b),  b = 0..3,
 *
 * where A_l^0..3 are the four subbands of the orthonormal 2D Haar analysis
 * (2x2 taps of +-1/2) of the level-(l-1) low-pass band (level 0 is x itself),
 * (*) is a k x k cross-correlation with zero 'same' padding at the level's own
 * resolution, and the synthesis of level l adds the reconstruction of level l+1
 * into the low-pass band before its inverse Haar step.  Band order: 0 low-pass,
 * 1 top-row-minus-bottom-row, 2 left-column-minus-right-column, 3 diagonal.
 *
 * Layout
 *   activations  x, y, dy, dx: NCHW contiguous, fp32 (WTCONV_F32) or fp16
 *                (WTCONV_F16) per the descriptor; device memory, 16-byte aligned.
 *   parameters   always fp32, device memory:
 *                w_base [C][k][k], bias [C] (may be NULL: zero bias), s_base [C],
 *                w_lvl [L][4C][k][k] and s_lvl [L][4C] with band b of channel c
 *                at index 4c+b (both may be NULL when L == 0).
 *   gradients    fp32, same shapes as their parameters; OVERWRITTEN, never
 *                accumulated.  dw/ds are gradients of the raw (unfolded)
 *                weights and scales.
 * Shape rules  n, c, h, w >= 1; k in {1, 3, 5, 7}; 0 <= L <= WTCONV_MAX_LEVELS;
 *              h, w and their round-up to multiples of 2^L <= WTCONV_MAX_SIDE.
 * Odd maps     Where 2^L does not divide h or w, every level map with an odd
 *              side is padded with one zero row (bottom) / column (right)
 *              before its Haar analysis and that level's synthesis is cropped
 *              back, so level l is ceil(h / 2^l) x ceil(w / 2^l) (the pages do
 *              not treat odd sides; this is the reading taken).  The library
 *              computes it as the layer on copies zero-padded to multiples of
 *              2^L, cropped, which is the same operator; all three calls then
 *              need a workspace (two padded activation copies plus the padded
 *              layer's own workspace).  The unfused baseline requires 2^L to
 *              divide h and w.
 * fp16 mode    fp16 storage of activations only: every product and sum is fp32,
 *              each output element is rounded once to fp16 (round to nearest
 *              even).
 * Ownership    The caller allocates every buffer, including the workspace
 *              (size from wtconv_workspace_size, 256-byte aligned; its contents
 *              need no initialisation and are scratch after the call).  The
 *              library allocates no device memory and holds no state between
 *              calls; calls are reentrant.  The one exception is
 *              wtconv_backward_weight_noalloc, whose partial results live in a
 *              static device array of the library (see there).
 * Execution    All work is enqueued on `stream` (0 = the null stream) with no
 *              host synchronisation; outputs are ready when the stream reaches
 *              that point.  Inputs and outputs must not overlap (y != x,
 *              dx != dy).  Results are bitwise reproducible run to run (no
 *              floating-point atomics).  Only kernels are enqueued (no memset,
 *              copy or allocation), so calls may be captured into a HIP graph
 *              on a capturing stream and replayed; the workspace and buffers
 *              captured must then stay allocated.
 * Errors       Arguments are validated before any HIP call; a bad argument
 *              returns its status code and enqueues nothing.  A failed kernel
 *              launch returns WTCONV_ERR_HIP.  Asynchronous faults are reported
 *              by the HIP runtime at the caller's next synchronisation.
 */
#ifndef WTCONV_H
#define WTCONV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define WTCONV_MAX_LEVELS 6
#define WTCONV_MAX_SIDE 4096

typedef enum {
    WTCONV_OK = 0,
    WTCONV_ERR_NULL = 1,        /* a required pointer is NULL */
    WTCONV_ERR_SHAPE = 2,       /* sizes, levels or divisibility rule violated */
    WTCONV_ERR_UNSUPPORTED = 3, /* kernel size or dtype not built */
    WTCONV_ERR_WORKSPACE = 4,   /* workspace missing or smaller than required */
    WTCONV_ERR_HIP = 5,         /* the HIP runtime rejected a launch */
    WTCONV_ERR_ALIAS = 6        /* an output overlaps an input */
} wtconv_status_t;

typedef enum { WTCONV_F32 = 0, WTCONV_F16 = 1 } wtconv_dtype_t;

typedef enum {
    WTCONV_OP_FWD = 0,
    WTCONV_OP_BWD_DATA = 1,
    WTCONV_OP_BWD_WEIGHT = 2,
    WTCONV_OP_BWD = 3  /* wtconv_backward: dx and all parameter gradients */
} wtconv_op_t;

typedef struct {
    int64_t n, c, h, w;   /* activation shape, NCHW */
    int32_t k;            /* odd kernel size of the base and every per-level conv */
    int32_t levels;       /* number of Haar levels L */
    int32_t dtype;        /* wtconv_dtype_t of the activations */
} wtconv_desc_t;

/* hipStream_t without pulling in the HIP headers. */
typedef struct ihipStream_t *wtconv_stream_t;

/* Bytes of device workspace `op` needs for `desc` on the current device.  The
 * forward and the data backward need none when a plane fits one workgroup
 * (or L <= 1) and 2^L divides h and w; for larger planes with L >= 2 they keep
 * the level-1 low-pass map and the deeper levels' term there, and for sides
 * 2^L does not divide the zero-padded copies of the input and output.  Errors
 * as for the op itself. */
wtconv_status_t wtconv_workspace_size(const wtconv_desc_t *desc, wtconv_op_t op, size_t *bytes);

/* y = WTConv(x).  The per-channel scales are folded into the weights (and the
 * base scale into the bias) on chip, the Haar analysis is recomputed on chip
 * from the staged input, and the synthesis of all levels is one closed-form
 * pass indexed by the bits of each output coordinate (technical summary,
 * Methodology, reformulations 1-3).  x is read once and y written once. */
wtconv_status_t wtconv_forward(const wtconv_desc_t *desc, const void *x, const float *w_base, const float *bias,
                               const float *s_base, const float *w_lvl, const float *s_lvl, void *y,
                               void *workspace, size_t workspace_bytes, wtconv_stream_t stream);

/* dx = d<dy, WTConv(x)>/dx.  The layer is linear in x and the orthonormal Haar
 * synthesis is the transpose of the analysis, so this is the same fused pass
 * on dy with every kernel turned by 180 degrees and no bias.  Forward outputs
 * and all gradients are part of the method (technical summary, Key
 * Contributions). */
wtconv_status_t wtconv_backward_data(const wtconv_desc_t *desc, const void *dy, const float *w_base,
                                     const float *s_base, const float *w_lvl, const float *s_lvl, void *dx,
                                     void *workspace, size_t workspace_bytes, wtconv_stream_t stream);

/* Parameter gradients of <dy, WTConv(x)>, with the chain rule through the
 * folded scales (technical summary, Methodology, reformulation 3):
 *   dw_base = s0 * G0,  dbias = s0 * Gb,  ds_base = <W0, G0> + b0 * Gb,
 *   dw_lvl  = s_l * G_l, ds_lvl = <W_l, G_l>   (per channel and band),
 * where G0 / G_l are the correlations, summed over N, H and W, of dy (or its
 * Haar analysis) with x (or its Haar analysis) and Gb = sum dy.  Needs the
 * workspace from wtconv_workspace_size(desc, WTCONV_OP_BWD_WEIGHT).  dw_lvl and
 * ds_lvl may be NULL when L == 0. */
wtconv_status_t wtconv_backward_weight(const wtconv_desc_t *desc, const void *x, const void *dy,
                                       const float *w_base, const float *bias, const float *s_base,
                                       const float *w_lvl, const float *s_lvl, float *dw_base, float *dbias,
                                       float *ds_base, float *dw_lvl, float *ds_lvl, void *workspace,
                                       size_t workspace_bytes, wtconv_stream_t stream);

/* dx and all parameter gradients in one call (technical summary, Key
 * Contributions: forward outputs and all parameter gradients).  By default it
 * runs wtconv_backward_data and then wtconv_backward_weight.  With
 * WTCONV_FUSED_BWD=1 in the environment, planes that fit one workgroup run as
 * one fused pass instead: x and dy are read once, dy's Haar pyramid is built
 * once on chip and serves both the data backward's convolution (kernels turned
 * by 180 degrees) and the correlation with x's pyramid, and dx is written once
 * (5 E e bytes of activation traffic instead of 6 E e).  On MI355X the fused
 * pass measured slower than the two calls (it holds both pyramids and the
 * accumulators, so fewer waves stay in flight), hence the default.  The
 * results are those of the two calls (to rounding).  Arguments as theirs; dx
 * must not overlap x or dy; the workspace is wtconv_workspace_size(desc,
 * WTCONV_OP_BWD) under the same environment. */
wtconv_status_t wtconv_backward(const wtconv_desc_t *desc, const void *x, const void *dy, const float *w_base,
                                const float *bias, const float *s_base, const float *w_lvl, const float *s_lvl,
                                void *dx, float *dw_base, float *dbias, float *ds_base, float *dw_lvl, float *ds_lvl,
                                void *workspace, size_t workspace_bytes, wtconv_stream_t stream);

/* ---- The weight backward without a workspace argument --------------------
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): the same
 * gradients as wtconv_backward_weight, with the partial results kept in a
 * static device array of WTCONV_NOALLOC_SCRATCH_BYTES bytes that the library
 * holds on every GPU it runs on until the process ends.  Nothing is allocated
 * by the call.  Calls whose workspace (wtconv_workspace_size(desc,
 * WTCONV_OP_BWD_WEIGHT)) exceeds the array return WTCONV_ERR_WORKSPACE before
 * anything is enqueued (planes that fit one workgroup need a few MB; the
 * large-plane paths with L >= 2 keep low-pass maps there and are refused).
 * All calls on one GPU share its array: calls that overlap on one GPU (on
 * different streams, or from several threads) race and give wrong gradients;
 * calls in stream order do not.  Other errors as for wtconv_backward_weight;
 * WTCONV_ERR_HIP if the array's device address cannot be obtained. */
#define WTCONV_NOALLOC_SCRATCH_BYTES (16u << 20)
wtconv_status_t wtconv_backward_weight_noalloc(const wtconv_desc_t *desc, const void *x, const void *dy,
                                               const float *w_base, const float *bias, const float *s_base,
                                               const float *w_lvl, const float *s_lvl, float *dw_base, float *dbias,
                                               float *ds_base, float *dw_lvl, float *ds_lvl, wtconv_stream_t stream);

/* ---- Unfused baseline (test and benchmark use only) ----------------------
 * The same layer composed of separate kernels with every intermediate in HBM:
 * per level a Haar analysis pass, a depthwise convolution pass and a scale
 * pass, then per level (deepest first) an add of the low-pass band and a
 * synthesis pass, and the base convolution, scale and final add (the
 * composition the pages measure the fused kernel against: technical summary,
 * Problem Statement, and its count of element moves).  The backward calls are
 * the step-by-step adjoints of that composition.  Same arguments as the fused
 * calls; the caller allocates one workspace of wtconv_unfused_workspace_size()
 * bytes (256-byte aligned) and passes the same workspace to all three calls:
 * the forward leaves its intermediates there and both backward calls read
 * them, so a backward call must follow a forward on the same inputs and
 * parameters.  Intermediates are stored in the activation type.  Errors:
 * WTCONV_ERR_SHAPE for an invalid descriptor, WTCONV_ERR_NULL for a missing
 * pointer, WTCONV_ERR_WORKSPACE when the workspace is too small,
 * WTCONV_ERR_HIP for a launch error. */
wtconv_status_t wtconv_unfused_workspace_size(const wtconv_desc_t *desc, size_t *bytes);
wtconv_status_t wtconv_unfused_forward(const wtconv_desc_t *desc, const void *x, const float *w_base,
                                       const float *bias, const float *s_base, const float *w_lvl,
                                       const float *s_lvl, void *y, void *workspace, size_t workspace_bytes,
                                       wtconv_stream_t stream);
wtconv_status_t wtconv_unfused_backward_data(const wtconv_desc_t *desc, const void *dy, const float *w_base,
                                             const float *s_base, const float *w_lvl, const float *s_lvl, void *dx,
                                             void *workspace, size_t workspace_bytes, wtconv_stream_t stream);
wtconv_status_t wtconv_unfused_backward_weight(const wtconv_desc_t *desc, const void *x, const void *dy,
                                               const float *w_base, const float *bias, const float *s_base,
                                               const float *w_lvl, const float *s_lvl, float *dw_base,
                                               float *dbias, float *ds_base, float *dw_lvl, float *ds_lvl,
                                               void *workspace, size_t workspace_bytes, wtconv_stream_t stream);

/* Human-readable name of a status code (static string). */
const char *wtconv_status_string(wtconv_status_t status);

/* Library version, "major.minor.patch". */
const char *wtconv_version(void);

#ifdef __cplusplus
}
#endif

#endif /* WTCONV_H */
