/*
 * igemm_conv.h -- forward 2-D convolution as an implicit GEMM on MI355X
 * (gfx950), behind a plain C ABI.
 *
 * The operation is the one documented on the page "dispatch_amd_4wave_conv2d"
 * (Modular kernel library, nn/conv/gpu/amd/dispatch):
 *   - summary: try to run a forward Conv2D on the GPU; report whether the call
 *     was handled or declined so the caller can fall back; with a residual
 *     source compute D = Conv(A, B) + beta * source in-kernel, where source is
 *     NHWC-contiguous with the output's shape;
 *   - Parameters: input type float8_e4m3fn, bfloat16 or float16; filter type
 *     equal to it; output bfloat16 for fp8 inputs, otherwise the input type;
 *     filter_is_fcrs selects the FCRS or RSCF filter layout;
 *   - Args: NHWC input, FCRS or RSCF filter, NHWC output; stride (1,1) or
 *     (2,2); dilation (1,1); symmetric padding (0,0), (1,1) or (2,2); one group.
 * The filter is first transposed into the (C_out, K = R*S*C_in) "NK" matrix,
 * and the GEMM gathers its other operand from the NHWC input on the fly so no
 * im2col matrix is written to memory (page "dispatch_fused_im2col_conv2d_apple",
 * summary).
 *
 * Definition computed (cross-correlation, zero padding on both sides):
 *   y[n,oh,ow,co] = sum_{r<R, s<S, ci<C_in}
 *                     x[n, oh*st - p + r, ow*st - p + s, ci] * W(r, s, ci, co)
 *   Ho = floor((H + 2p - R) / st) + 1,  Wo = floor((W + 2p - S) / st) + 1
 *   D  = y + beta * source  (when source != NULL), one rounding to the output
 *        type at the end (round to nearest even); accumulation is fp32.
 *
 * Conventions for every entry point:
 *   - All tensor pointers are device pointers to caller-owned memory
 *     (hipMalloc / torch allocations).  The library keeps no tensor state.
 *   - Shapes are int64 arrays: in_nhwc = {N, H, W, C_in};
 *     filt_dims is the filter's stored shape: {R, S, C_in, C_out} for RSCF
 *     (filter_is_fcrs = 0) or {C_out, C_in, R, S} for FCRS (filter_is_fcrs = 1);
 *     out_nhwc = {N, Ho, Wo, C_out}.  All tensors are densely packed.
 *   - stride, dilation, padding are int32 pairs {height, width}.
 *   - stream is a hipStream_t passed as void* (NULL = the null stream).  Work
 *     is enqueued asynchronously; the caller synchronizes.
 *   - No exceptions cross the ABI; the functions are thread-safe.
 */
#ifndef IGEMM_CONV_H
#define IGEMM_CONV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element type codes (page "dispatch_amd_4wave_conv2d", Parameters). */
enum {
    IGC_DTYPE_BF16 = 0,        /* bfloat16 in, bfloat16 out            */
    IGC_DTYPE_FP16 = 1,        /* float16 in, float16 out              */
    IGC_DTYPE_FP8_E4M3FN = 2   /* OCP float8 e4m3fn in, bfloat16 out   */
};

/* Reasons a call is declined (0 = accepted).  The first five follow the
 * page's rules; the rest are this library's own limits. */
enum {
    IGC_OK = 0,
    IGC_DECLINE_DTYPE = 1,         /* dtype code not one of the three        */
    IGC_DECLINE_STRIDE = 2,        /* stride not (1,1) or (2,2)              */
    IGC_DECLINE_DILATION = 3,      /* dilation not (1,1)                     */
    IGC_DECLINE_PADDING = 4,       /* padding not (0,0), (1,1) or (2,2)      */
    IGC_DECLINE_GROUPS = 5,        /* groups not 1                           */
    IGC_DECLINE_SHAPE = 6,         /* negative dims, R or S < 1, or the
                                      filter's C_in differs from the input's */
    IGC_DECLINE_OUTPUT_SHAPE = 7,  /* Ho or Wo < 1, or out_nhwc is not
                                      {N, Ho, Wo, C_out}                     */
    IGC_DECLINE_VECTOR_WIDTH = 8,  /* C_in * element bytes not a multiple of
                                      16: conv2d_im2col only (it moves
                                      16-byte vectors); the convolutions
                                      take any C_in (an element-wise gather) */
    IGC_DECLINE_ALIGNMENT = 9,     /* a tensor pointer not 16-byte aligned   */
    IGC_DECLINE_NULL_POINTER = 10, /* NULL pointer for a non-empty tensor,
                                      or NULL shape/parameter array          */
    IGC_DECLINE_OVERLAP = 11,      /* output overlaps input, filter or
                                      workspace; workspace overlaps input,
                                      filter or source; or source overlaps
                                      output without being exactly it        */
    IGC_DECLINE_WORKSPACE = 12,    /* workspace given but smaller than
                                      conv2d_workspace_bytes()               */
    IGC_DECLINE_SIZE_LIMIT = 13,   /* a size beyond the kernels' 32-bit index
                                      ranges (see conv2d_fwd_check)          */
    IGC_DECLINE_EPILOGUE = 14      /* fused epilogue: unknown activation,
                                      scale/bias not 4-byte aligned, or
                                      scale/bias overlapping the output or
                                      the workspace                          */
};

/*
 * Fused elementwise epilogue.  Page "dispatch_amd_4wave_conv2d" (Parameters:
 * elementwise_lambda_fn) lets the caller fuse an elementwise function into
 * the convolution's epilogue, called per output element with its (m, co)
 * coordinates; page "dispatch_fused_im2col_conv2d_apple" (Parameters:
 * maybe_epilogue_func) does the same in NHWC coordinates.  A C ABI cannot
 * carry a device closure, so this library offers one fixed family, per
 * output element (n, oh, ow, co), in fp32:
 *   v = scale[co] * conv + bias[co]
 *   v = v + beta * source          (when source != NULL)
 *   v = act(v)                     relu: v if v > 0 else +0
 *                                  silu: v / (1 + exp(-v))
 *   output = round_to_nearest_even(v)
 * scale and bias are device arrays of C_out floats (caller-owned, 4-byte
 * aligned, not overlapping the output), either may be NULL (1 and 0).
 * A NULL igc_epilogue pointer, or {NULL, NULL, IGC_ACT_NONE}, is exactly
 * conv2d_fwd / conv2d_fwd_nk.
 */
enum {
    IGC_ACT_NONE = 0,
    IGC_ACT_RELU = 1,
    IGC_ACT_SILU = 2
};

typedef struct igc_epilogue {
    const float* scale;    /* [C_out] or NULL */
    const float* bias;     /* [C_out] or NULL */
    int32_t activation;    /* IGC_ACT_* */
} igc_epilogue;

/* Version of this ABI. */
int32_t conv2d_abi_version(void);

/* Build flags of this library: bit 0 set in the LDS-poison debug build
 * (libigemmconv_ldspoison.so), whose kernels first fill their LDS with 0xFF
 * bytes (NaN in every element type) so that a read running ahead of its data
 * shows up as NaN outputs; 0 in the normal build. */
int32_t conv2d_build_flags(void);

/* Human-readable name of a decline reason code (static string). */
const char* conv2d_reason_string(int32_t reason);

/*
 * Pointer-free acceptance check of a problem's shapes and parameters (no
 * HIP call): page "dispatch_amd_4wave_conv2d" (Parameters and Args: element
 * types, stride, dilation, symmetric padding, groups, NHWC output shape) plus
 * this library's size limits (IGC_DECLINE_SIZE_LIMIT).  Returns IGC_OK or
 * the decline reason; a call
 * with these shapes is then accepted unless its pointers fail the rules of
 * conv2d_fwd_check (alignment, NULL, overlap, workspace size).
 */
int32_t conv2d_fwd_query(const int64_t in_nhwc[4], int32_t filter_is_fcrs,
                         const int64_t filt_dims[4], const int64_t out_nhwc[4],
                         const int32_t stride[2], const int32_t dilation[2],
                         const int32_t padding[2], int32_t groups, int32_t dtype);

/*
 * Host-only acceptance check (no HIP call, no memory access): the gate of
 * the page's dispatcher plus this library's limits.  Pointers are only
 * compared and tested for alignment, never dereferenced.  workspace may be
 * NULL (the library then allocates).  Returns IGC_OK or a decline reason.
 * Size limits: N*Ho*Wo, C_out, R*S*C_in, and (R*W + S)*C_in each below 2^31,
 * and the NK matrix (conv2d_workspace_bytes) below 2^31 bytes.
 */
int32_t conv2d_fwd_check(const void* input, const int64_t in_nhwc[4],
                         const void* filter, int32_t filter_is_fcrs,
                         const int64_t filt_dims[4],
                         const void* output, const int64_t out_nhwc[4],
                         const int32_t stride[2], const int32_t dilation[2],
                         const int32_t padding[2], int32_t groups,
                         int32_t dtype, const void* source, float beta,
                         const void* workspace, size_t workspace_bytes);

/*
 * Forward convolution (page "dispatch_amd_4wave_conv2d", whole page).
 *   input    [N, H, W, C_in] of dtype.
 *   filter   RSCF or FCRS (filter_is_fcrs) of dtype.
 *   output   [N, Ho, Wo, C_out] of the output type; fully overwritten.
 *   source   NULL, or [N, Ho, Wo, C_out] of the output type; then
 *            output = conv + beta * source.  source == output (in place) is
 *            allowed.  beta is applied literally (IEEE: 0 * NaN is NaN).
 *   workspace  device scratch for the NK filter of at least
 *            conv2d_workspace_bytes() bytes; NULL makes the library take it
 *            stream-ordered from hipMallocAsync and release it with
 *            hipFreeAsync on the same stream.
 * Enqueues the filter transpose and the implicit-GEMM kernel on stream.
 * Returns 1 = handled (work enqueued), 0 = declined (nothing enqueued, no
 * memory touched; conv2d_fwd_check gives the reason), or -(hipError_t) if a
 * HIP call failed.
 */
int32_t conv2d_fwd(const void* input, const int64_t in_nhwc[4],
                   const void* filter, int32_t filter_is_fcrs,
                   const int64_t filt_dims[4],
                   void* output, const int64_t out_nhwc[4],
                   const int32_t stride[2], const int32_t dilation[2],
                   const int32_t padding[2], int32_t groups,
                   int32_t dtype, const void* source, float beta,
                   void* workspace, size_t workspace_bytes, void* stream);

/*
 * conv2d_fwd for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation): the
 * NK filter matrix goes to a static device scratch array of the library,
 * IGC_NOALLOC_SCRATCH_BYTES bytes per GPU, held until the process ends; no
 * hipMalloc, hipFree or other allocating call is made.  Arguments as
 * conv2d_fwd without the workspace.  Returns 1 = handled, 0 = declined
 * (conv2d_fwd_check with a NULL workspace gives the reason, or the NK
 * matrix, conv2d_workspace_bytes(), exceeds IGC_NOALLOC_SCRATCH_BYTES), or
 * -(hipError_t).  The first call on each device looks up the scratch's
 * device address (make it outside graph capture).  Every call on one GPU
 * shares its scratch: calls that overlap in time on one GPU (other streams,
 * other threads) race and must be ordered by the caller.
 */
#define IGC_NOALLOC_SCRATCH_BYTES ((size_t)8 << 20)
int32_t conv2d_fwd_noalloc(const void* input, const int64_t in_nhwc[4],
                           const void* filter, int32_t filter_is_fcrs,
                           const int64_t filt_dims[4],
                           void* output, const int64_t out_nhwc[4],
                           const int32_t stride[2], const int32_t dilation[2],
                           const int32_t padding[2], int32_t groups,
                           int32_t dtype, const void* source, float beta, void* stream);

/*
 * Name of the GEMM kernel conv2d_fwd / conv2d_fwd_nk launch for this problem
 * (a static string: "igemm_fwd_tapfold_kernel", "igemm_fwd_band_kernel",
 * "igemm_fwd_patch_kernel", "igemm_fwd_wide_kernel",
 * "igemm_fwd_resident_kernel", "igemm_fwd_kernel", or "none" when nothing is
 * launched because the output is empty), or NULL when the shapes or
 * parameters would be declined.  Host-only; pointers play no part (their
 * checks come on top, see conv2d_fwd_check).  A selection rule of this
 * library (page 1 names only its own 4-wave kernel), reported so that
 * profiles and measurements can name what ran.  The name is the one for an
 * MI355X (256 CUs, 160 KB of LDS per CU); a launch plans with the figures
 * of the device it runs on.
 */
const char* conv2d_fwd_kernel_name(const int64_t in_nhwc[4], int32_t filter_is_fcrs,
                                   const int64_t filt_dims[4], const int64_t out_nhwc[4],
                                   const int32_t stride[2], const int32_t dilation[2],
                                   const int32_t padding[2], int32_t groups, int32_t dtype);

/*
 * Bytes of the NK filter matrix: C_out rows of conv2d_nk_row_pitch()
 * elements each.  0 for an invalid dtype or negative dims.
 */
size_t conv2d_workspace_bytes(const int64_t filt_dims[4],
                              int32_t filter_is_fcrs, int32_t dtype);

/*
 * Elements per NK row: K = R*S*C_in rounded up to a multiple of
 * 128 bytes' worth of elements (64 for bf16/fp16, 128 for fp8); for
 * C_out <= 64 plus 16 bytes of zeros (8 or 16 elements) that keep LDS
 * copies of the rows free of bank conflicts.  Wider filters keep rows a
 * whole number of 128-byte lines.
 */
int64_t conv2d_nk_row_pitch(const int64_t filt_dims[4], int32_t filter_is_fcrs,
                            int32_t dtype);

/*
 * Filter transpose alone (page "dispatch_fused_im2col_conv2d_apple", summary:
 * the filter becomes the (C_out, K = R*S*C_in) NK matrix):
 *   nk[co * pitch + (r*S + s)*C_in + ci] = W(r, s, ci, co)   for k < K
 *   nk[co * pitch + k] = 0                                     for K <= k < pitch
 * with pitch = conv2d_nk_row_pitch().  A bit copy: values are not converted.
 * nk must be 16-byte aligned and hold nk_bytes >= conv2d_workspace_bytes().
 * Returns 1 = enqueued, 0 = declined (bad dtype/dims/pointers, too small,
 * or an NK matrix of 2^31 bytes or more), or -(hipError_t).
 */
int32_t conv2d_filter_to_nk(const void* filter, int32_t filter_is_fcrs,
                            const int64_t filt_dims[4], int32_t dtype,
                            void* nk, size_t nk_bytes, void* stream);

/*
 * The implicit-GEMM kernel alone, on an NK matrix made by
 * conv2d_filter_to_nk from a filter of shape filt_dims / filter_is_fcrs.
 * Arguments and returns as conv2d_fwd, with nk in place of the filter and no
 * workspace.  The gather, the MFMA contraction, the edge masks and the fused
 * residual epilogue all run in this one launch.
 */
int32_t conv2d_fwd_nk(const void* input, const int64_t in_nhwc[4],
                      const void* nk, int32_t filter_is_fcrs,
                      const int64_t filt_dims[4],
                      void* output, const int64_t out_nhwc[4],
                      const int32_t stride[2], const int32_t dilation[2],
                      const int32_t padding[2], int32_t groups,
                      int32_t dtype, const void* source, float beta,
                      void* stream);

/*
 * conv2d_fwd with the fused elementwise epilogue above (epilogue may be
 * NULL).  Arguments and returns otherwise as conv2d_fwd; a call whose
 * epilogue fails conv2d_epilogue_check is declined (0).
 */
int32_t conv2d_fwd_epilogue(const void* input, const int64_t in_nhwc[4],
                            const void* filter, int32_t filter_is_fcrs,
                            const int64_t filt_dims[4],
                            void* output, const int64_t out_nhwc[4],
                            const int32_t stride[2], const int32_t dilation[2],
                            const int32_t padding[2], int32_t groups,
                            int32_t dtype, const void* source, float beta,
                            const igc_epilogue* epilogue,
                            void* workspace, size_t workspace_bytes, void* stream);

/* conv2d_fwd_nk with the fused elementwise epilogue (may be NULL). */
int32_t conv2d_fwd_nk_epilogue(const void* input, const int64_t in_nhwc[4],
                               const void* nk, int32_t filter_is_fcrs,
                               const int64_t filt_dims[4],
                               void* output, const int64_t out_nhwc[4],
                               const int32_t stride[2], const int32_t dilation[2],
                               const int32_t padding[2], int32_t groups,
                               int32_t dtype, const void* source, float beta,
                               const igc_epilogue* epilogue, void* stream);

/*
 * Host-only gate of conv2d_fwd_epilogue (no HIP call, no memory access):
 * conv2d_fwd_check's rules, then the epilogue's (conv2d_epilogue_check),
 * and scale / bias must not overlap the workspace (the filter transpose
 * writes it before the GEMM reads them).  Returns IGC_OK or a decline
 * reason; conv2d_fwd_epilogue declines exactly when this is not IGC_OK.
 */
int32_t conv2d_fwd_epilogue_check(const void* input, const int64_t in_nhwc[4],
                                  const void* filter, int32_t filter_is_fcrs,
                                  const int64_t filt_dims[4], const void* output,
                                  const int64_t out_nhwc[4], const int32_t stride[2],
                                  const int32_t dilation[2], const int32_t padding[2],
                                  int32_t groups, int32_t dtype, const void* source, float beta,
                                  const igc_epilogue* epilogue, const void* workspace,
                                  size_t workspace_bytes);

/*
 * Host-only check of an epilogue against an output of shape out_nhwc
 * (pointers compared, never dereferenced): IGC_OK, IGC_DECLINE_EPILOGUE,
 * IGC_DECLINE_NULL_POINTER (out_nhwc NULL) or IGC_DECLINE_SHAPE (negative
 * dims).  A NULL epilogue is IGC_OK.
 */
int32_t conv2d_epilogue_check(const igc_epilogue* epilogue, const void* output,
                              const int64_t out_nhwc[4]);

/*
 * Materialised im2col, for measuring what the fused gather saves (page
 * "dispatch_fused_im2col_conv2d_apple", summary: the fused kernel gathers
 * the [M, K] patch matrix on the fly instead of writing it to memory and
 * running a GEMM over it).  Writes
 *   A[m][k] = x[n, oh*st - p + r, ow*st - p + s, ci]   (0 in the padding)
 * with m = (n*Ho + oh)*Wo + ow and k = (r*S + s)*C_in + ci, in rows of Kp
 * elements: K = R*S*C_in rounded up to a multiple of 128 bytes, zero past K.
 * A bit copy of the input's elements.  filt_rs = {R, S}; the shape rules
 * (dtype, stride, padding, Ho/Wo >= 1, C_in * element bytes % 16 == 0) are
 * conv2d_fwd's.  a_out: device memory of at least conv2d_im2col_bytes(),
 * 16-byte aligned, not overlapping the input.
 * Read as an NHWC tensor [N, Ho, Wo, Kp], A is the input of a 1x1, stride-1,
 * padding-0 convolution whose NK matrix is the one conv2d_filter_to_nk makes
 * from the original filter: conv2d_fwd_nk with in_nhwc = {N, Ho, Wo, Kp} and
 * FCRS filt_dims = {C_out, Kp, 1, 1} then computes the same convolution.
 * Returns 1 = enqueued (or nothing to do), 0 = declined, or -(hipError_t).
 */
int32_t conv2d_im2col(const void* input, const int64_t in_nhwc[4],
                      const int64_t filt_rs[2], const int32_t stride[2],
                      const int32_t padding[2], int32_t dtype,
                      void* a_out, size_t a_bytes, void* stream);

/* Bytes of the im2col matrix: N*Ho*Wo*Kp elements; 0 if declined. */
size_t conv2d_im2col_bytes(const int64_t in_nhwc[4], const int64_t filt_rs[2],
                           const int32_t stride[2], const int32_t padding[2],
                           int32_t dtype);

/*
 * Transposed convolution (page "conv_transposed_gpu": NHWC input, filter in
 * RSFC layout [R][S][F][C] with F output and C input channels, stride,
 * dilation and padding per spatial axis; the page runs it through cuDNN's
 * backward-data path and applies an elementwise epilogue as a separate
 * pass).  Definition, cross-correlation form, per axis stride st, dilation
 * d and padding p cut from both ends:
 *   out[n, oh, ow, f] = sum over (ih, iw, r, s, c) with
 *                         oh = ih*sh - ph + r*dh,  ow = iw*sw - pw + s*dw
 *                       of in[n, ih, iw, c] * W[r][s][f][c]
 *   Ho = (H - 1)*sh - 2ph + dh*(R - 1) + 1, likewise Wo
 * i.e. the adjoint of the forward convolution whose RSCF filter is W.  Then
 * the same fused epilogue as conv2d_fwd_epilogue (scale, bias, residual
 * source, activation; all optional) and one rounding.
 * Any stride, dilation and padding (each >= 1, >= 1, >= 0) and any R, S.
 * Along each axis the output rows of phase a (oh = st*q + a) take the taps
 * r with r*d = a + p (mod st); each (row phase, column phase) pair is one
 * forward implicit GEMM over the input with that tap subset flipped and the
 * channel roles swapped (the NK transpose does both), which stores through
 * an output map straight into its rows and columns of the output and reads
 * the residual source there: no intermediate buffers, every output element
 * gets the fused epilogue and one rounding in a GEMM.  A phase without taps
 * gets the epilogue alone.  When all phases have one shape (strides 1 and 2
 * among others) they run as one launch.
 * Any C (C * element bytes not a multiple of 16: the phases run on the
 * tiled kernel's element gather).  Library limits: (H-1)*sh + dh*(R-1)
 * + 1, the same along W, and the padding below 2^30; sh*sw <= 4096 phases;
 * (33*sh*Wo + 32*sw) * F * 2 below 2^31 bytes; each phase's forward problem
 * within conv2d_fwd_check's size limits (IGC_DECLINE_SIZE_LIMIT).  Dtypes,
 * alignment and overlap rules as conv2d_fwd.
 *   in_nhwc = {N, H, W, C}, filt_rsfc = {R, S, F, C}, out_nhwc = {N, Ho, Wo, F}
 *   workspace: at least conv2d_transposed_workspace_bytes() (the phases' NK
 *   matrices), or NULL (stream-ordered allocation as in conv2d_fwd);
 *   source == output is allowed.
 * Returns 1 = handled, 0 = declined (conv2d_transposed_check gives the
 * reason), or -(hipError_t).
 */
int32_t conv2d_transposed_fwd(const void* input, const int64_t in_nhwc[4],
                              const void* filter, const int64_t filt_rsfc[4],
                              void* output, const int64_t out_nhwc[4],
                              const int32_t stride[2], const int32_t dilation[2],
                              const int32_t padding[2], int32_t dtype,
                              const void* source, float beta,
                              const igc_epilogue* epilogue,
                              void* workspace, size_t workspace_bytes, void* stream);

/* Host-only gate of conv2d_transposed_fwd: IGC_OK or a decline reason. */
int32_t conv2d_transposed_check(const void* input, const int64_t in_nhwc[4],
                                const void* filter, const int64_t filt_rsfc[4],
                                const void* output, const int64_t out_nhwc[4],
                                const int32_t stride[2], const int32_t dilation[2],
                                const int32_t padding[2], int32_t dtype,
                                const void* source, float beta,
                                const igc_epilogue* epilogue,
                                const void* workspace, size_t workspace_bytes);

/* Workspace conv2d_transposed_fwd needs for this problem (the phases' NK
 * matrices); 0 if the problem would be declined. */
size_t conv2d_transposed_workspace_bytes(const int64_t in_nhwc[4], const int64_t filt_rsfc[4],
                                         const int32_t stride[2], const int32_t dilation[2],
                                         const int32_t padding[2], int32_t dtype);

/*
 * General forward convolution: the parameters that page
 * "dispatch_amd_4wave_conv2d" (Args: stride, dilation, symmetric_padding,
 * num_groups) names and its dispatcher restricts, here all accepted within
 * the limits below.  Definition (cross-correlation, zero padding):
 *   y[n,oh,ow,co] = sum_{r<R, s<S, c<Cg}
 *                     x[n, oh*sh - pt + r*dh, ow*sw - pl + s*dw, g*Cg + c] * W(r, s, c, co)
 *   g  = co / (C_out / groups),  Cg = C_in / groups
 *   Ho = floor((H + pt + pb - dh*(R-1) - 1) / sh) + 1, likewise Wo with
 *        (W, pl, pr, dw, S, sw)
 * then the fused epilogue of conv2d_fwd_epilogue (scale, bias, residual
 * source, activation; all optional; scale / bias indexed by co over all
 * C_out channels) and one rounding.
 *   filter     RSCF {R, S, Cg, C_out} or FCRS {C_out, Cg, R, S} (the filter's
 *              C_in is the per-group count, as in every framework's grouped
 *              convolution); filt_dims is that stored shape.
 *   params     stride >= 1, dilation >= 1, padding >= 0 before (top, left)
 *              and after (bottom, right) each axis, groups >= 1 dividing
 *              C_in and C_out.
 *   workspace  conv2d_fwd_general_workspace_bytes(...) bytes for this
 *              problem (its NK matrix), or NULL for a stream-ordered
 *              allocation.
 * A problem inside the page's gate (one group, unit dilation, stride (1,1)
 * or (2,2), equal padding 0, 1 or 2 on every side) runs exactly as
 * conv2d_fwd_epilogue; one group at unit dilation and equal strides (any)
 * with other paddings or strides runs on the same forward kernels.  Several groups at
 * unit dilation and stride (1,1) or (2,2) run as super-groups on the band
 * kernel where it admits them: q consecutive groups become one problem of
 * q*Cg input and q*Fg output channels with a block-diagonal NK matrix
 * (zeros between different groups' channels), q*Fg <= 64 and q*Cg *
 * element bytes a power-of-two multiple of 32 (64 for fp8).  One group at
 * stride 1 whose dilation divides the padding before each axis and the
 * input and output extents runs on the band kernel as dh*dw dilation
 * phases (each an undilated convolution over every dh-th input row and
 * dw-th column, stored through an output map; one grouped launch, the
 * plain NK matrix).  Any other
 * problem runs on the tiled implicit-GEMM kernel, all groups in one launch
 * (as does any problem whose Cg * element bytes is not a multiple of 16:
 * the tiled kernel then gathers element by element).  Library limits: H + pt + pb,
 * W + pl + pr, dh*(R-1) and
 * dw*(S-1) below 2^30, and conv2d_fwd_check's size limits with Cg for C_in
 * (IGC_DECLINE_SIZE_LIMIT).  Decline codes: STRIDE, DILATION, PADDING,
 * GROUPS (groups < 1 or not dividing C_out), SHAPE (C_in != groups * Cg),
 * and the pointer rules of conv2d_fwd_epilogue_check.
 * Returns 1 = handled, 0 = declined (conv2d_fwd_general_check gives the
 * reason), or -(hipError_t).
 */
typedef struct igc_conv_params {
    int32_t stride[2];      /* {sh, sw} */
    int32_t dilation[2];    /* {dh, dw} */
    int32_t pad_begin[2];   /* {pt, pl}: zero rows above, columns left */
    int32_t pad_end[2];     /* {pb, pr}: zero rows below, columns right */
    int32_t groups;
} igc_conv_params;

int32_t conv2d_fwd_general(const void* input, const int64_t in_nhwc[4],
                           const void* filter, int32_t filter_is_fcrs,
                           const int64_t filt_dims[4],
                           void* output, const int64_t out_nhwc[4],
                           const igc_conv_params* params, int32_t dtype,
                           const void* source, float beta,
                           const igc_epilogue* epilogue,
                           void* workspace, size_t workspace_bytes, void* stream);

/* Host-only gate of conv2d_fwd_general (pointers compared, never
 * dereferenced): IGC_OK or a decline reason. */
int32_t conv2d_fwd_general_check(const void* input, const int64_t in_nhwc[4],
                                 const void* filter, int32_t filter_is_fcrs,
                                 const int64_t filt_dims[4],
                                 const void* output, const int64_t out_nhwc[4],
                                 const igc_conv_params* params, int32_t dtype,
                                 const void* source, float beta,
                                 const igc_epilogue* epilogue,
                                 const void* workspace, size_t workspace_bytes);

/* Pointer-free gate of conv2d_fwd_general's shapes and parameters. */
int32_t conv2d_fwd_general_query(const int64_t in_nhwc[4], int32_t filter_is_fcrs,
                                 const int64_t filt_dims[4], const int64_t out_nhwc[4],
                                 const igc_conv_params* params, int32_t dtype);

/* Name of the GEMM kernel conv2d_fwd_general launches for this problem
 * (as conv2d_fwd_kernel_name), or NULL when it would be declined. */
const char* conv2d_fwd_general_kernel_name(const int64_t in_nhwc[4], int32_t filter_is_fcrs,
                                           const int64_t filt_dims[4],
                                           const int64_t out_nhwc[4],
                                           const igc_conv_params* params, int32_t dtype);

/* 1 when conv2d_fwd / conv2d_fwd_epilogue run this problem as one kernel
 * launch that transposes the stored filter into its LDS itself (no NK
 * matrix, the workspace is not touched): problems on the band kernel in
 * bf16 or fp16 with an RSCF filter of C_out a multiple of 8, or an FCRS
 * filter of R*S 1 or 9.  0 when a filter transpose launch into the
 * workspace precedes the GEMM kernel, or when the problem would be
 * declined.  conv2d_fwd_general does the same for its problems of one
 * group on the band kernel.  A library choice (page
 * "dispatch_fused_im2col_conv2d_apple", summary, transposes the filter once
 * ahead of the GEMM); the results are the same bits either way. */
int32_t conv2d_fwd_filter_in_kernel(const int64_t in_nhwc[4], int32_t filter_is_fcrs,
                                    const int64_t filt_dims[4], const int64_t out_nhwc[4],
                                    const int32_t stride[2], const int32_t dilation[2],
                                    const int32_t padding[2], int32_t groups, int32_t dtype);

/* Workspace conv2d_fwd_general needs for this problem: the NK matrix, C_out
 * rows of conv2d_nk_row_pitch's pitch for a K of R*S*Cg (plain groups) or
 * R*S*q*Cg (super-groups of q); 0 when the problem would be declined. */
size_t conv2d_fwd_general_workspace_bytes(const int64_t in_nhwc[4], int32_t filter_is_fcrs,
                                          const int64_t filt_dims[4],
                                          const int64_t out_nhwc[4],
                                          const igc_conv_params* params, int32_t dtype);

#ifdef __cplusplus
}
#endif

#endif /* IGEMM_CONV_H */
