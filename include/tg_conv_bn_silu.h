/*
 * tg_conv_bn_silu.h -- C ABI of the fused conv2d + BatchNorm + SiLU library
 * for AMD Instinct MI355X (gfx950). Library: libtgconv.so.
 *
 * The operation ("Fusing an Epilogue", teenygrad docs, sections "The problem"
 * and "The shape of it"): a 2-D convolution whose output, while still in
 * registers, is scaled and shifted per output channel (inference BatchNorm
 * folded to one scale and one bias per channel) and passed through
 * SiLU(v) = v * sigmoid(v), then stored once:
 *
 *   acc[n,p,q,k] = sum_{r<kh, s<kw, c<C_in} x[n, p*stride-pad+r, q*stride-pad+s, c] * w[k,r,s,c]
 *                  (x is zero outside [0,H) x [0,W); cross-correlation, no flip)
 *   v            = acc * bn_scale[k] + bn_bias[k]
 *   y[n,p,q,k]   = v * sigmoid(v)
 *
 * with P = floor((H + 2*pad - kh)/stride) + 1, Q = floor((W + 2*pad - kw)/stride) + 1.
 *
 * Layouts (all dense, no strides): x NHWC [N][H][W][C_in]; w OHWI
 * [C_out][kh][kw][C_in] (channels-last filters, stored that way once at load
 * time -- "When the fusion you want is impossible, fuse into the producer",
 * layout-conversion paragraph); y NHWC [N][P][Q][C_out]; bn_scale, bn_bias
 * fp32 [C_out]. x, w and y share one dtype (fp16 or fp32); accumulation and
 * the epilogue are fp32; fp16 results are rounded to nearest even.
 *
 * Ownership: the caller owns every device buffer. A plan owns host memory
 * only; create/destroy never touch device memory. Entry points never abort,
 * never print and never read the process environment (kernel-variant
 * overrides are explicit: tg_conv_bn_silu_create_tuned). run() and
 * bn_fold() are asynchronous on the given stream (a
 * hipStream_t passed as void*, NULL = the null stream) and do not
 * synchronise; launch failures are reported as TG_ERR_HIP.
 *
 * Thread safety: a plan is immutable after create; concurrent run() calls
 * with one plan on different streams are allowed. y must not alias x, w,
 * bn_scale, bn_bias or the workspace (not checked).
 */
#ifndef TG_CONV_BN_SILU_H
#define TG_CONV_BN_SILU_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct tg_conv_bn_silu_plan tg_conv_bn_silu_plan; /* opaque, host memory */

typedef enum {
    TG_OK = 0,
    TG_ERR_INVALID_ARGUMENT = 1, /* NULL pointer, non-positive size, window larger than padded input */
    TG_ERR_UNSUPPORTED = 2,      /* valid, but not served by the requested kernel or too large */
    TG_ERR_ALIGNMENT = 3,        /* a forced vector kernel got a pointer that is not 16-byte aligned */
    TG_ERR_WORKSPACE = 4,        /* unfused baseline: workspace missing or too small */
    TG_ERR_HIP = 5               /* a HIP runtime call or kernel launch failed */
} tg_status;

/* TG_F8_E4M3 is an output dtype only (tg_conv_bn_act_create_out): OCP FP8
 * E4M3 (1 sign, 4 exponent, 3 mantissa bits, bias 7, largest finite 448),
 * one byte per element, rounded to nearest even; results beyond +-448 are
 * outside the format and not specified. */
typedef enum { TG_F16 = 0, TG_F32 = 1, TG_F8_E4M3 = 2 } tg_dtype;

/* Kernel selection ("Fusing an Epilogue", section "Three kernels for one
 * operation": one scalar, one spatially tiled, one GEMM-shaped kernel, picked
 * by shape). A value may be OR-ed with TG_UNFUSED to run the three-kernel
 * baseline instead: that conv kernel with an identity epilogue writing t1,
 * then a BatchNorm kernel t1 -> t2, then a SiLU kernel t2 -> y ("The problem"
 * section of the same page). Or it may be OR-ed with TG_SPLIT for the split
 * form that "When not to fuse" (same page) and "Kernel Fusion" (cheatsheet
 * page, the passage on when fusion does not pay) weigh against the fused
 * one: the conv kernel with an identity epilogue writing t1, then one
 * BatchNorm+SiLU kernel t1 -> y. TG_UNFUSED and TG_SPLIT exclude each other. */
typedef enum {
    TG_KERNEL_AUTO = 0,   /* the dispatch table decides (see tg_dispatch_choose) */
    TG_KERNEL_SCALAR = 1, /* one output element per lane; any shape, fp16 and fp32 */
    TG_KERNEL_TILED = 2,  /* direct conv on an output-row band staged in LDS; fp16,
                             C_out <= 64, padded input row band must fit in LDS */
    TG_KERNEL_IGEMM = 3,  /* implicit GEMM on fp16 MFMA with the epilogue in registers;
                             fp16, C_in % 8 == 0 */
    TG_UNFUSED = 0x100,   /* flag: run conv, bn and silu as three kernels */
    TG_SPLIT = 0x200      /* flag: run conv, then bn+silu, as two kernels */
} tg_kernel;

/* Dispatch tables. TG_DISPATCH_MI355X (default) holds thresholds measured on
 * MI355X. TG_DISPATCH_PAGES reproduces the thresholds the teenygrad page
 * writes down ("Three kernels for one operation"): GEMM for 1x1 convolutions
 * with at least 32 output channels, else tiled for more than 16 output
 * channels, else scalar (reading the thresholds as counts of output channels). */
typedef enum { TG_DISPATCH_MI355X = 0, TG_DISPATCH_PAGES = 1 } tg_dispatch;

/* Build a plan for one shape. Host only: validates, computes P and Q, picks
 * the kernel (TG_KERNEL_AUTO: the default dispatch table) and its tile and
 * grid. Returns TG_ERR_INVALID_ARGUMENT for out == NULL, any size < 1,
 * pad < 0 or a window larger than the padded input; TG_ERR_UNSUPPORTED when
 * any of x, w, y has 2^31 or more elements, when a forced kernel does not
 * serve the shape or dtype, or for an unknown dtype/kernel value. On error
 * *out is set to NULL. */
tg_status tg_conv_bn_silu_create(tg_conv_bn_silu_plan **out, int N, int H, int W, int C_in,
                                 int C_out, int kh, int kw, int stride, int pad, tg_dtype dtype,
                                 tg_kernel kernel);

/* Same as create, choosing the AUTO kernel from the given dispatch table. */
tg_status tg_conv_bn_silu_create_with_table(tg_conv_bn_silu_plan **out, int N, int H, int W,
                                            int C_in, int C_out, int kh, int kw, int stride,
                                            int pad, tg_dtype dtype, tg_kernel kernel,
                                            tg_dispatch table);

/* Run the planned operation on `stream` -- conv, BatchNorm and SiLU in one
 * kernel whose epilogue works on the output tile while it is in registers
 * ("Fusing an Epilogue", section "The shape of it"), or the unfused / split
 * sequence the plan's kernel flags select. x, w, y: device pointers in the
 * plan's dtype and the layouts above; bn_scale, bn_bias: device fp32
 * [C_out] (from tg_bn_fold). workspace/workspace_bytes: device scratch for the
 * unfused baseline (two intermediates t1 and t2 of y's size) and the split
 * form (one intermediate t1); see tg_conv_bn_silu_query. Ignored and may be
 * NULL/0 for fused kernels. The workspace must not alias x, w or y.
 * Errors: TG_ERR_INVALID_ARGUMENT for a NULL plan or data pointer;
 * TG_ERR_ALIGNMENT when a forced tiled/igemm plan gets x, w or y not 16-byte
 * aligned (an AUTO plan falls back to the scalar kernel instead);
 * TG_ERR_WORKSPACE when the unfused or split workspace is NULL or too small;
 * TG_ERR_HIP when a launch fails. Nothing is launched on error. */
tg_status tg_conv_bn_silu_run(const tg_conv_bn_silu_plan *plan, const void *x, const void *w,
                              const float *bn_scale, const float *bn_bias, void *y,
                              void *workspace, size_t workspace_bytes, void *stream);

/* Training-mode BatchNorm: the batch's own statistics instead of running
 * ones. Per output channel k, over all M = N*P*Q conv outputs acc:
 *   mean_k = sum(acc)/M, var_k = sum((acc - mean_k)^2)/M   (biased),
 *   y = silu(gamma_k * (acc - mean_k) / sqrt(var_k + eps) + beta_k),
 * the batch-normalising transform (Ioffe and Szegedy, 2015). The statistics
 * are a reduction over every block's outputs, which "Kernel Fusion"
 * (cheatsheet page, passages on reductions and on synchronization
 * boundaries) says cannot be fused without a kernel boundary, so the call
 * runs in passes on `stream`. 1x1 layers (the one-workgroup-per-CU
 * kernel) and stems with C_out <= 32: a pass of the conv that reads x and
 * stores nothing forms the
 * per-channel statistics from the fp32 accumulators (count, mean and
 * squared deviations per workgroup, fp64); a small kernel combines them in
 * a fixed order (results are deterministic) and folds them into one scale
 * and one bias; the fused kernel then computes the conv again and writes y
 * (the layer is bound by HBM: reading x twice costs less than writing and
 * re-reading t1). Other layers: the plan's conv kernel writes the conv
 * output t1 into y, a reduction over t1 forms fp64 partial sums, the same
 * fixed-order combine and fold follow, and a streaming kernel applies
 * BatchNorm and SiLU to y in place (t1 written once and read once). gamma, beta: device fp32 [C_out]. running_mean/running_var:
 * device fp32 [C_out] updated in place as r = (1-momentum)*r +
 * momentum*batch_value, with the unbiased variance var_k*M/(M-1); both NULL
 * for no update. batch_mean/batch_var: device fp32 [C_out] outputs (the
 * biased variance), each may be NULL. y must not alias x. workspace (the
 * per-channel scale and bias and the statistics partials, a few MB at
 * most): at least the size from tg_conv_bn_silu_train_workspace, 16-byte
 * aligned for the vector kernels, not aliasing any other argument. Errors: TG_ERR_INVALID_ARGUMENT for a
 * NULL plan/x/w/gamma/beta/y, only one of running_mean/running_var given,
 * eps < 0, momentum outside [0, 1], or M < 2; TG_ERR_UNSUPPORTED for a plan
 * whose activation is not SiLU; TG_ERR_WORKSPACE;
 * TG_ERR_ALIGNMENT (forced kernels only, as for run); TG_ERR_HIP. */
tg_status tg_conv_bn_silu_train_run(const tg_conv_bn_silu_plan *plan, const void *x,
                                    const void *w, const float *gamma, const float *beta,
                                    float eps, float momentum, float *running_mean,
                                    float *running_var, float *batch_mean, float *batch_var,
                                    void *y, void *workspace, size_t workspace_bytes,
                                    void *stream);

/* Workspace bytes tg_conv_bn_silu_train_run needs for this plan (host only).
 * TG_ERR_INVALID_ARGUMENT for NULL arguments. */
tg_status tg_conv_bn_silu_train_workspace(const tg_conv_bn_silu_plan *plan, size_t *bytes);

/* For callers that cannot allocate device memory -- code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc:
 * tg_conv_bn_silu_train_run with its workspace (scale, bias and statistics
 * partials) in a static device array of TG_STATIC_SCRATCH_BYTES that the
 * library holds on each GPU it runs on, until the process ends, instead of a
 * caller's buffer. The call allocates nothing: at its first call on a device
 * (the current device, which must be the stream's) it looks up the array's
 * address there. Every byte of the array a call reads it has written earlier
 * in the same call, so nothing needs clearing; calls that overlap on one GPU
 * (two streams, two host threads) share the array and race -- serialise
 * them. Errors: TG_ERR_UNSUPPORTED when the plan's training workspace
 * (tg_conv_bn_silu_train_workspace) exceeds TG_STATIC_SCRATCH_BYTES, checked
 * before anything touches the GPU; TG_ERR_HIP when the array's address
 * cannot be taken or a launch fails; the other arguments and errors as for
 * tg_conv_bn_silu_train_run. */
#define TG_STATIC_SCRATCH_BYTES (4u << 20)
tg_status tg_conv_bn_silu_train_run_static(const tg_conv_bn_silu_plan *plan, const void *x,
                                           const void *w, const float *gamma, const float *beta,
                                           float eps, float momentum, float *running_mean,
                                           float *running_var, float *batch_mean,
                                           float *batch_var, void *y, void *stream);

/* Activation in the epilogue. The fused kernels apply, after the folded
 * BatchNorm v = acc*bn_scale[k] + bn_bias[k], one of: SiLU v*sigmoid(v)
 * (the default of every other create), ReLU max(v, 0), GELU in its exact
 * form v*Phi(v) = v/2*(1 + erf(v/sqrt 2)), or nothing (BatchNorm only, i.e.
 * a conv with a per-channel scale and bias). "Fusing an Epilogue", section
 * "What an epilogue is": activations, bias adds and scaling are the
 * elementwise work that belongs in the producer's epilogue. */
typedef enum { TG_ACT_SILU = 0, TG_ACT_RELU = 1, TG_ACT_GELU = 2, TG_ACT_NONE = 3 } tg_activation;

/* Same as tg_conv_bn_silu_create (MI355X dispatch table) with the epilogue's
 * activation chosen; run() then applies it. TG_ERR_UNSUPPORTED for an
 * unknown activation, or an activation other than SiLU together with
 * TG_UNFUSED or TG_SPLIT (whose streaming kernels apply SiLU); a plan with
 * an activation other than SiLU is rejected by tg_conv_bn_silu_train_run
 * (TG_ERR_UNSUPPORTED). */
tg_status tg_conv_bn_act_create(tg_conv_bn_silu_plan **out, int N, int H, int W, int C_in,
                                int C_out, int kh, int kw, int stride, int pad, tg_dtype dtype,
                                tg_kernel kernel, tg_activation act);

/* Same as tg_conv_bn_act_create, with y stored in y_dtype: the input dtype,
 * or TG_F8_E4M3 for fp16 inputs -- a cast to a narrower dtype done in the
 * epilogue ("Fusing an Epilogue", section "What an epilogue is"), which
 * halves the bytes of y. y is then N*P*Q*C_out bytes, 16-byte aligned for
 * the vector kernels as before. TG_ERR_UNSUPPORTED for another y_dtype,
 * fp8 with fp32 inputs, or fp8 with TG_UNFUSED / TG_SPLIT; an fp8 plan is
 * rejected by tg_conv_bn_silu_train_run. */
tg_status tg_conv_bn_act_create_out(tg_conv_bn_silu_plan **out, int N, int H, int W, int C_in,
                                    int C_out, int kh, int kw, int stride, int pad,
                                    tg_dtype dtype, tg_kernel kernel, tg_activation act,
                                    tg_dtype y_dtype);

/* Same as tg_conv_bn_silu_run, adding a residual in the epilogue:
 * y = act(acc*bn_scale + bn_bias) + residual, elementwise -- the residual add
 * that "Kernel Fusion" (cheatsheet page, the passage on elementwise chains)
 * counts among the operations that fuse freely. residual: device, y's shape
 * and dtype (NHWC [N][P][Q][C_out]); it is read once, and y must not alias
 * it. For fp16 the activated value is rounded to fp16 first and the sum is
 * formed in fp32 and rounded once more. Errors as for run, plus
 * TG_ERR_INVALID_ARGUMENT for a NULL residual and TG_ERR_UNSUPPORTED for an
 * unfused, split or fp8-output plan. */
tg_status tg_conv_bn_silu_run_residual(const tg_conv_bn_silu_plan *plan, const void *x,
                                       const void *w, const float *bn_scale,
                                       const float *bn_bias, const void *residual, void *y,
                                       void *stream);

/* Load-time filter pre-pack ("When the fusion you want is impossible, fuse
 * into the producer", section "The general form": work that would repeat at
 * every call is done once, when the weights are loaded). For a plan whose
 * kernel is the patch-staged implicit GEMM (fp16, stride 1, C_in % 64 == 0:
 * the 3x3 and 7x7 layers), the OHWI filter is rewritten once into the order
 * in which that kernel's filter loads land in its LDS ring, so every load
 * instruction reads one contiguous kilobyte; the packed form is specific to
 * the plan (its tile) and the output of tg_conv_bn_silu_run_packed is
 * bit-identical to tg_conv_bn_silu_run with the OHWI filter.
 *   tg_conv_bn_silu_packed_filter_bytes: *bytes = size of the packed filter
 *     (TG_ERR_UNSUPPORTED, *bytes = 0, for a plan whose kernel takes no packed
 *     filter, including unfused and split plans; TG_ERR_INVALID_ARGUMENT for
 *     NULL pointers). Host only.
 *   tg_conv_bn_silu_pack_filter: w (device OHWI [C_out][kh][kw][C_in] fp16)
 *     -> w_packed (device, w_packed_bytes >= the size above, 16-byte
 *     aligned, not overlapping w). TG_ERR_WORKSPACE for a short buffer,
 *     TG_ERR_ALIGNMENT, TG_ERR_HIP on launch failure. Asynchronous.
 *   tg_conv_bn_silu_run_packed: tg_conv_bn_silu_run with the packed filter
 *     (the plan's activation and output dtype apply; no workspace). x, y and
 *     w_packed must be 16-byte aligned (TG_ERR_ALIGNMENT: there is no scalar
 *     fallback for a packed filter); other errors as for run. */
tg_status tg_conv_bn_silu_packed_filter_bytes(const tg_conv_bn_silu_plan *plan, size_t *bytes);
tg_status tg_conv_bn_silu_pack_filter(const tg_conv_bn_silu_plan *plan, const void *w,
                                      void *w_packed, size_t w_packed_bytes, void *stream);
tg_status tg_conv_bn_silu_run_packed(const tg_conv_bn_silu_plan *plan, const void *x,
                                     const void *w_packed, const float *bn_scale,
                                     const float *bn_bias, void *y, void *stream);

/* Explicit kernel-variant overrides, for measurement sweeps and for tests
 * that exercise a variant the dispatch table does not pick for the shape
 * ("Fusing an Epilogue", section "Three kernels for one operation": the
 * thresholds are measured, so every candidate must be runnable on demand).
 * Same as tg_conv_bn_act_create_out, plus `tuning`: NULL or a string of
 * comma-separated key=value pairs (decimal values below 2^20), resolved into
 * the plan here; run() reads nothing else. Keys:
 *   cu=<waves per 64-channel slice, 0 = off>, cu_pd=<1..3>   1x1 C_in=64
 *       one-workgroup-per-CU kernel and its input prefetch depth;
 *   igemm_rw=0|1, rw_nf, rw_cs, rw_ncw, rw_wg_per_cu, nt=0|1   the
 *       register-weights 1x1 kernel, its split, grid and non-temporal stores;
 *   stream=<waves per CU>, xdma=<1..4>   the streaming 1x1 kernel (opt-in)
 *       and its full-line input staging depth;
 *   band=0|1   the band implicit GEMM (opt-in; stride 1, C_in % 64 == 0,
 *       C_out 64 or 128: all output channels of a band of pixels per
 *       workgroup; it takes no packed filter);
 *   igemm_patch=0|1, patch_cfg=<i>   the patch-staged implicit GEMM and a
 *       forced tile (ignored when it does not fit the shape; a forced
 *       patch or direct-to-LDS tile also turns the band kernel off);
 *   igemm_dma=0|1, dma_cfg=<i>, igemm_cfg=<i>   the direct-to-LDS and the
 *       classic implicit GEMM and their tiles;
 *   stem=<workgroups per CU, 0 = off>, stem_rows=<rows per band>   the RGB
 *       stem kernel;
 *   tiled_mfma=0|1, tm_pipe=0|1, tm_rows, tm_wg_per_cu   the band-staged MFMA
 *       tiled kernel, its persistent form, band height and grid.
 * Unknown keys, malformed text or out-of-range values: TG_ERR_INVALID_ARGUMENT.
 * Other errors as for tg_conv_bn_act_create_out. */
tg_status tg_conv_bn_silu_create_tuned(tg_conv_bn_silu_plan **out, int N, int H, int W,
                                       int C_in, int C_out, int kh, int kw, int stride,
                                       int pad, tg_dtype dtype, tg_kernel kernel,
                                       tg_activation act, tg_dtype y_dtype, const char *tuning);

/* Free a plan. NULL is a no-op. */
tg_status tg_conv_bn_silu_destroy(tg_conv_bn_silu_plan *plan);

/* Fold inference BatchNorm into one scale and one bias per output channel,
 * once per weight load ("When the fusion you want is impossible, fuse into
 * the producer", section "The general form": do once at load time what would
 * otherwise repeat per use): scale = gamma / sqrt(var + eps),
 * bias = beta - mean * scale, in fp32 on the device. All pointers are device
 * fp32 [C_out]; bn_scale/bn_bias must not alias the inputs. Errors:
 * TG_ERR_INVALID_ARGUMENT for NULL pointers, C_out < 1 or eps < 0;
 * TG_ERR_HIP on launch failure. Asynchronous on `stream`. */
tg_status tg_bn_fold(const float *gamma, const float *beta, const float *mean, const float *var,
                     float eps, int C_out, float *bn_scale, float *bn_bias, void *stream);

/* Layout conversions for callers holding PyTorch-layout tensors ("When the
 * fusion you want is impossible, fuse into the producer", layout paragraph:
 * store the filters channels-last once, at load time, and the per-call
 * conversion kernels disappear, with bit-identical output). Each is a pure
 * permutation on the device, bit-exact for fp16 and fp32, asynchronous on
 * `stream`; src and dst are device buffers that must not overlap.
 *   tg_filter_oihw_to_ohwi: w [C_out][C_in][kh][kw] -> [C_out][kh][kw][C_in],
 *     once per weight load;
 *   tg_nchw_to_nhwc: x [N][C][H][W] -> [N][H][W][C];
 *   tg_nhwc_to_nchw: y [N][H][W][C] -> [N][C][H][W] (H, W: y's extent).
 * Errors: TG_ERR_INVALID_ARGUMENT for NULL or identical pointers or a size
 * < 1; TG_ERR_UNSUPPORTED for an unknown dtype or 2^31 or more elements;
 * TG_ERR_HIP on launch failure. */
tg_status tg_filter_oihw_to_ohwi(const void *src, void *dst, int C_out, int C_in, int kh, int kw,
                                 tg_dtype dtype, void *stream);
tg_status tg_nchw_to_nhwc(const void *src, void *dst, int N, int C, int H, int W,
                          tg_dtype dtype, void *stream);
tg_status tg_nhwc_to_nchw(const void *src, void *dst, int N, int C, int H, int W,
                          tg_dtype dtype, void *stream);

/* Describe a plan: output extent (P, Q as in the formula at the top), the
 * kernel of the page's three that run() will launch ("Fusing an Epilogue",
 * section "Three kernels for one operation"; for aligned
 * pointers; may include TG_UNFUSED or TG_SPLIT) and the workspace it needs. Any out
 * pointer may be NULL. TG_ERR_INVALID_ARGUMENT for a NULL plan. */
tg_status tg_conv_bn_silu_query(const tg_conv_bn_silu_plan *plan, int *P, int *Q,
                                tg_kernel *chosen, size_t *workspace_bytes);

/* Human-readable summary of the plan's kernel, tile and grid, written into
 * buf (always NUL-terminated when len > 0). */
tg_status tg_conv_bn_silu_describe(const tg_conv_bn_silu_plan *plan, char *buf, size_t len);

/* The dispatch table alone, as a host-only function: which fused kernel the
 * given table picks for this shape and dtype (never TG_KERNEL_AUTO). Same
 * validation as create. */
tg_status tg_dispatch_choose(int N, int H, int W, int C_in, int C_out, int kh, int kw, int stride,
                             int pad, tg_dtype dtype, tg_dispatch table, tg_kernel *chosen);

/* Static strings; never NULL. */
const char *tg_status_string(tg_status s);
const char *tg_kernel_name(tg_kernel k);

#ifdef __cplusplus
}
#endif

#endif /* TG_CONV_BN_SILU_H */
