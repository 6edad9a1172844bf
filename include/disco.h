/*
 * disco.h — C ABI of the gfx950 DISCO sparse-contraction library (libdisco.so).
 *
 * The operations are the three named on the torch-harmonics "disco-kernel-dev"
 * page, section "Architecture snapshot":
 *   - the CSR sparse contraction from the input grid to the K-expanded output
 *     (B, C, K, Ho, Wo)                                        -> disco_fwd
 *   - the CSR transpose contraction from (B, C, K, Ho, Wo) back to the input
 *     grid, computed as an atomic-free gather (section "Backward direction —
 *     gather vs scatter": each input pixel accumulates from its neighbourhood)
 *                                                              -> disco_bwd
 *   - contraction followed by the dense channel/basis einsum    -> disco_fused_conv
 *
 * With s = Wi / Wo (an integer >= 1) and psi rows r = k*Ho + ho:
 *   out[b,c,k,ho,wo] = sum_{e in row r} val_e * x[b,c,hi_e,(wi_e + s*wo) mod Wi]
 *   gx = F^T gout      (exact transpose of the map above)
 *   y[b,o,ho,wo]     = sum_{c,k} W[o,c,k] * out[b,c,k,ho,wo]
 *
 * Conventions shared by every call
 *   - Tensors are dense, contiguous, row-major, last index fastest; `data` is a
 *     device pointer on the device the psi handle was created on.  The caller
 *     owns every tensor buffer.
 *   - Supported dtypes: DISCO_F32, DISCO_BF16 and DISCO_F16 (the precisions
 *     the page's test rules name, section "Test coverage requirements").  All
 *     tensors of one call share one dtype.  Accumulation is always fp32; a
 *     16-bit output is rounded once (round-to-nearest-even) from the fp32
 *     accumulator.  psi values are fp32 (kpacked section of the page: values
 *     stored as fp32), except on the bf16 matrix-core paths, which take psi
 *     rounded to bf16 as their multiplicand.
 *   - Outputs are fully overwritten (no accumulate flag); rows with no psi
 *     entries are written as exact zeros.
 *   - `stream` is a hipStream_t (0 = the null stream).  Work is enqueued
 *     asynchronously; the calls never synchronise the host with the device.
 *   - Every argument is validated on the host before anything is enqueued; on
 *     any error nothing is written and a status is returned.  The text of the
 *     last error of the calling thread is available from disco_last_error().
 *   - Only gfx950 devices are accepted (the page's kernels check the device
 *     architecture on the host and refuse others; section "Adding a new kernel
 *     variant", step 1).
 */
#ifndef DISCO_H
#define DISCO_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum disco_status {
    DISCO_OK = 0,
    DISCO_ERR_INVALID_ARGUMENT = 1,   /* null handle / tensor / data pointer, wrong device */
    DISCO_ERR_SHAPE = 2,              /* Wi % Wo != 0, or shapes disagree with psi / each other */
    DISCO_ERR_DTYPE = 3,              /* dtype not F32/BF16/F16, unsupported by the op, or dtypes of one call differ */
    DISCO_ERR_PSI = 4,                /* malformed CSR (row_ptr, column range, nnz >= 2^31) */
    DISCO_ERR_UNSUPPORTED_DEVICE = 5, /* device is not gfx950 */
    DISCO_ERR_OOM = 6,                /* device or host allocation failed */
    DISCO_ERR_HIP = 7                 /* a HIP runtime call or kernel launch failed */
} disco_status;

typedef enum disco_dtype {
    DISCO_F32 = 0,
    DISCO_BF16 = 1,
    DISCO_F16 = 2
} disco_dtype;

/* Host-side CSR filter ("psi").  Rows r = k*Ho + ho, K*Ho rows in all.
 * Column of an entry = input pixel (col_hi[e], col_wi[e]): the input latitude
 * and the longitude offset from output longitude 0.  Entries of one row may be
 * in any order; a (hi, wi) pair may appear at most once per row.
 * All arrays are host memory, read during disco_psi_create only. */
typedef struct disco_csr_desc {
    int32_t K, Ho, Wo, Hi, Wi;
    int64_t nnz;              /* must equal row_ptr[K*Ho] and be < 2^31 */
    const int64_t *row_ptr;   /* [K*Ho + 1], row_ptr[0] == 0, non-decreasing */
    const int32_t *col_hi;    /* [nnz], in [0, Hi) */
    const int32_t *col_wi;    /* [nnz], in [0, Wi) */
    const float *val;         /* [nnz] */
} disco_csr_desc;

/* Device tensor view.  shape[0..ndim-1] are used; the rest are ignored. */
typedef struct disco_tensor {
    void *data;               /* device pointer */
    int32_t dtype;            /* disco_dtype */
    int32_t ndim;
    int64_t shape[5];
} disco_tensor;

typedef struct disco_psi_s *disco_psi;

/* Validate the CSR, derive the device plans (longitude-run segments of the
 * forward rows grouped by shared support, and the row-inverted psi used by the
 * backward gather), and upload them to `device` (a HIP device ordinal).
 * Host arrays are copied; the caller may free them on return.  May block the
 * host until the uploads finish.  On success *out_handle owns all device
 * memory of the plan; release it with disco_psi_destroy.  A handle is
 * read-only after creation and may be used from several streams at once. */
disco_status disco_psi_create(const disco_csr_desc *csr, int device, disco_psi *out_handle);

/* Free a handle (NULL is accepted).  The caller must ensure no enqueued call
 * still uses it. */
disco_status disco_psi_destroy(disco_psi h);

/* Forward contraction.  x: (B, C, Hi, Wi) -> out: (B, C, K, Ho, Wo). */
disco_status disco_fwd(disco_psi h, const disco_tensor *x, disco_tensor *out, void *stream);

/* Transpose contraction.  gout: (B, C, K, Ho, Wo) -> gx: (B, C, Hi, Wi).
 * Atomic-free: every gx element is produced by one thread in a fixed order,
 * so results are bitwise reproducible run to run. */
disco_status disco_bwd(disco_psi h, const disco_tensor *gout, disco_tensor *gx, void *stream);

/* Fused convolution.  x: (B, C, Hi, Wi), W: (Co, C, K) -> y: (B, Co, Ho, Wo).
 * The contraction is computed on chip in channel chunks and never written to
 * device memory.  BF16 and F16: the einsum runs on bf16 or fp16 MFMA tiles with
 * fp32 accumulation (contraction chunks are rounded to the data type before the
 * MFMA).  F32: fp32 throughout (fp32 psi, an fp32 contraction chunk, the einsum
 * on the fp32 matrix cores) — the fp32 variant the 16-bit ones are compared
 * with (same page, "Test coverage requirements").
 * Memory: with BF16/F16 data and K < 16 the call takes a temporary of Co * C * 32 bytes from a
 * memory pool the library keeps per device (stream-ordered: taken and returned on `stream`; the pool
 * keeps freed memory for reuse until the process ends) to hold W in rows of 16 elements; if none can be
 * had the kernel stages W element by element instead, with the same result.  With F32 data, and with
 * 16-bit data on shapes outside the matrix-core kernel's plan (K > 16, Wi > 2 Wo, Wo not a multiple of 8),
 * the call takes a temporary of the same pool holding W in the vector-ALU fused kernel's einsum operand
 * order (Co and C rounded up to its 16-channel tiles and channel chunks: about Co * C * K elements); if
 * none can be had the call returns DISCO_ERR_OOM before anything is written. */
disco_status disco_fused_conv(disco_psi h, const disco_tensor *x, const disco_tensor *W,
                              disco_tensor *y, void *stream);

/* Fused convolution that also keeps its contraction, for a training step whose backward then need not
 * recompute it: y as disco_fused_conv, and out[b,c,k,ho,wo] = the contraction F x (B, C, K, Ho, Wo) in
 * the data type (each fp32 accumulator rounded once, RNE).  On the matrix-core fused kernel (BF16 and
 * F16 data on its plan) out holds the very values the einsum multiplied; otherwise (F32 data, shapes
 * outside that plan) out comes from disco_fwd, whose summation order may differ from the fused
 * kernel's by rounding.  Same page, "Python dispatch layer": the fused autograd function keeps what
 * its backward needs.  out is caller-owned and overwritten; it must not overlap x, W or y
 * (DISCO_ERR_INVALID_ARGUMENT). */
disco_status disco_fused_conv_save(disco_psi h, const disco_tensor *x, const disco_tensor *W, disco_tensor *y,
                                   disco_tensor *out, void *stream);

/* The einsum alone: the second half of the fused convolution, for a contraction that is already
 * in device memory (for instance the forward's output kept for the weight gradient).  Same page,
 * "Architecture snapshot" ("contraction + einsum"):
 *   y[b,o,ho,wo] = sum_{c,k} W[o,c,k] * t[b,c,k,ho,wo]
 * t: (B, C, K, Ho, Wo), W: (Co, C, K) -> y: (B, Co, Ho, Wo), on the current device (no psi).
 * BF16 and F16 only, K <= 16 (DISCO_ERR_SHAPE otherwise).  Runs the fused kernel's matrix-core
 * einsum tile with t streamed from device memory: fp32 accumulation in a fixed order, y rounded
 * once (RNE), bitwise reproducible run to run.  All tensors are caller-owned; y is overwritten.
 * K < 16 takes the same stream-ordered W temporary as disco_fused_conv (same fallback). */
disco_status disco_einsum(const disco_tensor *W, const disco_tensor *t, disco_tensor *y, void *stream);

/* Backward of the fused convolution: the gradients of <gy, y> for y = disco_fused_conv(x, W),
 *   gx[b,c]   = F^T g[b,c],  g[b,c,k,ho,wo] = sum_o W[o,c,k] * gy[b,o,ho,wo]
 *   dW[o,c,k] = sum_{b,ho,wo} gy[b,o,ho,wo] * out[b,c,k,ho,wo],  out = F x
 * (torch-harmonics "disco-kernel-dev" page, "Python dispatch layer": the fused autograd function
 * pairs the fused forward with the CSR transpose backward; "Test coverage requirements": fused
 * and unfused agree in output and gradient).
 * x: (B, C, Hi, Wi), W: (Co, C, K), gy: (B, Co, Ho, Wo) -> gx: (B, C, Hi, Wi), dW: (Co, C, K).
 * BF16 and F16; Co and Ho*Wo must be multiples of 8, K <= 256, and one batch of gy, of a channel
 * chunk of g, and W must each stay below 2 GiB (the matrix-core loads address 32-bit offsets).
 * gx: when Wi = Wo and K <= 16, gx[b,c] = sum_{o,k} W[o,c,k] (F_k^T gy[b,o]) is the fused convolution
 * of gy over the per-basis transpose of psi (built by disco_psi_create) with W' = W permuted to
 * (C, Co, K), its contraction rounded to the data type before the einsum as in disco_fused_conv;
 * otherwise channel chunks of g (the data type, on the matrix cores) and the transpose contraction.
 * dW: the forward contraction (the data type) per channel chunk and a split product whose fp32
 * partials are summed in a fixed order.  Results are bitwise reproducible run to run.  gx and dW must not overlap any
 * input (DISCO_ERR_INVALID_ARGUMENT).  `workspace` is caller-owned device memory (256-byte aligned) of at
 * least the size disco_fused_conv_bwd_workspace reports for (B, C, Co); its contents on entry
 * are ignored and on return are unspecified.  Calls sharing one workspace must not overlap.
 * Where gx takes the fused launch, the recomputed contraction and the dW products run on the
 * library's second stream beside it, with the same ordering guarantees as disco_fused_conv_bwd_saved
 * (the call behaves as if everything ran on `stream`). */
disco_status disco_fused_conv_bwd_workspace(disco_psi h, int64_t B, int64_t C, int64_t Co, size_t *bytes);
disco_status disco_fused_conv_bwd(disco_psi h, const disco_tensor *x, const disco_tensor *W, const disco_tensor *gy,
                                  disco_tensor *gx, disco_tensor *dW, void *workspace, size_t workspace_bytes,
                                  void *stream);

/* The same backward with the weight gradient's operand taken from `out`, the contraction that
 * disco_fused_conv_save wrote for the same x, instead of recomputing it from x (x is not needed).
 * out: (B, C, K, Ho, Wo); the other arguments, the workspace and the results as disco_fused_conv_bwd,
 * whose results it reproduces bitwise when out comes from disco_fused_conv_save.
 * The weight-gradient products run on a second stream that the library keeps per device (default
 * priority, created on first use, never destroyed): it waits for everything enqueued on `stream`
 * before the call, and `stream` waits for it before the call returns (also on an error return), so
 * the call behaves as if everything ran on `stream`.  Concurrent calls on one device share that
 * stream, so their weight-gradient work serialises; under graph capture of `stream` the fork and
 * join are captured as event dependencies. */
disco_status disco_fused_conv_bwd_saved(disco_psi h, const disco_tensor *out, const disco_tensor *W,
                                        const disco_tensor *gy, disco_tensor *gx, disco_tensor *dW, void *workspace,
                                        size_t workspace_bytes, void *stream);

/* The backward of the fused convolution (the same operation, results and restrictions as
 * disco_fused_conv_bwd) for callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation.  It takes no workspace and calls
 * no allocating routine: its workspace is the library's own scratch array of 64 MiB per device
 * (held from the library's load until the process ends).  The channel chunks shrink until the
 * workspace fits; shapes whose workspace cannot fit 64 MiB are refused with DISCO_ERR_SHAPE before
 * anything is enqueued (the fixed buffers alone must fit: 32 C Co bytes of permuted W where gx takes the
 * fused launch over the transposed psi, else 2 (C K Co + B Ho Wo Co) bytes of W^T and gy^T).  Every call on
 * one device uses the same array: calls that overlap on one device (other streams, other threads)
 * race and must not be issued.  The array's contents on entry are ignored. */
disco_status disco_fused_conv_bwd_noalloc(disco_psi h, const disco_tensor *x, const disco_tensor *W,
                                          const disco_tensor *gy, disco_tensor *gx, disco_tensor *dW, void *stream);

/* Message of the last non-OK status returned on the calling thread ("" if none). */
const char *disco_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* DISCO_H */
