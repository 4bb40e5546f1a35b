/*
 * kq.h — C ABI of the KronQ per-linear-layer quantization solver for MI355X (gfx950).
 *
 * The method (KronQ: LLM Quantization via Kronecker-Factored Hessian; summary
 * on hyper.ai, section "Method"; explainer on gist.science, "Metodologia")
 * models the Hessian of a linear layer y = W x as H ~ H_X (x) H_G and
 * quantizes W column by column with the GPTAQ update, after bidirectional
 * incoherence processing (BiIP). This library implements that per-layer path
 * as five device stages plus a host-side allocator:
 *
 *   kq_accumulate_cov   H_X = X~^T X~ / N, D = dX^T X~ / N, H_G = G^T G / N
 *   kq_biip             diagonal scalings S_X, S_G and random Hadamard U, V
 *   kq_sensitivity      s = tr(H_G') * tr(H_X')
 *   kq_cholesky_inv     upper U with U^T U = (H_X' + delta I)^-1
 *   kq_gptaq_quantize   blocked column sweep onto a 2/3/4-bit grid
 *   kq_allocate_bits    widths by descending s under an average-bit budget
 *
 * Conventions (all calls):
 *  - Matrices are dense and row-major; the row stride equals the column
 *    count. Token-major activations X (N x d_in) hold one token per row, so
 *    X^T X is the page's E[x x^T] up to 1/N.
 *  - Pointers are DEVICE pointers unless marked "host". The caller owns every
 *    buffer; the library allocates no device memory and creates no stream or
 *    event. Scratch memory is passed in as (ws, ws_bytes); kq_workspace_size
 *    gives the size each call needs. The only state kept between calls is the
 *    measurement hook of kq_set_kernel_events (two caller-owned event handles
 *    per thread, unset by default), the testing knob of kq_set_gemm_tile
 *    (per thread, automatic by default), a 64-byte pinned host buffer
 *    per calling thread (hipHostMalloc on first use, kept until the process
 *    ends) through which the calls below read their host results, and the
 *    host copy of the last launch schedule kq_accumulate_cov built on the
 *    thread (rebuilt when the shapes or the requested outputs change);
 *    nothing else carries over from one call to the next.
 *  - Device work is enqueued on `stream` and is asynchronous, except calls
 *    that return host values: kq_sensitivity and kq_layer_objective wait
 *    until the stream is idle before returning; kq_cholesky_inv waits for
 *    its factorization (to report a non-positive pivot) and returns with the
 *    inverse still enqueued. These waits poll the stream (the calling
 *    thread spins) rather than block.
 *  - Arguments are validated on the host before anything is launched;
 *    errors return a kq_status and kq_last_error() gives a message (per
 *    thread). Calls on disjoint buffers may run concurrently.
 *  - Sizes are int64; every dimension must be >= 1 unless stated.
 */
#ifndef KQ_H
#define KQ_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  KQ_OK = 0,
  KQ_ERR_ARG = 1,          /* null pointer, bad enum, bad scalar */
  KQ_ERR_SHAPE = 2,        /* bad dimension or block size */
  KQ_ERR_NOT_PD = 3,       /* factorisation met a non-positive pivot (see info) */
  KQ_ERR_NONFINITE = 4,    /* NaN or Inf met where a finite value is required */
  KQ_ERR_WORKSPACE = 5,    /* ws_bytes smaller than kq_workspace_size */
  KQ_ERR_HIP = 6,          /* a HIP runtime call failed */
  KQ_ERR_UNSUPPORTED = 7   /* valid request this library does not implement */
} kq_status;

typedef enum { KQ_BF16 = 0, KQ_F32 = 1 } kq_dtype;

typedef enum {
  KQ_OP_ACCUMULATE_COV = 0,
  KQ_OP_BIIP = 1,
  KQ_OP_SENSITIVITY = 2,
  KQ_OP_CHOLESKY_INV = 3,
  KQ_OP_FORM_P = 4,
  KQ_OP_GPTAQ_QUANTIZE = 5,
  KQ_OP_LAYER_OBJECTIVE = 6,
  KQ_OP_APPLY_QUANTIZED = 7, /* n_tok argument of kq_workspace_size = batch */
  KQ_OP_YAQA_QUANTIZE = 8,
  KQ_OP_APPLY_QUANTIZED_A4 = 9 /* n_tok argument of kq_workspace_size = batch */
} kq_op;

/* Grid and sweep configuration (KronQ summary, Method and experiments:
 * uniform 2/3/4-bit weight-only grids, per output channel or in groups of
 * 128 input columns; GPTAQ lazy block of 128 columns). */
typedef struct {
  int32_t bits;   /* 2, 3 or 4 (codes in [0, 2^bits - 1]) */
  int32_t group;  /* 0 = one grid per output channel; else 128 (columns per group) */
  int32_t block;  /* lazy-update block of the sweep; must be 128 */
  int32_t flags;  /* reserved, must be 0 */
} kq_quant_cfg;

/* Message for the last failing call on this thread ("" if none). */
const char* kq_last_error(void);

/* Library version string. */
const char* kq_version(void);

/* Measurement hook; not part of the method and not needed to use it.
 * After kq_set_kernel_events(op, start, stop), every later call of `op` made
 * from this thread records `start` on its stream right before the op's main
 * kernel is enqueued and `stop` right after, so the caller can time that one
 * kernel with hipEventElapsedTime on the stream it actually ran on. This is
 * the only state the library keeps between calls (per thread).
 *   op     KQ_OP_ACCUMULATE_COV: the main kernel is the covariance
 *          kernel (bf16 inputs: the tile kernel that computes H_X, D and H_G
 *          together; the drift pre-pass and the split reduction lie outside
 *          the bracket). For fp32 inputs the bracket holds the three
 *          products and the drift pass.
 *          KQ_OP_GPTAQ_QUANTIZE: the first 512-column superblock's lazy
 *          trailing update, the sweep's largest GEMM (d_out x (d_in - 512)
 *          x 512; none if d_in <= 512).
 *          KQ_OP_APPLY_QUANTIZED: the product with the packed codes (one
 *          launch per 4 vectors of the batch; the two transforms, and the
 *          sum of the matrix-core path's partial planes in the output
 *          transform, lie outside the bracket).
 *          KQ_OP_APPLY_QUANTIZED_A4: the integer product (one launch for
 *          the whole batch; the transforms and the input quantization lie
 *          outside).
 *   start, stop  events created by the caller (who owns and destroys them);
 *          both NULL switches the hook off.
 * Errors: KQ_ERR_UNSUPPORTED for other ops, KQ_ERR_ARG if exactly one event
 * is NULL. */
kq_status kq_set_kernel_events(kq_op op, hipEvent_t start, hipEvent_t stop);

/* Testing knob; not part of the method and not needed to use it.
 * The library's fp32 matrix products (factorization updates, triangular
 * inverse, P, the fold and the sweep's lazy updates) run either on the fp32
 * matrix cores with a 64-, 128- or 256-wide output tile, or, for large
 * products with op(A) = A, on the bf16 matrix cores as six products of
 * three-term bf16 splits of the fp32 operands (128-wide tile; fp32-level
 * accuracy, fp32 accumulation), chosen per product from its shape. After
 * kq_set_gemm_tile(tile), later calls made from this thread use:
 *   tile   0: the choice by shape (the default);
 *          64: the 64-wide fp32 tile everywhere;
 *          128 or 256: that fp32 tile wherever a product allows it (a
 *          product computed in place, and the output-start-masked products
 *          of kq_yaqa_quantize, always take the 64-wide tile);
 *          3: the three-term bf16 kernel for every product it can take
 *          (op(A) = A, not in place, no output start), whatever its size;
 *          the others by shape.
 * Every choice computes each output from the same operands with fp32
 * accumulation; results differ only in rounding and summation order.
 * Errors: KQ_ERR_ARG for any other value. */
kq_status kq_set_gemm_tile(int tile);

/* Bytes of scratch memory `op` needs for the given sizes (host output).
 * n_tok and dtype matter for KQ_OP_ACCUMULATE_COV only; cfg for
 * KQ_OP_GPTAQ_QUANTIZE only (may be NULL elsewhere). For square-matrix ops
 * (CHOLESKY_INV, FORM_P) pass the matrix order as d_in. */
kq_status kq_workspace_size(kq_op op, int64_t d_out, int64_t d_in, int64_t n_tok,
                            kq_dtype dtype, const kq_quant_cfg* cfg, size_t* bytes);

/* Stage 1 — covariances (KronQ summary, Method: Fisher equation and the
 * K-FAC step H ~ H_X (x) H_G; GPTAQ objective: the asymmetric term dX X^T).
 *   HX <- alpha * Xq^T Xq + beta * HX        (d_in x d_in, full symmetric)
 *   D  <- alpha * dX^T Xq + beta * D         (d_in x d_in, not symmetric)
 *   HG <- alpha * G^T G   + beta * HG        (d_out x d_out, full symmetric)
 * X, Xq: n_tok x d_in token-major inputs of the full-precision and the
 * quantized model; G: n_tok x d_out output gradients. dt = KQ_BF16 (uint16
 * bf16 patterns) or KQ_F32. dX = X - Xq in fp32, rounded to bf16 (nearest
 * even) when dt = KQ_BF16. Products are exact, sums are fp32.
 * Stream chunks of tokens by calling with beta = 0 on the first chunk and
 * beta = 1 after, alpha = 1 / (total tokens). HX, D, HG may each be NULL to
 * skip that output (D needs X and Xq; HX needs Xq; HG needs G). */
kq_status kq_accumulate_cov(const void* X, const void* Xq, const void* G, kq_dtype dt,
                            int64_t n_tok, int64_t d_in, int64_t d_out,
                            float alpha, float beta,
                            float* HX, float* D, float* HG,
                            void* ws, size_t ws_bytes, hipStream_t stream);

/* Stage 2 — bidirectional incoherence processing (KronQ summary, Method:
 * BiIP scaling equation and rotation equation), in place:
 *   s_j = (HX_jj / ||W_:,j||^2)^(1/4),  t_i = (HG_ii / ||W_i,:||^2)^(1/4)
 *   (a zero diagonal or zero norm gives 1; both from the unscaled W)
 *   W  <- U diag(t) W diag(s) V^T
 *   HX <- V diag(1/s) HX diag(1/s) V^T,   D <- V diag(1/s) D diag(1/s) V^T
 *   HG <- U diag(1/t) HG diag(1/t) U^T
 * with V = blockdiag(H_b / sqrt(b)) diag(sign_in) over d_in (Sylvester H_b,
 * b = blk_in) and U likewise over d_out with sign_out, blk_out. blk = 0
 * selects the largest power of two dividing the dimension; a nonzero blk
 * must be a power of two in [1, 8192] dividing it (blocks above 8192 return
 * KQ_ERR_UNSUPPORTED). W: d_out x d_in; HX, D: d_in x d_in; HG:
 * d_out x d_out; D may be NULL. sign_in, sign_out: int8 +-1 (device).
 * s_x (d_in) and s_g (d_out) receive s and t (device, may be NULL). */
kq_status kq_biip(float* W, float* HX, float* D, float* HG, int64_t d_out, int64_t d_in,
                  const int8_t* sign_in, const int8_t* sign_out,
                  int64_t blk_in, int64_t blk_out, float* s_x, float* s_g,
                  void* ws, size_t ws_bytes, hipStream_t stream);

/* Stage 5 — sensitivity (KronQ summary, Method: s = tr(H_G) * tr(H_X), taken
 * after BiIP). Reads the diagonals of HX (d_in x d_in) and HG (d_out x d_out)
 * and sums them in fp64. trHX, trHG, s: host outputs (any may be NULL).
 * Synchronizes the stream. */
kq_status kq_sensitivity(const float* HX, const float* HG, int64_t d_in, int64_t d_out,
                         double* trHX, double* trHG, double* s,
                         void* ws, size_t ws_bytes, hipStream_t stream);

/* Stage 3 — inverse-Hessian factor for the OBS update (KronQ summary,
 * Method: the column update uses rows of H_X^-1). With
 * delta = damp * mean(diag H), computes the upper-triangular U (n x n, lower
 * part set to 0) with U^T U = (H + delta I)^-1, so that U_pp * U_{p,p:} is
 * row p of the inverse of the trailing block (H + delta I)_{p:,p:}.
 * H: n x n symmetric; only its upper triangle (j >= i) is read. fp32 throughout. info (host, may be NULL)
 * receives 0, or k+1 where k is the original column index of the first
 * non-positive pivot (the factorisation proceeds from the last column to the
 * first); that case returns KQ_ERR_NOT_PD and leaves U undefined.
 * Waits for the factorization before returning (the pivot status is read on
 * the host); the triangular inverse that completes U is enqueued on the
 * stream after that check, so U is ready when the stream's work before the
 * next synchronization point has run, as for the asynchronous calls. */
kq_status kq_cholesky_inv(const float* H, int64_t n, float damp, float* U, int32_t* info,
                          void* ws, size_t ws_bytes, hipStream_t stream);

/* The GPTAQ asymmetric correction (KronQ summary, Method: the matrix P of the
 * OBS update, not written out on the pages). P = triu_1(D U^T) U (n x n,
 * strictly upper, zeros elsewhere): row p equals D_{p,F} ((H+delta I)_{FF})^-1
 * with F = {p+1, ..., n-1}. kq_gptaq_quantize forms it internally; this entry
 * exposes it for inspection. */
kq_status kq_form_p(const float* D, const float* U, int64_t n, float* P,
                    void* ws, size_t ws_bytes, hipStream_t stream);

/* Stage 4 — GPTAQ column sweep (KronQ summary, Method: column-wise OBS
 * update dW_{:,p+1:} = -delta_p [H_X^-1]_{p,p+1:} + W_{:,p} P_{p,p+1:};
 * H_G cancels from it, gist.science Metodologia, Proposition 1).
 * W: d_out x d_in; on entry the processed weights W0', on exit the
 * dequantized W^'. U: the factor from kq_cholesky_inv. D: the processed
 * drift term (NULL = plain GPTQ, P = 0). For each column p in order:
 *   q = clamp(rint(w_p / scale) + zero, 0, 2^bits - 1),  w^_p = scale (q - zero)
 *   w_{p+1:} -= ((w_p - w^_p) / U_pp) U_{p,p+1:} ;  w_{p+1:} += W0_p P_{p,p+1:}
 * Grid (fp32): lo = min(v, 0), hi = max(v, 0) ([-1,1] if both 0),
 * scale = (hi - lo) / (2^bits - 1), zero = rint(-lo / scale); per output
 * channel from W0', or per group of 128 columns from the working values when
 * the sweep reaches the group. Outputs: codes (d_out x d_in, uint8),
 * scale, zero (d_out x n_groups fp32, n_groups = 1 per channel, else
 * ceil(d_in / 128)). d_in must be a positive multiple of 128. */
kq_status kq_gptaq_quantize(float* W, const float* U, const float* D,
                            int64_t d_out, int64_t d_in, const kq_quant_cfg* cfg,
                            uint8_t* codes, float* scale, float* zero,
                            void* ws, size_t ws_bytes, hipStream_t stream);

/* Rounding with output-side feedback: the generalized LDLQ of YAQA (notes on
 * YAQA, arXiv 2505.22988, section "key designs", item 4, Eq. 5/6: for a
 * Kronecker sketch H_O (x) H_I the codes are the fixed point of
 * W = Q(W* + L_O'^T Dl L_I' + L_O'^T Dl + Dl L_I'), Dl = W* - W, L' = L - I
 * with L the unit-triangular LDL factor; item 1: it settles within
 * d_out + d_in - 1 steps), on KronQ's sketch H_G' (x) H_X'. In terms of the
 * inverse factors the rounded input of entry (i, j) is
 *   z_ij = W*_ij - sum_{k<=i, l<=j, (k,l)!=(i,j)} U_out[k][i] e_kl U_in[l][j],
 *   e_kl = (z_kl - w^_kl) / (U_out[k][k] U_in[l][l]),
 *   q = clamp(rint(z / scale) + zero, 0, 2^bits - 1),  w^ = scale (q - zero);
 * with U_out = I this is the column sweep of kq_gptaq_quantize.
 *   W        d_out x d_in; on entry the processed weights W0', on exit W^'.
 *   U_in     kq_cholesky_inv of H_X' (d_in x d_in, upper).
 *   U_out    kq_cholesky_inv of H_G' (d_out x d_out, upper).
 *   D        the processed drift term or NULL; with D the target is the GPTAQ
 *            fold W* = W0' + W0' P, P = triu_1(D U_in^T) U_in (as in
 *            kq_gptaq_quantize), else W* = W0'.
 *   cfg      bits 2..8; group must be 0 (one grid per output channel, from
 *            W0' as in kq_gptaq_quantize: group grids depend on the moment a
 *            row reaches a group, which this order does not fix, so they
 *            return KQ_ERR_UNSUPPORTED); block must be 128 (unused).
 *   codes    d_out x d_in uint8;  scale, zero: d_out fp32.
 * Any d_out, d_in >= 1. Workspace from
 * kq_workspace_size(KQ_OP_YAQA_QUANTIZE, d_out, d_in, ...) (sized for a
 * non-NULL D). Asynchronous: every launch is enqueued on `stream`, and the
 * call creates no stream or event of its own; fp32 arithmetic. */
kq_status kq_yaqa_quantize(float* W, const float* U_in, const float* U_out, const float* D,
                           int64_t d_out, int64_t d_in, const kq_quant_cfg* cfg,
                           uint8_t* codes, float* scale, float* zero,
                           void* ws, size_t ws_bytes, hipStream_t stream);

/* Mixed-precision allocation (KronQ summary, Method: sublayers with larger
 * s get wider codes). Host only, deterministic. Visits the L sublayers in
 * descending s (ties by index) and gives each the widest of `widths` that
 * still leaves every unvisited sublayer the narrowest width within
 * sum(bits_l * n_params_l) <= avg_budget * sum(n_params_l).
 * s, n_params, widths: host arrays; bits_out: host array of L. */
kq_status kq_allocate_bits(const double* s, const int64_t* n_params, int32_t L,
                           const int32_t* widths, int32_t n_widths, double avg_budget,
                           int32_t* bits_out);

/* Layer objective (KronQ summary, Method: Kronecker objective and its GPTAQ
 * extension), a metric rather than a stage:
 *   obj = tr[HG (dW HX dW^T + 2 W0 D dW^T)],  dW = W0 - What
 * (D may be NULL). fp32 products, fp64 final sum. obj: host output.
 * Synchronizes the stream. */
kq_status kq_layer_objective(const float* W0, const float* What, const float* HX,
                             const float* D, const float* HG, int64_t d_out, int64_t d_in,
                             double* obj, void* ws, size_t ws_bytes, hipStream_t stream);

/* ---------------------------------------------------------------------
 * Inference with the quantized layer (KronQ explainer, gist.science,
 * "Limitazioni": at inference only the orthogonal transforms remain, as in
 * QuIP#). The sweep quantized W' = U S_G W S_X V^T; the layer in its
 * original basis is W^ = S_G^-1 U^T W^' V S_X^-1 with W^' = scale (q - zero).
 *
 * Packing: each row of codes is a little-endian bit stream, code j in bits
 * [bits j, bits j + bits) of consecutive 32-bit words; rows are padded to a
 * multiple of 4 words (16 bytes). */

/* Words per packed row for d_in codes of `bits` bits (host output). */
kq_status kq_packed_row_words(int64_t d_in, int32_t bits, int64_t* words);

/* codes (d_out x d_in uint8, each < 2^bits) -> packed (d_out x row words,
 * uint32). bits in {2, 3, 4, 8}. Asynchronous. */
kq_status kq_pack_codes(const uint8_t* codes, int64_t d_out, int64_t d_in, int32_t bits,
                        uint32_t* packed, hipStream_t stream);

/* y = S_G^-1 U^T (W^' (V (S_X^-1 x))) for a batch of vectors, the transforms
 * applied to the vectors (the layer is never formed).
 *   packed, bits        codes from kq_pack_codes
 *   scale, zero         the grids of kq_gptaq_quantize (d_out x n_groups)
 *   group               0 (one grid per row) or 128
 *   s_x, s_g            the BiIP scalings (kq_biip outputs, d_in / d_out)
 *   sign_in, sign_out   the Hadamard signs given to kq_biip, with its blocks
 *                       blk_in, blk_out (0 = largest power of two dividing)
 *   x                   batch x d_in fp32, row-major (not modified)
 *   y                   batch x d_out fp32 output
 * d_in must be a multiple of 32 (of 128 with groups), and 1 <= batch <=
 * 65536 (the launch grids' limit). Workspace from
 * kq_workspace_size(KQ_OP_APPLY_QUANTIZED, d_out, d_in, batch, ...).
 * Asynchronous; fp32 arithmetic. */
kq_status kq_apply_quantized(const uint32_t* packed, int32_t bits, const float* scale,
                             const float* zero, int32_t group, const float* s_x, const float* s_g,
                             const int8_t* sign_in, const int8_t* sign_out, int64_t blk_in,
                             int64_t blk_out, const float* x, int64_t batch, int64_t d_out,
                             int64_t d_in, float* y, void* ws, size_t ws_bytes, hipStream_t stream);

/* Bytes of device scratch memory behind kq_apply_quantized_noalloc (one
 * copy per GPU, held until the process ends). */
#define KQ_NOALLOC_SCRATCH_BYTES (64u << 20)

/* kq_apply_quantized for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc. Same arguments, results and errors as kq_apply_quantized,
 * without (ws, ws_bytes): the scratch memory is a fixed array of
 * KQ_NOALLOC_SCRATCH_BYTES inside the library, one per GPU, whose device
 * address is looked up once per device on the first call made with that
 * device current (the device of `stream` must be the current device). The
 * call allocates nothing. Sizes whose workspace
 * (kq_workspace_size(KQ_OP_APPLY_QUANTIZED, d_out, d_in, batch)) exceeds
 * KQ_NOALLOC_SCRATCH_BYTES return KQ_ERR_WORKSPACE before any launch. Every
 * call on a GPU shares that GPU's array: calls that may overlap on one GPU
 * (two streams, two threads) race and must be ordered by the caller. No
 * state of one call is read by the next (the array's contents are
 * rewritten before use). Asynchronous. */
kq_status kq_apply_quantized_noalloc(const uint32_t* packed, int32_t bits, const float* scale,
                                     const float* zero, int32_t group, const float* s_x,
                                     const float* s_g, const int8_t* sign_in, const int8_t* sign_out,
                                     int64_t blk_in, int64_t blk_out, const float* x, int64_t batch,
                                     int64_t d_out, int64_t d_in, float* y, hipStream_t stream);

/* Weights and activations both quantized (the W2A4 setting; KronQ explainer,
 * gist.science, "Quantizzazione di Pesi e Attivazioni": activations follow
 * the QuaRot recipe). The rotated input x2 = V S_X^-1 x of each vector is
 * rounded to 4 bits on its own symmetric grid,
 *   s_b = clip * max_k |x2_bk| / 7,   a_bk = clamp(rint(x2_bk / s_b), -8, 7)
 * (fp32, ties to even; an all-zero vector has s_b = 0 and a_b = 0), and
 *   y = S_G^-1 U^T (W^' (s a)),
 * with the product W^' (s a) exact in integers (2-bit codes times 4-bit
 * inputs) before one scaling per row and vector.
 *   packed              2-bit codes from kq_pack_codes, one grid per row
 *   scale, zero         the grids of kq_gptaq_quantize (d_out floats each)
 *   s_x, s_g, sign_in, sign_out, blk_in, blk_out   as kq_apply_quantized
 *   x                   batch x d_in fp32, row-major (not modified)
 *   clip                clipping ratio of the activation grid, 0 < clip <= 1
 *   y                   batch x d_out fp32 output
 *   act_codes           NULL, or batch x d_in int8 output: the codes a
 *   act_scale           NULL, or batch floats output: the scales s
 * d_in must be a multiple of 512, d_out of 4, and 1 <= batch <= 65536 (the
 * launch grids' limit). packed, x, y, s_x and
 * act_codes must be 16-byte aligned. Workspace from
 * kq_workspace_size(KQ_OP_APPLY_QUANTIZED_A4, d_out, d_in, batch, ...).
 * Asynchronous. Errors: KQ_ERR_ARG (NULL, alignment, clip), KQ_ERR_SHAPE
 * (sizes, blocks), KQ_ERR_UNSUPPORTED (a block above 8192), KQ_ERR_WORKSPACE,
 * KQ_ERR_HIP. */
kq_status kq_apply_quantized_a4(const uint32_t* packed, const float* scale, const float* zero,
                                const float* s_x, const float* s_g, const int8_t* sign_in,
                                const int8_t* sign_out, int64_t blk_in, int64_t blk_out,
                                const float* x, int64_t batch, int64_t d_out, int64_t d_in,
                                float clip, float* y, int8_t* act_codes, float* act_scale,
                                void* ws, size_t ws_bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* KQ_H */
