/*
 * asp.h -- C ABI of libasp: the deflated Action-Subspace-Protection (ASP)
 * NVFP4 W4A4 linear layer on AMD Instinct MI355X (gfx950).
 *
 * The operation (model card "FastWAM UR3 3-task -- 4-bit quantisations",
 * section "What ASP is, and what the deflated form means"; Q-WAM abstract):
 * for one linear layer with weight W (N x K), bias b (N), smoothing vector s
 * (K), block Hadamard H and protected basis V (K x r, orthonormal columns),
 *
 *     x_tilde = (x / s) H                                (activation side)
 *     u       = x_tilde V
 *     y       = u (W_tilde V)^T
 *             + NVFP4GEMM( x_tilde - u V^T , W_tilde (I - V V^T) )
 *             + b,            with W_tilde = W diag(s) H  (weight side)
 *
 * NVFP4 (same page, method table): E2M1 elements in blocks of 16 consecutive
 * K elements with one E4M3 scale per block, for both operands.  The low-rank
 * branch stays in bf16 (same section): u and W_tilde V are rounded to bf16
 * for their product; the deflation uses the unrounded u.
 *
 * Readings this library takes where the pages are silent:
 *   - H: blocks of 128 consecutive channels, Sylvester order, 1/sqrt(128);
 *   - block scale S = E4M3FN(amax/6), round to nearest even, saturating at
 *     448 (no per-tensor second-level scale); element code = E2M1(|v|/S),
 *     round to nearest, ties to the even code, saturating at 6, sign copied
 *     from v (a zero scale gives magnitude 0 for the whole block);
 *   - the deflated operands are rounded to float32 before quantisation.
 *
 * Conventions for every entry point:
 *   - Row-major, K contiguous.  Row vectors: x is M x K, y is M x N.
 *   - Packed codes: row of `cols` elements -> cols/2 bytes; byte j holds
 *     element 2j in bits [3:0] and element 2j+1 in bits [7:4].
 *   - Block scales: one E4M3FN byte per 16 consecutive elements,
 *     [rows][cols/16].
 *   - bf16 values are passed as uint16_t bit patterns.
 *   - Every call returns an asp_status (int32_t).  Nothing throws across the
 *     ABI.  On failure asp_last_error() gives a thread-local description.
 *     Arguments are fully validated before anything is launched or written.
 *   - "device" pointers are HIP device memory owned by the caller; "host"
 *     pointers are ordinary host memory owned by the caller.  The library
 *     never allocates, frees or retains caller memory.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Device entry
 *     points only enqueue work and return; faults raised while kernels run
 *     surface at the caller's next synchronisation with that stream.
 *   - Device pointers must be 16-byte aligned.  Inputs must be finite.
 *   - Supported shapes: K a positive multiple of 128 (device entry points:
 *     at most 2^20); 0 <= M < 2^31 (M == 0 is a no-op); 1 <= N < 2^31;
 *     0 <= r <= 64.  Out-of-range shapes return ASP_ERR_SHAPE before
 *     anything is enqueued.
 */
#ifndef ASP_H
#define ASP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
#define ASP_OK 0
#define ASP_ERR_ARG 1         /* null pointer, unknown dtype, bad count */
#define ASP_ERR_SHAPE 2       /* shape outside the supported set */
#define ASP_ERR_ALIGN 3       /* device pointer not 16-byte aligned */
#define ASP_ERR_UNSUPPORTED 4 /* valid request this build does not handle */
#define ASP_ERR_WORKSPACE 5   /* workspace too small */
#define ASP_ERR_HIP 6         /* a HIP runtime call failed (launch, query) */
#define ASP_ERR_INTERNAL 7

/* Element types of x and y. */
#define ASP_F32 0
#define ASP_BF16 1

#define ASP_HADAMARD_BLOCK 128
#define ASP_QUANT_BLOCK 16
#define ASP_MAX_RANK 64

/* ABI revision of this header; bumps on any signature change. */
int32_t asp_abi_version(void);

/* Digest of the sources this library was built from (16 hex digits: sha256
 * of csrc/ and include/, as the build computes it), so that a caller holding
 * the sources can refuse a stale build.  Static text; never fails. */
const char* asp_source_digest(void);

/* Static text for a status code. */
const char* asp_status_string(int32_t status);

/* Thread-local description of the last failure on this thread ("" if none). */
const char* asp_last_error(void);

/* ------------------------------------------------------------------ host */

/*
 * Bytes of the packed weight buffers for an N x K layer of rank r:
 * codes N*K/2, scales N*K/16, low-rank factor N*r*2 (bf16).  These are the
 * model card's 4.00 bits per weight for the codes plus 0.5 bits for the E4M3
 * scales ("Verification -- NVFP4 deflated ASP", residency table).
 */
int32_t asp_packed_sizes(int64_t N, int64_t K, int32_t r, size_t* code_bytes,
                         size_t* scale_bytes, size_t* wv_bytes);

/*
 * Host-side weight packer (once per layer; CPU, synchronous).
 * Computes, in float64, W_tilde = W diag(s) H, L = W_tilde V and the deflated
 * weight W_d = W_tilde - L V^T (model card, "What ASP is, and what the
 * deflated form means": the 4-bit weight holds W_tilde (I - V V^T), the
 * low-rank branch the exact W_tilde V kept in bf16).  W_d is rounded to
 * float32 and NVFP4-quantised row-wise along K; L is rounded to bf16.
 *   w          host, N x K float32
 *   s          host, K float32, all > 0
 *   v          host, K x r float32 (NULL iff r == 0)
 *   w_codes    host out, N x K/2 bytes
 *   w_scales   host out, N x K/16 bytes
 *   wv         host out, N x r bf16 bits (NULL allowed iff r == 0)
 *   w_prequant host out, N x K float32 W_d before quantisation, or NULL
 *   n_threads  worker threads (<= 0: one per hardware thread)
 */
int32_t asp_pack_weight(int64_t N, int64_t K, int32_t r, const float* w,
                        const float* s, const float* v, uint8_t* w_codes,
                        uint8_t* w_scales, uint16_t* wv, float* w_prequant,
                        int32_t n_threads);

/*
 * The shared-weight arm of the same page (section "What ASP is, and what
 * the deflated form means": a cheaper variant with a single 4-bit weight and
 * only the basis V kept beside it).  Reading taken: the 4-bit weight is W_tilde itself (not deflated),
 * and the low-rank factor is derived from that one quantised weight, L =
 * DQ(Q(W_tilde)) V (decoded exactly, products in float64, rounded to bf16).
 * Arguments, layouts and the device path (asp_forward with the same
 * activation prep) as for asp_pack_weight; w_prequant receives float32(W_tilde).
 * Without quantisation it also reduces to x W^T + b, since the projector is
 * needed on one side only.
 */
int32_t asp_pack_weight_shared(int64_t N, int64_t K, int32_t r, const float* w,
                               const float* s, const float* v, uint8_t* w_codes,
                               uint8_t* w_scales, uint16_t* wv, float* w_prequant,
                               int32_t n_threads);

/*
 * NVFP4 quantiser on the host (the packer's last step, exposed for checks):
 * rows x cols float32 -> codes (rows x cols/2) and scales (rows x cols/16).
 * cols must be a positive multiple of 16.  All pointers host.
 */
int32_t asp_quantize_nvfp4_host(const float* in, int64_t rows, int64_t cols,
                                uint8_t* codes, uint8_t* scales);

/* Bytes of a layer's prep constants for K channels and rank r. */
int32_t asp_prep_pack_bytes(int64_t K, int32_t r, size_t* bytes);

/*
 * Per-layer constants of the activation prep (CPU, once per layer), from the
 * smoothing vector and the basis that define the layer's transforms (model
 * card, "What ASP is, and what the deflated form means": x_tilde = (x/s) H,
 * u = x_tilde V).  The buffer holds, in float64-derived form:
 *   1 / (s sqrt(128)) per channel (float64);
 *   V'' = diag(1/s) H V, so that u = x V'' (three bf16 terms, each the
 *   rounding of what the earlier ones leave: 24 or more significant bits);
 *   V itself, for the deflation (three bf16 terms: a float32 V exactly).
 * Its layout is private to the library; upload it unchanged.
 *   s          host, K float32, all > 0
 *   v          host, K x r float32 (NULL iff r == 0)
 *   prep_pack  host out, asp_prep_pack_bytes(K, r) bytes
 */
int32_t asp_pack_prep(int64_t K, int32_t r, const float* s, const float* v,
                      uint8_t* prep_pack);

/* ---------------------------------------------------------------- device */

/*
 * NVFP4 quantiser on the GPU: same arithmetic and layout as the host one.
 *   in (device, rows x cols float32) -> codes, scales (device).
 */
int32_t asp_quantize_nvfp4(const float* in, int64_t rows, int64_t cols,
                           uint8_t* codes, uint8_t* scales, void* stream);

/*
 * NVFP4 dequantiser on the GPU: out[i][j] = E2M1(code) * E4M3(scale), float32
 * (exact: every such product is a float32 value).  All pointers device.
 */
int32_t asp_dequantize_nvfp4(const uint8_t* codes, const uint8_t* scales,
                             int64_t rows, int64_t cols, float* out,
                             void* stream);

/* Workspace bytes asp_act_prep needs (partial sums of u; 0 when r == 0). */
int32_t asp_act_prep_workspace_bytes(int64_t M, int64_t K, int32_t r,
                                     size_t* bytes);

/*
 * Activation prep (every call): smooth-divide x/s, block Hadamard,
 * u = x_tilde V, deflation x_tilde - u V^T, NVFP4 quantise and pack
 * (model card, "What ASP is, and what the deflated form means").
 *   x          device, M x K, element type x_dtype (ASP_F32 or ASP_BF16)
 *   prep_pack  device, the layer's asp_pack_prep output
 *   x_codes    device out, M x K/2;  x_scales device out, M x K/16
 *   u          device out, M x r float32 (NULL allowed iff r == 0)
 *   prequant   device out, M x K float32 deflated activation before
 *              quantisation, or NULL (a check hook; costs bandwidth)
 *   workspace  device scratch of asp_act_prep_workspace_bytes bytes for the
 *              partial sums of u (NULL allowed when that is 0, i.e. r == 0);
 *              16-byte aligned; contents undefined afterwards
 * Deterministic: the same inputs give the same bits on every call, and a
 * row's results do not depend on the other rows of the batch.
 */
int32_t asp_act_prep(const void* x, int32_t x_dtype, int64_t M, int64_t K,
                     int32_t r, const uint8_t* prep_pack, uint8_t* x_codes,
                     uint8_t* x_scales, float* u, float* prequant,
                     void* workspace, size_t workspace_bytes, void* stream);

/*
 * The two launches of asp_act_prep as separate entry points (for profiling
 * each kernel on its own).  asp_act_prep_u writes the partial sums of u into
 * the workspace (nothing when r == 0); asp_act_prep_q, called afterwards on
 * the same stream with the same x, M, K, r, prep_pack and workspace, adds
 * them and produces x_codes, x_scales, u (and prequant).  Together they equal
 * asp_act_prep bit for bit.  Arguments as for asp_act_prep.
 */
int32_t asp_act_prep_u(const void* x, int32_t x_dtype, int64_t M, int64_t K,
                       int32_t r, const uint8_t* prep_pack, void* workspace,
                       size_t workspace_bytes, void* stream);
int32_t asp_act_prep_q(const void* x, int32_t x_dtype, int64_t M, int64_t K,
                       int32_t r, const uint8_t* prep_pack, uint8_t* x_codes,
                       uint8_t* x_scales, float* u, float* prequant,
                       void* workspace, size_t workspace_bytes, void* stream);

/*
 * 4-bit GEMM with fused low-rank and bias epilogue:
 *   y = DQ(x_codes, x_scales) DQ(w_codes, w_scales)^T + bf16(u) wv^T + bias
 * The NVFP4 operands are decoded in registers to exact fp16 values (an E2M1
 * value times an E4M3 scale has at most 6 significant bits) and contracted
 * on MFMA with float32 accumulation; no dequantised copy of either operand
 * is written to memory (model card, "Verification -- NVFP4 deflated ASP":
 * no dequantised weight copy anywhere).
 *   x_codes, x_scales  device, M x K/2, M x K/16 (asp_act_prep output)
 *   u                  device, M x r float32 (NULL iff r == 0)
 *   w_codes, w_scales  device, N x K/2, N x K/16 (asp_pack_weight output)
 *   wv                 device, N x r bf16 bits (NULL iff r == 0)
 *   bias               device, N float32, or NULL for none
 *   y                  device out, M x N, element type y_dtype
 */
int32_t asp_gemm_lowrank(const uint8_t* x_codes, const uint8_t* x_scales,
                         const float* u, int64_t M, int64_t N, int64_t K,
                         int32_t r, const uint8_t* w_codes,
                         const uint8_t* w_scales, const uint16_t* wv,
                         const float* bias, void* y, int32_t y_dtype,
                         void* stream);

/*
 * Name of the GPU kernel asp_gemm_lowrank launches for an M x N x K call, as
 * a profiler lists it (for example "k_gemm<4, 2, 2, 3>"); "" for a shape the
 * GEMM rejects.  Host only; the string is static and owned by the library.
 */
const char* asp_gemm_kernel_name(int64_t M, int64_t N, int64_t K);

/* Workspace bytes asp_forward needs (activation codes, scales, u, prep scratch). */
int32_t asp_workspace_bytes(int64_t M, int64_t N, int64_t K, int32_t r,
                            size_t* bytes);

/*
 * The whole layer on the GPU: asp_act_prep then asp_gemm_lowrank, enqueued
 * on `stream`, with the activation codes, scales and u in the caller's
 * workspace (device, at least asp_workspace_bytes bytes, 256-byte aligned).
 * prep_pack, w_codes, w_scales and wv are the layer's asp_pack_prep and
 * asp_pack_weight outputs uploaded to the device.
 */
int32_t asp_forward(const void* x, int32_t x_dtype, int64_t M, int64_t N,
                    int64_t K, int32_t r, const uint8_t* prep_pack,
                    const uint8_t* w_codes, const uint8_t* w_scales,
                    const uint16_t* wv, const float* bias, void* y,
                    int32_t y_dtype, void* workspace, size_t workspace_bytes,
                    void* stream);

/* Bytes of the device-resident workspace of asp_forward_noalloc (48 MiB per
 * GPU): enough for M x K up to about 4096 x 14336 at r = 0. */
#define ASP_NOALLOC_SCRATCH_BYTES (48u << 20)

/*
 * asp_forward without a workspace argument, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc.  The workspace is a file-scope device array of
 * ASP_NOALLOC_SCRATCH_BYTES, one per GPU, whose address the library takes on
 * its first call on that GPU and which lives until the process ends; this
 * call allocates and frees nothing.  Inputs, outputs, their layout and the
 * result are exactly those of asp_forward (the same kernels, the same bits).
 *   stream  selects the GPU (its device; NULL: the current device)
 * Errors: as asp_forward, and ASP_ERR_WORKSPACE (before anything is enqueued)
 * when asp_workspace_bytes(M, N, K, r) exceeds ASP_NOALLOC_SCRATCH_BYTES.
 * Every call on one GPU uses that GPU's one array: calls that overlap on one
 * GPU (other streams, other threads, before an earlier one has finished)
 * race and corrupt each other's results; serialise them on one stream.
 */
int32_t asp_forward_noalloc(const void* x, int32_t x_dtype, int64_t M, int64_t N,
                            int64_t K, int32_t r, const uint8_t* prep_pack,
                            const uint8_t* w_codes, const uint8_t* w_scales,
                            const uint16_t* wv, const float* bias, void* y,
                            int32_t y_dtype, void* stream);

/*
 * Several layers that share M, K and r (for example projections that read
 * the same input) in one call: each of the three kernels is launched once
 * for the whole group, so small layers fill more of the GPU and share the
 * launch cost.  Layer i computes exactly what asp_forward computes with
 * x[i], prep_pack[i], w_codes[i], w_scales[i], wv[i], bias[i], N[i], y[i]
 * and workspace[i]; the GEMM kernel is chosen for the group's total width
 * sum(N), so the float32 accumulation order of a layer can differ from a
 * lone asp_forward call when that choice differs (asp_gemm_kernel_name(M,
 * sum(N), K) names it).
 *   n_layers          1..8
 *   x .. workspace    host arrays of n_layers device pointers (x[i] may
 *                     repeat); bias may be NULL (no bias anywhere) and so
 *                     may its entries; wv may be NULL when r == 0
 *   N                 host array of n_layers output widths
 *   workspace_bytes   host array; each at least asp_workspace_bytes(M,
 *                     N[i], K, r), each workspace 256-byte aligned; the
 *                     workspaces must not overlap
 * Errors as asp_forward; nothing is enqueued unless every layer validates.
 */
int32_t asp_forward_group(int32_t n_layers, const void* const* x,
                          int32_t x_dtype, int64_t M, int64_t K, int32_t r,
                          const uint8_t* const* prep_pack,
                          const uint8_t* const* w_codes,
                          const uint8_t* const* w_scales,
                          const uint16_t* const* wv, const float* const* bias,
                          const int64_t* N, void* const* y, int32_t y_dtype,
                          void* const* workspace,
                          const size_t* workspace_bytes, void* stream);

/*
 * asp_forward_group one kernel at a time (for profiling each launch on its
 * own): stages is a bit mask of 1 = k_prep_u (the partial sums of u), 2 =
 * k_prep_q (codes, scales, u), 4 = the GEMM; 7 is asp_forward_group.  Each
 * stage reads what the earlier ones left in the workspaces, so they must run
 * in that order on one stream with the same arguments.
 */
int32_t asp_forward_group_stages(int32_t stages, int32_t n_layers,
                                 const void* const* x, int32_t x_dtype,
                                 int64_t M, int64_t K, int32_t r,
                                 const uint8_t* const* prep_pack,
                                 const uint8_t* const* w_codes,
                                 const uint8_t* const* w_scales,
                                 const uint16_t* const* wv,
                                 const float* const* bias, const int64_t* N,
                                 void* const* y, int32_t y_dtype,
                                 void* const* workspace,
                                 const size_t* workspace_bytes, void* stream);

/* ------------------------------------------------------- calibration */

/*
 * Per-layer smoothing search (model card, section "What ASP is, and what the
 * deflated form means": the smoothing exponents of each layer are picked
 * from a grid by that layer's own deflated-ASP NVFP4 output error on
 * calibration activations).  For candidate c the smoothing vector is
 *     s_k = max_m |x_mk|^alphas[c] / max_n |W_nk|^betas[c]
 * in float64 (a zero maximum replaced by 1e-5), rounded to float32; the weight
 * is packed with it (asp_pack_weight, host), the layer runs on the device
 * (asp_forward, float32 output) and mse[c] is the mean over the M x N outputs
 * of the squared difference to the unquantised x W^T + b (a float32 GEMM on
 * the device; squares summed in float64 in a fixed order, so the result is
 * deterministic).  *best = the index of the smallest mse (ties: the earlier).
 * Runs on `stream` and synchronises it before returning (offline use).
 *   x              device, M x K calibration activations (x_dtype)
 *   w, bias, v     host float32: N x K, N or NULL, K x r (NULL iff r == 0)
 *   alphas, betas  host, n_candidates each
 *   mse, best      host out, n_candidates doubles and one index
 *   workspace      device, asp_smoothing_search_workspace_bytes bytes,
 *                  256-byte aligned
 */
int32_t asp_smoothing_search_workspace_bytes(int64_t M, int64_t N, int64_t K,
                                             int32_t r, int32_t n_candidates,
                                             size_t* bytes);
int32_t asp_smoothing_search(const void* x, int32_t x_dtype, int64_t M,
                             int64_t K, const float* w, const float* bias,
                             int64_t N, const float* v, int32_t r,
                             const float* alphas, const float* betas,
                             int32_t n_candidates, double* mse,
                             int32_t* best, void* workspace,
                             size_t workspace_bytes, void* stream);

/*
 * Top-r eigenspace of a layer's action metric: the protected basis V.
 * Model card "FastWAM UR3 3-task -- 4-bit quantisations", section "What ASP
 * is, and what the deflated form means": V spans the top eigenspace of the
 * metric G = E[J^T J] (J: the action's sensitivity to the layer input);
 * Q-WAM, Figure 3(b): its leading eigenvalues fall quickly.  G itself is the
 * caller's (it needs the trained model); this finds its leading eigenpairs.
 *
 * Subspace iteration on G + mu I (mu = 2^-16 ||G||_F, or 1 when G = 0, so the
 * iterates keep full rank) from the caller's random start V0, Cholesky QR
 * after every product, a second Cholesky QR pass, then Rayleigh-Ritz on
 * G itself (Jacobi rotations on the p x p projection).  All arithmetic is
 * float64.  Convergence of pair i goes as ((lam_{p+1} + mu)/(lam_i + mu))^iters:
 * choose p above r and iters from the spectrum's decay; resid reports
 * ||G v_i - theta_i v_i|| so the caller can check it.
 *
 *   g        device float32 K x K, symmetric positive semi-definite (only
 *            symmetric G is meaningful: its rows are read as its columns)
 *   K        a positive multiple of 128, at most 65536
 *   v0       device float32 K x p, full column rank (e.g. N(0, 1) draws)
 *   p        block width: 16, 32, 48 or 64
 *   r        1 <= r <= p: eigenpairs returned
 *   iters    >= 0 products with G before the Rayleigh-Ritz step
 *   v        device out float32 K x r, orthonormal columns, column i the Ritz
 *            vector of the i-th largest Ritz value; its entry of largest
 *            magnitude (first row on ties) is positive
 *   evals    device out float32 r, largest first; all NaN when the
 *            orthonormalisation broke down (G not finite, or far from PSD)
 *   resid    device out float32 r or NULL: ||G v_i - evals_i v_i||_2
 *   workspace device, asp_top_eigenspace_workspace_bytes bytes, 256-byte
 *            aligned; overwritten
 * Results are bitwise reproducible (every reduction has a fixed order).
 * asp_top_eigenspace_slices reports how many K-slices the G V product uses
 * (each slice's partial product is summed in a fixed order).
 */
int32_t asp_top_eigenspace_workspace_bytes(int64_t K, int32_t p, int32_t r,
                                           size_t* bytes);
int32_t asp_top_eigenspace_slices(int64_t K, int32_t p, int32_t* slices);
/*
 * The metric product the eigenspace iteration is built on, as K-sliced
 * partial sums: yp[s] = G[:, slice s] V[slice s, :] for s < S, with
 * S = asp_top_eigenspace_slices(K, p) equal slices of K, so that
 * G V = yp[0] + ... + yp[S-1].  float64 MFMA arithmetic.
 *   g   device float32 K x K (K, p as for asp_top_eigenspace)
 *   v   device float64 K x p
 *   yp  device out float64 S x K x p
 */
int32_t asp_metric_product_partials(const float* g, int64_t K, const double* v,
                                    int32_t p, double* yp, void* stream);
int32_t asp_top_eigenspace(const float* g, int64_t K, const float* v0,
                           int32_t p, int32_t r, int32_t iters, float* v,
                           float* evals, float* resid, void* workspace,
                           size_t workspace_bytes, void* stream);

/*
 * SVDQuant-style INT4 W4A4 arm.  Model card "FastWAM UR3 3-task -- 4-bit
 * quantisations": method table (the second checkpoint: INT4 with groups of 64
 * for weights and activations, contracted on INT8 tensor cores, exact for
 * 4-bit codes) and section "Verification -- INT4 SVDQuant".  The smoothed
 * weight W_hat = W diag(s) is split into a rank-r bfloat16 branch L1 L2 (its
 * truncated SVD: L2 = V_r^T, the top right singular vectors, L1 = W_hat V_r)
 * and a residual R = W_hat - L1 L2 quantised to INT4 together with
 * x_hat = float32(x * float32(1/s)):
 *     y = bfloat16(u) L1^T + sum_g sx[m,g] sw[n,g] sum_{k in g} qx qw + b,
 *     u = x diag(1/s) V_r (float32 accumulation).
 * Group quantiser (both operands): scale = bfloat16(float32(amax) / 7), code =
 * clamp(rint(v / scale), -8, 7) in float32 (ties to even); a zero scale gives
 * zero codes.  Codes: two's-complement nibbles, element 2j in the low nibble
 * of byte j, rows of K/2 bytes.  Scales, group-major: (K/64) rows of N128
 * (weights: bfloat16 bits, padding zero) or M128 (activations: the bfloat16
 * values held as float32, padding undefined) entries, the count rounded up
 * to 128.
 *
 * asp_svdq_packed_sizes: bytes of the codes, scales, L1 (N x rp32 bf16, r
 *   rounded up to 32, zero padded) and prep pack of one layer (host).
 * asp_svdq_gram: g (host, K x K float32, exactly symmetric) = W_hat^T W_hat
 *   in float64; its top-r eigenvectors (asp_top_eigenspace) are V_r.
 * asp_svdq_pack_weight (host): from W (N x K), s (K, positive) and V_r
 *   (K x r float32, orthonormal columns; NULL iff r == 0) writes codes,
 *   scales, l1 and prep (1/s and diag(1/s) V_r for u), all host buffers of
 *   asp_svdq_packed_sizes bytes.
 * asp_svdq_act_quant (device): x (M x K, f32 or bf16) -> x_codes (M x K/2)
 *   and x_scales ((K/64) x M128 float32), using the 1/s of prep_pack.
 * asp_svdq_gemm (device): y from activation codes/scales, u (M x rp32
 *   float32, the columns past r zero; rounded to bfloat16 inside), the packed
 *   weight, l1 and bias (N or NULL).
 * asp_svdq_forward (device): the whole layer, with u, the activation codes
 *   and scales in the caller's workspace (asp_svdq_workspace_bytes bytes,
 *   256-byte aligned).  K a multiple of 128; 0 <= r <= 64; M >= 0.
 */
int32_t asp_svdq_packed_sizes(int64_t N, int64_t K, int32_t r, size_t* code_bytes,
                              size_t* scale_bytes, size_t* l1_bytes, size_t* prep_bytes);
int32_t asp_svdq_gram(int64_t N, int64_t K, const float* w, const float* s, float* g);
int32_t asp_svdq_pack_weight(int64_t N, int64_t K, int32_t r, const float* w,
                             const float* s, const float* v, uint8_t* codes,
                             uint16_t* scales, uint16_t* l1, uint8_t* prep);
int32_t asp_svdq_workspace_bytes(int64_t M, int64_t N, int64_t K, int32_t r, size_t* bytes);
int32_t asp_svdq_act_quant(const void* x, int32_t x_dtype, int64_t M, int64_t K,
                           const uint8_t* prep_pack, uint8_t* x_codes,
                           float* x_scales, void* stream);
int32_t asp_svdq_gemm(const uint8_t* x_codes, const float* x_scales, const float* u,
                      int64_t M, int64_t N, int64_t K, int32_t r, const uint8_t* w_codes,
                      const uint16_t* w_scales, const uint16_t* l1, const float* bias,
                      void* y, int32_t y_dtype, void* stream);
int32_t asp_svdq_forward(const void* x, int32_t x_dtype, int64_t M, int64_t K, int32_t r,
                         const uint8_t* prep_pack, const uint8_t* w_codes,
                         const uint16_t* w_scales, const uint16_t* l1, const float* bias,
                         int64_t N, void* y, int32_t y_dtype, void* workspace,
                         size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* ASP_H */
