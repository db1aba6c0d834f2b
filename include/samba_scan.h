/*
 * samba_scan.h -- C ABI of the MI355X (gfx950) selective-scan core of a Mamba layer,
 * as used in the Samba hybrid model.
 *
 * What is computed (page "Samba: Simple Hybrid State Space Models for Efficient
 * Unlimited Context Language Modeling", paper-graph-ui summary, section 3.4), per
 * sequence s, channel d and token t:
 *
 *   u_t   = SiLU(conv_b[d] + sum_{k=0..3} conv_w[d][k] * x_{t-3+k})   "Input Projection and
 *                                                                     Short Convolution"
 *   Delta = softplus(dt_t + dt_bias[d])                               "Input-Dependent
 *                                                                     Selective Gating"
 *   h_t[n] = exp(Delta * A[d][n]) * h_{t-1}[n] + Delta * B_t[n] * u_t  "The State Space
 *   y_t    = sum_n C_t[n] * h_t[n] + D[d] * u_t                          Model Update (S6)"
 *   out_t  = y_t * SiLU(z_t)                                           "Gated Output"
 *
 * The conv is causal with the previous three pre-conv inputs taken from the history
 * (zeros at a fresh sequence start), tap k multiplying x_{t-3+k}; A is used as given
 * (normally negative, A = -exp(A_log)); the gate is SiLU(z) -- these follow "Samba Guide:
 * Hybrid Mamba & Sliding Window Architecture", "Step 1: The Selective State Space (Mamba)
 * Layer".  The scan entry points take x, dt, B, C and z as inputs; the projections that
 * make them (and the layer's output projection, the attention and MLP projections) are
 * bf16 matrix-core GEMMs of their own, samba_gemm below.  samba_scan_prefill_u /
 * samba_scan_varlen_u take the post-conv activation u instead of x.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Every array pointer is a DEVICE pointer on the current HIP device, owned by the
 *   caller; the library keeps no reference after the call returns.
 * - Token tensors are token-major and contiguous: x, dt, z, out are [tokens][d_inner]
 *   with the channel index fastest; B and C are [tokens][d_state] and shared by all
 *   channels of their sequence.
 * - I/O dtype `io` applies to x, dt, z, B, C, out and the conv history: SAMBA_F32
 *   (float) or SAMBA_BF16 (bfloat16 bits, stored as uint16).  Outputs in bf16 are
 *   rounded to nearest even.  Parameters and the state h are always float32; all
 *   arithmetic is float32.
 * - The recurrent state is [seq][d_inner][d_state] float32 (state index fastest).
 * - The conv history is [seq][3][d_inner] in the I/O dtype.  Prefill takes and returns it
 *   oldest token first; decode keeps it as a ring of three slots with a head index per
 *   sequence (the slot of the oldest token), so that a step writes one slot.  A prefill's
 *   conv_final can be passed unchanged as the next prefill's conv0, or as the decode ring
 *   with head 0.
 * - d_state must be in [1, 16]; d_inner >= 1; every pointer must be aligned to 16 bytes.
 * - Calls are asynchronous on `stream` (a hipStream_t; NULL = the default stream) and
 *   return once the work is enqueued.  Outputs must not overlap inputs or each other,
 *   except the in/out arguments of the decode steps and a prefill's h_final / conv_final
 *   passed as the very same pointers as h0 / conv0; the byte ranges the shapes define are
 *   compared on the host and an overlap is refused with SAMBA_ERR_INVALID_ARG.
 * - Errors: arguments are checked on the host before anything is enqueued; a failing
 *   check returns a non-zero samba_status, enqueues nothing and sets a thread-local
 *   message readable with samba_last_error().  A launch failure returns SAMBA_ERR_HIP.
 *   Faults inside a kernel surface at the caller's next synchronisation.  The library
 *   never aborts the process.
 * - Environment, read at every call, for tests and timing (each computes the same function;
 *   results may differ by rounding where the kernel changes):
 *   SAMBA_SCAN_PATH=lane|single|split forces the prefill kernel family (otherwise chosen by
 *   shape); SAMBA_GEMM_TILE=128|256 forces the GEMM tile size; SAMBA_DECODE_NOFUSE set makes
 *   samba_decode_step run every kernel separately instead of folding the conv and the next
 *   RMSNorm into the split-K reduces (bitwise the same results).
 */
#ifndef SAMBA_SCAN_H
#define SAMBA_SCAN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Each enum below also lists a FORCE_INT32 value that is never a valid argument: it makes
 * every int a value of the type, so an out-of-range argument is rejected by the checks
 * (SAMBA_ERR_INVALID_ARG) instead of being undefined behaviour in the C++ implementation. */
typedef enum { SAMBA_F32 = 0, SAMBA_BF16 = 1, SAMBA_DTYPE_FORCE_INT32 = -2147483647 - 1 } samba_dtype;

typedef enum {
    SAMBA_OK = 0,
    SAMBA_ERR_INVALID_ARG = 1, /* null/misaligned pointer, negative or inconsistent size */
    SAMBA_ERR_UNSUPPORTED = 2, /* valid request this build does not handle (d_state > 16) */
    SAMBA_ERR_WORKSPACE = 3,   /* workspace missing or smaller than samba_scan_workspace_bytes() */
    SAMBA_ERR_HIP = 4          /* the HIP runtime reported an error; see samba_last_error() */
} samba_status;

/* Layer parameters, all float32 device pointers, read-only.
 *   A       [d_inner][d_state]  multiplies Delta inside exp (page 1 section 3.4, "The State
 *                               Space Model Update (S6)")
 *   D       [d_inner]           skip weight; NULL means 0
 *   dt_bias [d_inner]           bias inside softplus ("Input-Dependent Selective Gating");
 *                               NULL means 0
 *   conv_w  [d_inner][4]        depthwise taps; tap k multiplies x_{t-3+k}
 *   conv_b  [d_inner]           conv bias; NULL means 0 */
typedef struct {
    const float *A;
    const float *D;
    const float *dt_bias;
    const float *conv_w;
    const float *conv_b;
} samba_params;

/* Size in bytes of the device workspace samba_scan_prefill / samba_scan_varlen need for
 * this problem (0 means none: pass NULL).  nseq is the batch (or number of packed
 * sequences), max_seqlen the longest sequence. */
size_t samba_scan_workspace_bytes(int nseq, int max_seqlen, int d_inner, int d_state);

/* Fixed-length prefill of `batch` sequences of `seqlen` tokens (the chunk-parallel form of
 * the recurrence, page 1 section 3.4 "The State Space Model Update (S6)", last paragraph;
 * passing the final state forward between chunks as in the Samba Guide's "Chunked
 * Prefilling" practice).
 *   x, dt, z, out [batch][seqlen][d_inner]; B, C [batch][seqlen][d_state]   (io dtype)
 *   z        may be NULL: no gate (out = y)
 *   h0       [batch][d_inner][d_state] float32 initial state; NULL = zeros
 *   conv0    [batch][3][d_inner] (io dtype) history before token 0; NULL = zeros
 *   h_final  [batch][d_inner][d_state] float32, may be NULL; may equal h0 (in place)
 *   conv_final [batch][3][d_inner] (io dtype), may be NULL; may equal conv0
 *   workspace / workspace_bytes: see samba_scan_workspace_bytes()
 * seqlen == 0 copies h0/conv0 (or zeros) into h_final/conv_final.  batch == 0 is a no-op. */
samba_status samba_scan_prefill(int batch, int seqlen, int d_inner, int d_state, samba_dtype io,
                                const void *x, const void *dt, const void *B, const void *C,
                                const void *z, const samba_params *params,
                                const float *h0, const void *conv0,
                                void *out, float *h_final, void *conv_final,
                                void *workspace, size_t workspace_bytes, void *stream);

/* Packed variable-length prefill: sequence s covers tokens [cu_seqlens[s], cu_seqlens[s+1])
 * of the packed arrays (x, dt, z, out [total_tokens][d_inner]; B, C [total_tokens][d_state]).
 * State and conv history restart at every sequence start from h0[s] / conv0[s] (zeros
 * when NULL) and are never carried across a boundary; h_final[s] / conv_final[s] receive
 * each sequence's final values.
 *   cu_seqlens  DEVICE int32 [nseq + 1], non-decreasing, cu_seqlens[0] = 0 and
 *               cu_seqlens[nseq] = total_tokens (the caller's contract; not re-read on
 *               the host)
 *   max_seqlen  host int >= every sequence length (sizes the launch) */
samba_status samba_scan_varlen(int nseq, const int32_t *cu_seqlens, int total_tokens, int max_seqlen,
                               int d_inner, int d_state, samba_dtype io,
                               const void *x, const void *dt, const void *B, const void *C,
                               const void *z, const samba_params *params,
                               const float *h0, const void *conv0,
                               void *out, float *h_final, void *conv_final,
                               void *workspace, size_t workspace_bytes, void *stream);

/* The same two calls from a precomputed u = SiLU(conv_b + sum_k conv_w[k] x_{t-3+k}) instead
 * of x: in a full Mamba layer, Delta, B and C are projections of u (page 1 section 3.4,
 * "Input-Dependent SSM Parameters": x_proj reads u), so u already exists -- samba_conv_silu
 * computes it, with the outgoing conv history -- before the scan runs.  The scan then skips
 * the conv: Delta = softplus(dt + dt_bias), h_t = exp(Delta A) h_{t-1} + Delta B_t u_t,
 * out = (C_t . h_t + D u_t) SiLU(z_t).
 *   u        [batch][seqlen][d_inner] (prefill_u) or [total_tokens][d_inner] (varlen_u), io dtype
 *   params   A required; D and dt_bias as above; conv_w and conv_b are not read (may be NULL)
 * Every other argument as for samba_scan_prefill / samba_scan_varlen (there is no conv
 * history in or out). */
samba_status samba_scan_prefill_u(int batch, int seqlen, int d_inner, int d_state, samba_dtype io,
                                  const void *u, const void *dt, const void *B, const void *C,
                                  const void *z, const samba_params *params, const float *h0,
                                  void *out, float *h_final, void *workspace, size_t workspace_bytes, void *stream);
samba_status samba_scan_varlen_u(int nseq, const int32_t *cu_seqlens, int total_tokens, int max_seqlen,
                                 int d_inner, int d_state, samba_dtype io, const void *u, const void *dt,
                                 const void *B, const void *C, const void *z, const samba_params *params,
                                 const float *h0, void *out, float *h_final, void *workspace,
                                 size_t workspace_bytes, void *stream);

/* One decode step: one new token for each of nseq resident sequences (the constant
 * per-token cost of the fixed-size state, page 1 section 5 "Experimental Analysis",
 * generation throughput; the recurrence of section 3.4 with L = 1).
 *   x, dt, z, out [nseq][d_inner]; B, C [nseq][d_state]   (io dtype); z may be NULL
 *   h          [nseq][d_inner][d_state] float32, IN/OUT: updated in place
 *   conv_ring  [nseq][3][d_inner] (io dtype), IN/OUT: the last three pre-conv inputs as a
 *              ring: with hd = ring_head_in[s] mod 3, slot (hd + k) mod 3 holds x_{t-3+k}
 *              (k = 0 oldest).  The step reads the three slots and writes the new input x_t
 *              into slot hd only.
 *   ring_head_in  DEVICE int32 [nseq], required: each sequence's head (any value; taken
 *              mod 3).  Not modified.  A prefill's conv_final is a ring with head 0.
 *   ring_head_out DEVICE int32 [nseq] or NULL: receives (hd + 1) mod 3, the head of the
 *              next step.  Must not overlap ring_head_in (every workgroup of a sequence
 *              reads its head during the step, so the heads are double-buffered).
 * Limits: nseq <= 65535 (SAMBA_ERR_UNSUPPORTED beyond).  Bytes moved per sequence and
 * channel: the state read and written (2 x 64 B at d_state 16), three ring slots read and
 * one written, x, dt, z read and out written. */
samba_status samba_scan_decode(int nseq, int d_inner, int d_state, samba_dtype io,
                               const void *x, const void *dt, const void *B, const void *C,
                               const void *z, const samba_params *params,
                               float *h, void *conv_ring, const int32_t *ring_head_in, int32_t *ring_head_out,
                               void *out, void *stream);

/* The short causal convolution and its SiLU alone (page 1 section 3.4, "Input Projection
 * and Short Convolution"): u_t = SiLU(conv_b + sum_k conv_w[k] x_{t-3+k}), the activation a
 * full Mamba layer feeds to its x_proj (whose outputs dt, B, C the scan consumes).  The
 * scan entry points recompute u from x internally; this call exists for x_proj's input.
 *   cu_seqlens NULL: nseq sequences of seqlen tokens, x and u [nseq][seqlen][d_inner];
 *              total_tokens is ignored.
 *   cu_seqlens non-NULL (DEVICE int32 [nseq + 1], as for samba_scan_varlen): packed
 *              sequences, x and u [total_tokens][d_inner]; seqlen is the longest
 *              sequence (max_seqlen, sizes the launch).
 *   conv_w [d_inner][4], conv_b [d_inner] (NULL = 0): float32, as in samba_params
 *   conv0  [nseq][3][d_inner] (io dtype) history before each sequence; NULL = zeros
 *   u      (io dtype) output; must not overlap x
 *   conv_final [nseq][3][d_inner] (io dtype), may be NULL: each sequence's last three
 *              inputs, oldest first (the history for the next chunk or for decode);
 *              must not overlap conv0.
 * Returns SAMBA_ERR_INVALID_ARG for negative sizes, NULL or misaligned required pointers
 * and overlapping outputs; nseq == 0 is a no-op. */
samba_status samba_conv_silu(int nseq, const int32_t *cu_seqlens, int seqlen, int total_tokens, int d_inner,
                             samba_dtype io, const void *x, const float *conv_w, const float *conv_b,
                             const void *conv0, void *u, void *conv_final, void *stream);

/* Size in bytes of the device workspace samba_scan_backward needs (nseq sequences of at
 * most seqlen tokens, total_tokens tokens in all). */
size_t samba_scan_backward_workspace_bytes(int nseq, int seqlen, int total_tokens, int d_inner, int d_state);

/* Gradients of the layer for training: reverse-mode differentiation of the computation
 * above (page 1 section 3.4, the steps from "Input Projection and Short Convolution" to
 * "Gated Output"; the pages train the model at 4K tokens, "Training Configurations and
 * Scaling").  The loss is taken as sum(dout . out) + sum(dh_final . h_final) +
 * sum(dconv_final . conv_final): dout is the gradient of the layer output, dh_final and
 * dconv_final (NULL = zero) those of the final state and outgoing conv history.
 *   cu_seqlens NULL: nseq sequences of seqlen tokens (token tensors [nseq][seqlen][...]);
 *              total_tokens is ignored.  Non-NULL: packed as for samba_scan_varlen, seqlen
 *              = the longest sequence.
 *   x, dt, B, C, z, params, h0, conv0: the forward call's inputs (the forward is
 *              recomputed; nothing from the forward call is needed)
 *   dout [tokens][d_inner] (io dtype); dh_final [nseq][d_inner][d_state] float32;
 *   dconv_final [nseq][3][d_inner] (io dtype)
 * Outputs (overwritten, not accumulated):
 *   dx, ddt, dz [tokens][d_inner], dB, dC [tokens][d_state]   io dtype; dz required when
 *              z is given (ignored otherwise)
 *   dA [d_inner][d_state], dD, ddt_bias, dconv_b [d_inner], dconv_w [d_inner][4]   float32,
 *              summed over all sequences and tokens (dD / ddt_bias / dconv_b are the
 *              gradients of a zero parameter when its pointer in params is NULL)
 *   dh0 [nseq][d_inner][d_state] float32, dconv0 [nseq][3][d_inner] io dtype: gradients of
 *              the initial state and history; either may be NULL
 *   workspace: at least samba_scan_backward_workspace_bytes() bytes, 256-byte aligned,
 *              contents irrelevant (SAMBA_ERR_WORKSPACE otherwise)
 * Outputs must not overlap inputs or each other.  Limits: nseq <= 65535 and seqlen <=
 * 65535 * 16 (SAMBA_ERR_UNSUPPORTED beyond). */
samba_status samba_scan_backward(int nseq, const int32_t *cu_seqlens, int seqlen, int total_tokens, int d_inner,
                                 int d_state, samba_dtype io, const void *x, const void *dt, const void *B,
                                 const void *C, const void *z, const samba_params *params, const float *h0,
                                 const void *conv0, const void *dout, const float *dh_final,
                                 const void *dconv_final, void *dx, void *ddt, void *dB, void *dC, void *dz,
                                 float *dA, float *dD, float *ddt_bias, float *dconv_w, float *dconv_b,
                                 float *dh0, void *dconv0, void *workspace, size_t workspace_bytes, void *stream);

/* Size in bytes of the device workspace samba_swa_prefill needs (the rotated keys). */
size_t samba_swa_workspace_bytes(int total_tokens, int n_kv_heads, int head_dim);

/* Sliding window attention, the other sequence mixer of the Samba layer stack (page 1,
 * "The Sliding Window Attention (SWA) Layer"): the query at position t of a sequence
 * attends to the keys at positions t - window .. t of the same sequence ("Window
 * Specification"), queries and keys rotated by RoPE with base rope_base ("Positional
 * Encoding"; pairs (2i, 2i+1) turn by position * base^(-2i/head_dim), positions counting
 * from each sequence start), softmax of the scores scaled by 1/sqrt(head_dim).  Query
 * head h reads key/value head h / (n_heads / n_kv_heads) (grouped-query attention, as in
 * the pages' 1.7B and 3.8B configurations).
 *   cu_seqlens NULL: nseq sequences of seqlen tokens, q, out [nseq][seqlen][n_heads][head_dim],
 *              k, v [nseq][seqlen][n_kv_heads][head_dim]; total_tokens is ignored.
 *              Non-NULL: packed as for samba_scan_varlen ([total_tokens][heads][head_dim]),
 *              seqlen = the longest sequence.
 *   io must be SAMBA_BF16 (the matrix-core operand type; SAMBA_ERR_UNSUPPORTED otherwise);
 *   head_dim 64 or 128 (SAMBA_ERR_UNSUPPORTED otherwise); window >= 0; rope_base > 1.
 *   workspace: at least samba_swa_workspace_bytes() bytes, 16-byte aligned.
 * out must not overlap the inputs or the workspace. */
samba_status samba_swa_prefill(int nseq, const int32_t *cu_seqlens, int seqlen, int total_tokens, int n_heads,
                               int n_kv_heads, int head_dim, int window, float rope_base, samba_dtype io,
                               const void *q, const void *k, const void *v, void *out, void *workspace,
                               size_t workspace_bytes, void *stream);

/* Size in bytes of the workspace samba_swa_decode needs (per-split partial results). */
size_t samba_swa_decode_workspace_bytes(int nseq, int n_heads, int head_dim);

/* One decode step of sliding window attention for nseq sequences over ring-buffer KV caches
 * (a query at position t reads the keys t - window .. t: "Window Specification" on page 1,
 * so each sequence keeps only window + 1 keys and values, whatever its length).
 *   q [nseq][n_heads][head_dim], k, v [nseq][n_kv_heads][head_dim]: the new token (bf16)
 *   pos      DEVICE int32 [nseq]: the new token's position (tokens before it); a sequence
 *            with pos < 0 is skipped (its out rows are set to 0). Not modified.
 *   k_cache, v_cache [nseq][n_kv_heads][window + 1][head_dim] bf16, IN/OUT: position p is
 *            kept in entry p mod (window + 1), keys rotated by RoPE at p; the step writes the
 *            new token's entry, then attends over the window.
 *   out [nseq][n_heads][head_dim] bf16.
 *   n_heads / n_kv_heads <= 16; head_dim 64 or 128; io must be SAMBA_BF16.
 *   workspace: at least samba_swa_decode_workspace_bytes() bytes, 16-byte aligned. */
samba_status samba_swa_decode(int nseq, int n_heads, int n_kv_heads, int head_dim, int window, float rope_base,
                              samba_dtype io, const void *q, const void *k, const void *v, const int32_t *pos,
                              void *k_cache, void *v_cache, void *out, void *workspace, size_t workspace_bytes,
                              void *stream);

/* samba_swa_decode for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same computation and
 * arguments without a workspace.  The split partials go to a device array inside the library
 * (samba_swa_decode_noalloc_max_bytes() bytes, 24 MiB, one copy per GPU held until the
 * process ends); the call allocates nothing.
 *   Limit: samba_swa_decode_workspace_bytes(nseq, n_heads, head_dim) must not exceed the
 *   array (e.g. 256 sequences x 32 heads x head_dim 128 fit); SAMBA_ERR_UNSUPPORTED
 *   otherwise, before anything is enqueued.
 *   Every call on one GPU uses that GPU's single array: calls that overlap on one GPU (on
 *   different streams, or from different threads) race and must be serialised by the
 *   caller.  The first call on a device looks the array's address up (hipGetSymbolAddress);
 *   a failure returns SAMBA_ERR_HIP. */
samba_status samba_swa_decode_noalloc(int nseq, int n_heads, int n_kv_heads, int head_dim, int window, float rope_base,
                                      samba_dtype io, const void *q, const void *k, const void *v, const int32_t *pos,
                                      void *k_cache, void *v_cache, void *out, void *stream);

/* Size in bytes of the device array samba_swa_decode_noalloc uses. */
size_t samba_swa_decode_noalloc_max_bytes(void);

/* Fills the ring-buffer caches from a prefill's keys and values (fixed length when
 * cu_seqlens is NULL, else packed as for samba_scan_varlen): each sequence's last
 * min(L, window + 1) tokens go to entry position mod (window + 1), keys rotated, so that a
 * following samba_swa_decode with pos = L continues the sequence. */
samba_status samba_swa_kv_fill(int nseq, const int32_t *cu_seqlens, int seqlen, int total_tokens, int n_kv_heads,
                               int head_dim, int window, float rope_base, samba_dtype io, const void *k,
                               const void *v, void *k_cache, void *v_cache, void *stream);

/* Epilogue of samba_gemm. */
typedef enum {
    SAMBA_GEMM_STORE = 0,  /* out bf16 = A . W^T */
    SAMBA_GEMM_ADD_F32 = 1, /* out fp32 = residual fp32 + A . W^T (the residual stream) */
    SAMBA_GEMM_SWIGLU = 2, /* W = [W1; W2] (2N rows): out bf16 = (A . W1^T) * SiLU(A . W2^T) */
    SAMBA_GEMM_FORCE_INT32 = -2147483647 - 1
} samba_gemm_epilogue;

/* Size in bytes of the workspace samba_gemm needs for this shape (0 when the K range is
 * not split; then workspace may be NULL). */
size_t samba_gemm_workspace_bytes(int M, int N, int K, samba_gemm_epilogue epilogue);

/* out[m][n] = epilogue(sum_k A[m][k] * W[n][k]): the linear projections of the Samba layers
 * (page "Samba: Simple Hybrid State Space Models ...": "Input Projection and Short
 * Convolution" H = X W_in, the low-rank Delta projection U W_r W_q, B = U W_b, C = U W_c,
 * the gate X W_g and output projection W_out of "Gated Output", the attention projections,
 * and "SwiGLU Formulation" (X W1) * SiLU(X W2) followed by W3), with fp32 accumulation.
 *   A   bf16 [M][lda] (rows of K used; lda >= K, lda % 8 == 0)
 *   W   bf16 [N][K] (one row per output feature: the transpose of a d_in x d_out matrix);
 *       SWIGLU: [2N][K], rows 0..N-1 = W1^T, rows N..2N-1 = W2^T
 *   out bf16 [M][ldo] (STORE, SWIGLU) or fp32 [M][ldo] (ADD_F32), ldo >= N
 *   residual fp32 [M][ldr] (ADD_F32 only; may be exactly out with ldr == ldo -- the
 *       residual stream updated in place -- but must not partially overlap it)
 *   K % 8 == 0 (16-byte rows; SAMBA_ERR_UNSUPPORTED otherwise); M, N, K >= 0;
 *   A and W 16-byte aligned, out and residual aligned to their element size.  workspace: samba_gemm_workspace_bytes() bytes, 256-byte
 *   aligned.  out must not overlap A, W or the workspace.  Deterministic: a split K range
 *   is summed in a fixed order. */
samba_status samba_gemm(int M, int N, int K, samba_gemm_epilogue epilogue, const void *A, int lda, const void *W,
                        void *out, int ldo, const float *residual, int ldr, void *workspace, size_t workspace_bytes,
                        void *stream);

/* RMSNorm of the rows of a float32 matrix (page 1, "The layer arrangement pattern": each
 * layer is preceded by RMSNorm): out[r][i] = x[r][i] / sqrt(mean_i(x[r][i]^2) + eps) * weight[i].
 *   x fp32 [rows][d], weight fp32 [d], out bf16 [rows][d]; eps >= 0.  out must not overlap x. */
samba_status samba_rmsnorm(int rows, int d, const float *x, const float *weight, float eps, void *out, void *stream);

/* Shape of a Samba model (page 1, "The Mamba Layer" parameter summary, "The Sliding Window
 * Attention (SWA) Layer", "The SwiGLU MLP Layer"; the 1.7B configuration is d_model 2048,
 * d_inner 4096, dt_rank 128, d_state 16, d_ff 8196 (stored as 8200), 32 query heads,
 * 4 KV heads, head_dim 64, window 2048, RoPE base 10000). */
typedef struct {
    int d_model;     /* d_m */
    int d_inner;     /* d_e = 2 d_m */
    int d_state;     /* d_s = 16 */
    int dt_rank;     /* d_r = d_m / 16, rank of the Delta projection */
    int d_ff;        /* MLP width as stored: d_p rounded up to a multiple of 8; the extra W1/W2
                      * rows and W3 columns must be zero (the result is then exactly that of d_p) */
    int n_heads;     /* query heads */
    int n_kv_heads;
    int head_dim;    /* 64 or 128 */
    int window;      /* sliding window w */
    float rope_base;
    float norm_eps;  /* RMSNorm epsilon */
} samba_model_config;

typedef enum {
    SAMBA_LAYER_MAMBA = 0,
    SAMBA_LAYER_SWA = 1,
    SAMBA_LAYER_MLP = 2,
    SAMBA_LAYER_FORCE_INT32 = -2147483647 - 1
} samba_layer_kind;

/* One layer of the stack: its kind, its RMSNorm weight, its weights (bf16, one row per output
 * feature, the projections that read the same input stacked into one matrix) and its decode
 * state (device memory updated in place by samba_decode_step).  Only the fields of the
 * layer's kind are read.
 * MAMBA ("The Mamba Layer"): H = X W_in, gate X W_g, U = SiLU(conv(H)), Delta from U W_r W_q
 *   + b, B = U W_b, C = U W_c, output (Y * SiLU(X W_g)) W_out:
 *   w_in_gate [2 d_inner][d_model] = [W_in^T; W_g^T];
 *   w_xproj [dt_rank + 2 d_state][d_inner] = [W_r^T; W_b^T; W_c^T];
 *   w_dt_up (W_q^T) [d_inner][dt_rank]; w_out [d_model][d_inner];
 *   ssm: A, D, dt_bias (b), conv_w, conv_b as for samba_scan_prefill;
 *   h [nseq][d_inner][d_state] fp32 and conv_state [nseq][3][d_inner] bf16, a ring whose
 *   head is samba_decode_step's conv_head (as conv_ring / ring_head_in of samba_scan_decode).
 * SWA ("The Sliding Window Attention (SWA) Layer"): w_qkv [(n_heads + 2 n_kv_heads) head_dim]
 *   [d_model] = [W_q^T; W_k^T; W_v^T]; w_o [d_model][n_heads head_dim]; k_cache, v_cache
 *   [nseq][n_kv_heads][window + 1][head_dim] ring buffers as for samba_swa_decode.
 * MLP ("SwiGLU Formulation"): w12 [2 d_ff][d_model] = [W1^T; W2^T]; w3 [d_model][d_ff]. */
typedef struct {
    int kind;
    const float *norm_w;
    const void *w_in_gate, *w_xproj, *w_dt_up, *w_out;
    samba_params ssm;
    float *h;
    void *conv_state;
    const void *w_qkv, *w_o;
    void *k_cache, *v_cache;
    const void *w12, *w3;
} samba_layer;

/* Workspace samba_decode_step needs for nseq sequences (intermediate activations and the
 * partial sums of the projections). */
size_t samba_decode_step_workspace_bytes(const samba_model_config *cfg, int nseq);

/* One generation step of a whole Samba stack for nseq sequences (one new token each):
 * for every layer, hidden += Layer(RMSNorm(hidden)) ("The layer arrangement pattern", with
 * the Mamba, SWA and MLP layers as defined on page 1), then out = RMSNorm(hidden) with
 * final_norm_w, and pos += 1 for every pos >= 0.
 *   layers     HOST array [n_layers] (the pointers in it are device pointers)
 *   hidden     fp32 [nseq][d_model] IN: the new tokens' embeddings; OUT: the residual stream
 *              after the last layer
 *   out        bf16 [nseq][d_model] or NULL (then final_norm_w is not read)
 *   pos        DEVICE int32 [nseq] IN/OUT: the new tokens' positions (SWA layers); a
 *              sequence with pos < 0 gets no attention output and keeps its position
 *   conv_head  DEVICE int32 [nseq] IN/OUT: the head of every Mamba layer's conv ring (the
 *              layers advance together); set to (head + 1) mod 3 for every sequence after the
 *              last layer.  May be NULL only when no layer is a Mamba layer.
 *   workspace  samba_decode_step_workspace_bytes(cfg, nseq) bytes, 256-byte aligned
 * d_model, d_inner, dt_rank and d_ff must be multiples of 8, d_state 16, nseq <= 65535.  Every
 * launch goes to `stream`
 * and the call allocates nothing, so the whole step can be captured into a HIP graph. */
samba_status samba_decode_step(const samba_model_config *cfg, int n_layers, const samba_layer *layers,
                               const float *final_norm_w, int nseq, float *hidden, void *out, int32_t *pos,
                               int32_t *conv_head, void *workspace, size_t workspace_bytes, void *stream);

/* Message describing the last failing call on this thread ("" if none).  The pointer
 * stays valid until the next call into the library on the same thread. */
const char *samba_last_error(void);

/* Library version string. */
const char *samba_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SAMBA_SCAN_H */
