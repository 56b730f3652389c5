/*
 * idattn.h - C ABI of the Interdomain Attention token mixer on AMD MI355X
 * (gfx950).  One shared library, libidattn.so; every entry point is plain C
 * with plain pointers and sizes.
 *
 * The method (arXiv 2605.24330, "Interdomain Attention: Beyond Token-Level
 * Key-Value Memory"; gist.science German summary, "Skalierbare
 * Implementierung", all four bullets; Chinese rendering of the paper, Fig. 1
 * caption for the state shapes):
 *   per batch row b, head h, position i, with R = d channels per head,
 *   c   = SC(x), a causal depthwise conv of width W, on q and on k
 *   xi  = SiLU(c) / (||SiLU(c)||^2 + eps_feat)             (norm over R; or,
 *         with IDATTN_FEATURE_UNIT, SiLU(c) / sqrt(||SiLU(c)||^2 + eps_feat);
 *         or, with IDATTN_FEATURE_RFF, [cos(Omega^T c), sin(Omega^T c)]/sqrt(d/2))
 *   z_k = g_k * xi_k / sqrt(mean(xi_k^2) + eps_norm) + b_k  (RMSNorm, key half)
 *   z_v = g_v * v    / sqrt(mean(v^2)    + eps_norm) + b_v  (RMSNorm, value half)
 *   abar_m = exp(Delta lambda_m), bbar_m = (abar_m - 1)/lambda_m * B_m,
 *   Delta = exp(log_dt_h)                                   (ZOH of S4D)
 *   U_m(i)     = abar_m U_m(i-1)     + bbar_m z_k(i)         (M x R complex)
 *   Gamma_m(i) = abar_m Gamma_m(i-1) + bbar_m z_v(i)         (M x d complex)
 *   s_m(i) = xi_q(i) . U_m(i)                                (row of F_q U^T)
 *   o_i    = Re sum_m s_m(i) Gamma_m(i)                      (F_q U^T Gamma,
 *                                                             no denominator)
 * Products are plain bilinear (no conjugation).  Tap W-1 of the conv
 * multiplies the current token; history before the first token is zero or
 * the caller's tail.
 *
 * Common rules for every entry point:
 *  - Ownership: every buffer is owned by the caller.  Device pointers must be
 *    device memory of the current HIP device, 16-byte aligned (else
 *    IDATTN_ERR_ARG).  The library never allocates, frees, synchronises, or
 *    changes the current device.
 *  - Streams: all device work is enqueued on `stream` (a hipStream_t passed as
 *    void*; NULL = the null stream).  Calls return after enqueueing.
 *  - Errors: every argument error is detected and returned before any HIP
 *    call is made, so validation works on a host without a GPU.  A failed
 *    kernel launch returns IDATTN_ERR_HIP.  Device faults surface at the
 *    caller's next synchronisation.  No C++ exception crosses the ABI.
 *    idattn_last_error() gives a thread-local text for the last failure.
 *  - NaN and Inf in the inputs propagate; they are not checked.
 *  - lambda must have a negative real part for a bounded state; this is not
 *    checked (the values live in device memory).
 *  - Results are bitwise reproducible for equal inputs and dims: no float
 *    atomics.
 */
#ifndef IDATTN_H
#define IDATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum idattn_status {
    IDATTN_OK = 0,
    IDATTN_ERR_NULL = 1,         /* a required pointer is NULL                  */
    IDATTN_ERR_SHAPE = 2,        /* a size is out of range or inconsistent      */
    IDATTN_ERR_UNSUPPORTED = 3,  /* a valid size this library has no kernel for */
    IDATTN_ERR_WORKSPACE = 4,    /* workspace missing or too small              */
    IDATTN_ERR_ALIAS = 5,        /* buffers overlap in a way that is not allowed */
    IDATTN_ERR_ARG = 6,          /* an enum or epsilon value is invalid          */
    IDATTN_ERR_HIP = 7           /* the HIP runtime reported an error            */
} idattn_status;

typedef enum idattn_io_dtype {
    IDATTN_IO_F32 = 0,   /* q, k, v, o and tails in float32  */
    IDATTN_IO_BF16 = 1   /* q, k, v, o and tails in bfloat16 */
} idattn_io_dtype;

typedef enum idattn_algo {
    IDATTN_ALGO_AUTO = 0,        /* CHUNKED for bf16 I/O, SEQUENTIAL for f32 I/O          */
    IDATTN_ALGO_SEQUENTIAL = 1,  /* fp32 recurrence, one time step after another         */
    IDATTN_ALGO_CHUNKED = 2      /* chunked parallel-in-time scan, fp16 MFMA operands,
                                    fp32 accumulation and state; bf16 I/O only           */
} idattn_algo;

/* The feature map xi applied to the conv outputs c of queries and keys
 * (y = SiLU(c)).  The gist.science summaries print the squared norm; the
 * Chinese rendering, section 1, names the feature map "SiLU/l_2", whose plain
 * reading is the unit-norm map.  Its section 3.1 (eqs. 5 and 6) gives random
 * Fourier features of a stationary kernel: here D = d/2 frequencies per head,
 * the columns of Omega_h = params->rff_omega[h], shared by queries and keys,
 * with the cosine half first and a 1/sqrt(D) factor so that xi(x) . xi(x') is
 * the mean of cos(w^T (x - x')) over the D frequencies.  The caller draws the
 * frequencies; eps_feat is unused with it.  The chunked algorithm computes
 * these features in a pre-pass (phases on the matrix cores in split fp16,
 * features stored in fp16 in the workspace) for dense batches; packed
 * batches with it run the sequential algorithm. */
typedef enum idattn_feature_norm {
    IDATTN_FEATURE_SQUARED = 0,  /* xi = y / (||y||^2 + eps_feat)        (default) */
    IDATTN_FEATURE_UNIT = 1,     /* xi = y / sqrt(||y||^2 + eps_feat)              */
    IDATTN_FEATURE_RFF = 2       /* xi = [cos(Omega^T c), sin(Omega^T c)] / sqrt(d/2) */
} idattn_feature_norm;

/* Sizes.  R == d.  Layout of q, k, v, o: contiguous [B][N][H][d]. */
typedef struct idattn_dims {
    int64_t B;        /* batch rows, >= 1                                     */
    int64_t N;        /* tokens per sequence, >= 0 (forward), 1..8 (decode);
                         all tokens T of a packed batch (varlen)           */
    int64_t H;        /* heads, >= 1                                          */
    int64_t d;        /* channels per head (= R); supported 16, 32, 64, 128   */
    int64_t M;        /* complex modes per head; supported 16, 32, 64         */
    int64_t W;        /* short-conv width; supported 1..8                     */
    int32_t io_dtype; /* idattn_io_dtype                                      */
    int32_t algo;     /* idattn_algo                                          */
    float eps_feat;   /* >= 0: xi = y / (||y||^2 + eps_feat)                   */
    float eps_norm;   /* >= 0: RMSNorm sqrt(mean(x^2) + eps_norm)              */
    int32_t feature_norm; /* idattn_feature_norm; 0 (zero-initialised) = squared */
} idattn_dims;

/* Per-head parameters, all float32 device buffers, read only. */
typedef struct idattn_params {
    const float *conv_q;  /* [H][d][W]; tap W-1 multiplies the current token */
    const float *conv_k;  /* [H][d][W]                                        */
    const float *gain;    /* [H][2d]: key-feature half, then value half       */
    const float *bias;    /* [H][2d]: key-feature half, then value half       */
    const float *log_dt;  /* [H]: Delta_h = exp(log_dt[h])                    */
    const float *A;       /* [H][M][2]: lambda (re, im), Re < 0               */
    const float *Bc;      /* [H][M][2]: B (re, im)                            */
    const float *rff_omega; /* [H][d][d/2]: Omega_h, column f = frequency w_f;
                               read only with IDATTN_FEATURE_RFF (then
                               non-NULL), else ignored and may be NULL        */
} idattn_params;

/*
 * Carried state (the method's fixed-size memory; the Chinese rendering, Fig. 1
 * caption, gives U as M x R and Gamma as M x d):
 *   state: float32 [B][H][M][2d][2] = complex64 [B][H][M][2d] interleaved
 *          (re, im); columns 0..d-1 hold U_m, columns d..2d-1 hold Gamma_m.
 *   tail:  io dtype [B][H][2][W-1][d]: the last W-1 raw (pre-conv) q tokens,
 *          then the last W-1 raw k tokens, oldest first.
 */

/* Bytes of device workspace idattn_forward needs for these dims (0 is
 * possible).  Returns IDATTN_OK and sets *bytes, or an argument error. */
idattn_status idattn_forward_workspace_size(const idattn_dims *dims, size_t *bytes);

/*
 * Forward pass over N tokens of every batch row (the scalable layer of the
 * gist.science summaries, "Skalierbare Implementierung": feature map, input
 * RMSNorm, S4D recurrence on [xi(k), v], denominator-free readout).
 *
 *  q, k, v   in   [B][N][H][d] io dtype
 *  o         out  [B][N][H][d] io dtype; must not overlap q, k, v
 *  state_in  in   NULL (zero state) or state layout above
 *  tail_in   in   NULL (zero conv history) or tail layout above
 *  state_out out  NULL or state layout; may equal state_in exactly (in place)
 *  tail_out  out  NULL or tail layout; may equal tail_in exactly (in place)
 *  workspace      device memory of at least idattn_forward_workspace_size bytes
 *  stream         hipStream_t as void*
 * N == 0 is allowed: o is not touched; state_out/tail_out receive state_in/
 * tail_in (or zeros).  Any partial overlap among the buffers is rejected.
 */
idattn_status idattn_forward(const idattn_dims *dims, const idattn_params *params,
                             const void *q, const void *k, const void *v, void *o,
                             const float *state_in, const void *tail_in,
                             float *state_out, void *tail_out,
                             void *workspace, size_t workspace_bytes, void *stream);

/*
 * idattn_forward for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * The same kernels and the same result as idattn_forward, with the workspace
 * taken from the library's own scratch array instead of the caller's:
 * IDATTN_NOALLOC_SCRATCH_BYTES of device memory that each GPU the library runs
 * on holds from the first use of the library on that device until the
 * process ends.  The call allocates and frees nothing.
 *
 *  arguments as for idattn_forward, without workspace and workspace_bytes.
 * Dims whose workspace (idattn_forward_workspace_size) exceeds
 * IDATTN_NOALLOC_SCRATCH_BYTES return IDATTN_ERR_WORKSPACE before any HIP
 * call; 192 MiB covers the chunked forward of B=8 H=12 N=4096 d=64,
 * B=4 H=16 N=4096 d=128 and B=1 H=16 N=14336 d=128.  Every call on one GPU
 * shares that GPU's array: calls that overlap in time on one GPU (other
 * streams, other threads) race and give wrong results.  Nothing needs
 * clearing between calls: each call writes every scratch byte it reads.
 */
#define IDATTN_NOALLOC_SCRATCH_BYTES ((size_t)192 << 20)

idattn_status idattn_forward_noalloc(const idattn_dims *dims, const idattn_params *params,
                                     const void *q, const void *k, const void *v, void *o,
                                     const float *state_in, const void *tail_in,
                                     float *state_out, void *tail_out, void *stream);

/*
 * Forward with the normalised readout of the derivation (German summary,
 * "Theoretische Herleitung"; Chinese rendering, Fig. 1: a third in-loop state
 * eta, M x 1, and the readout F_q U^T Gamma / (F_q U^T eta)), which the
 * scalable layer drops.  eta is the S4D response to a constant input of one,
 * with the same abar and bbar as the other channels:
 *   eta_m(i) = abar_m eta_m(i-1) + bbar_m,
 *   o_i = Re sum_m s_m(i) Gamma_m(i) / Re sum_m s_m(i) eta_m(i)
 * (no epsilon: a zero denominator gives Inf or NaN, passed through).
 *
 *  eta_in   in   NULL (zeros) or float32 [B][H][M][2] (complex, re, im)
 *  eta_out  out  NULL or [B][H][M][2]; may equal eta_in exactly (in place)
 *  all other arguments as for idattn_forward; the workspace is
 *  idattn_forward_normalized_workspace_size bytes.
 * dims->algo: AUTO takes the chunked algorithm wherever idattn_forward has it
 * (bf16, d in {64, 128}, M = 64, W <= 4), else the
 * sequential one; CHUNKED elsewhere returns IDATTN_ERR_UNSUPPORTED.  The
 * chunked algorithm forms the denominator in fp32 from the mode scores before
 * their fp16 rounding and eta in closed form (fp64), so eta_out is exact to
 * fp32 rounding.  One token per call from a carried state, tail and eta is
 * the decode step of this readout.
 */
idattn_status idattn_forward_normalized_workspace_size(const idattn_dims *dims, size_t *bytes);

idattn_status idattn_forward_normalized(const idattn_dims *dims, const idattn_params *params,
                                        const void *q, const void *k, const void *v, void *o,
                                        const float *state_in, const void *tail_in, const float *eta_in,
                                        float *state_out, void *tail_out, float *eta_out,
                                        void *workspace, size_t workspace_bytes, void *stream);

/*
 * Packed variable-length batch: dims->B sequences of different lengths laid
 * end to end on one token axis of dims->N = T tokens, each sequence
 * independent of the others with its own state and conv tail.  The
 * fixed-size state per sequence (Chinese rendering, section 1) is what makes
 * prompts of mixed lengths one call.  Same result, sequence by sequence, as
 * idattn_forward with B = 1 on that sequence's tokens.
 *
 *  cu_seqlens      in  device int32 [B + 1], 4-byte aligned, non-NULL:
 *                      sequence b is tokens cu_seqlens[b] .. cu_seqlens[b+1]-1;
 *                      it must rise from 0 to T (zero-length sequences
 *                      allowed).  Not checked on the host (device memory):
 *                      the sequential kernels clamp every bound into [0, T],
 *                      and the chunked path checks the table on the device
 *                      and runs nothing for a malformed one (outputs left
 *                      unwritten); either way a malformed table gives wrong
 *                      results but no access out of bounds.
 *  cu_seqlens_host in  NULL or the same table in host memory, checked (it must
 *                      rise from 0 to T, else IDATTN_ERR_SHAPE); the
 *                      algorithms do not need it.
 *  AUTO and CHUNKED run the chunked algorithm where it has a kernel (bf16,
 *  d in {64, 128}, M = 64, W <= 4, not the RFF map, B H <= 2^22): one launch
 *  sequence for the whole batch, whose plan (segments per sequence, chosen
 *  so that the segments spread over the compute units) is built on the
 *  device from cu_seqlens, so the call never waits on the device.
 *  q, k, v    in   [T][H][d] io dtype
 *  o          out  [T][H][d] io dtype
 *  state_in, tail_in, state_out, tail_out  as for idattn_forward, with B
 *                  sequences ([B][H][M][2d][2] and [B][H][2][W-1][d])
 *  workspace       at least idattn_forward_varlen_workspace_size bytes (enough
 *                  for either algorithm unless dims->algo is SEQUENTIAL)
 * T < 2^31.  CHUNKED without a kernel for these dims returns
 * IDATTN_ERR_UNSUPPORTED.  The workspace size depends on B, H and T only.
 * Overlap rules as for idattn_forward; cu_seqlens must not overlap any
 * output.
 */
idattn_status idattn_forward_varlen_workspace_size(const idattn_dims *dims, size_t *bytes);

idattn_status idattn_forward_varlen(const idattn_dims *dims, const idattn_params *params,
                                    const int32_t *cu_seqlens, const int32_t *cu_seqlens_host,
                                    const void *q, const void *k, const void *v, void *o,
                                    const float *state_in, const void *tail_in,
                                    float *state_out, void *tail_out,
                                    void *workspace, size_t workspace_bytes, void *stream);

/*
 * Autoregressive steps for every batch row (O(1) work and a fixed-size
 * state per token: Chinese rendering, section 1; German summary,
 * "Problemstellung"): N = dims->N new tokens per sequence, 1 <= N <= 8
 * (IDATTN_ERR_UNSUPPORTED above), the same result as idattn_forward over
 * those N tokens from the carried state and tail.  The state is streamed
 * through once per call whatever N is, so several tokens per call cost
 * little more than one.
 *
 *  q_t, k_t, v_t in  [B][N][H][d] io dtype ([B][H][d] for N = 1)
 *  o_t          out  [B][N][H][d] io dtype
 *  state     in/out  state layout, updated in place
 *  tail      in/out  tail layout, shifted in place by N tokens
 * No workspace.  o_t must not overlap any other buffer.
 */
idattn_status idattn_decode_step(const idattn_dims *dims, const idattn_params *params,
                                 const void *q_t, const void *k_t, const void *v_t, void *o_t,
                                 float *state, void *tail, void *stream);

/*
 * Decode steps with the normalised readout (see idattn_forward_normalized):
 * the same result as idattn_forward_normalized over these 1..8 tokens from
 * the carried state, tail and eta.
 *  eta  in/out  float32 [B][H][M][2] (complex), updated in place; non-NULL
 * Other arguments and rules as for idattn_decode_step.
 */
idattn_status idattn_decode_step_normalized(const idattn_dims *dims, const idattn_params *params,
                                            const void *q_t, const void *k_t, const void *v_t, void *o_t,
                                            float *state, void *tail, float *eta, void *stream);

/* Gradient outputs for the parameters, float32 device buffers laid out like
 * the matching fields of idattn_params (complex ones as (d/dRe, d/dIm)). */
typedef struct idattn_param_grads {
    float *conv_q;  /* [H][d][W] */
    float *conv_k;  /* [H][d][W] */
    float *gain;    /* [H][2d]   */
    float *bias;    /* [H][2d]   */
    float *log_dt;  /* [H]       */
    float *A;       /* [H][M][2] */
    float *Bc;      /* [H][M][2] */
} idattn_param_grads;

/* Bytes of device workspace idattn_backward needs for these dims. */
idattn_status idattn_backward_workspace_size(const idattn_dims *dims, size_t *bytes);

/*
 * Backward pass of idattn_forward: the gradients of
 *   L = sum(grad_o * o) + Re sum(conj(grad_state) * state_out)
 * with respect to q, k, v, every parameter and state_in, for the forward
 * over the same q, k, v, params, state_in and tail_in.  The layer is trained
 * inside language models (Chinese rendering, abstract and section 1; German
 * summary, "Skalierbare Implementierung"); the pages print no backward pass,
 * so these are the exact derivatives of the forward as this library reads
 * it.  Complex gradients are d/dRe + i d/dIm.  All arithmetic is fp32, one
 * time step after another (the sequential algorithm); the forward's
 * quantities are recomputed, not stored.  Feature maps SQUARED and UNIT
 * (RFF: IDATTN_ERR_UNSUPPORTED); dims->algo AUTO or SEQUENTIAL (CHUNKED:
 * IDATTN_ERR_UNSUPPORTED); dense batches only.  No gradient is returned for
 * tail_in.
 *
 *  q, k, v      in   [B][N][H][d] io dtype (the forward's inputs)
 *  state_in     in   NULL (zero state) or the state layout
 *  tail_in      in   NULL (zero history) or the tail layout
 *  grad_o       in   [B][N][H][d] io dtype
 *  grad_state   in   NULL (no loss on state_out) or the state layout
 *  grad_q, grad_k, grad_v  out  [B][N][H][d] io dtype
 *  grad_params  out  every field non-NULL; overwritten (not accumulated)
 *  grad_state_in out NULL or the state layout
 *  workspace    at least idattn_backward_workspace_size bytes
 * Results are bitwise reproducible: parameter gradients are summed over
 * batch rows and tokens in a fixed order.  No output may overlap another
 * buffer; N == 0 gives grad_state_in = grad_state (or zeros) and zero
 * parameter gradients.
 */
idattn_status idattn_backward(const idattn_dims *dims, const idattn_params *params,
                              const void *q, const void *k, const void *v,
                              const float *state_in, const void *tail_in,
                              const void *grad_o, const float *grad_state,
                              void *grad_q, void *grad_k, void *grad_v,
                              const idattn_param_grads *grad_params, float *grad_state_in,
                              void *workspace, size_t workspace_bytes, void *stream);

/* Static text for a status code ("IDATTN_OK", ...). */
const char *idattn_status_string(idattn_status status);

/* Thread-local detail of the last non-OK status returned on this thread. */
const char *idattn_last_error(void);

/* ABI version: major * 10000 + minor * 100 + patch. */
int idattn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* IDATTN_H */
