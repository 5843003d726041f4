/*
 * gma.h -- C ABI of libgma.so, the MI355X (gfx950) forward mixer of Gaussian Mixture
 * Attention (GMA).
 *
 * Method: "Gaussian Mixture Attention: Linear-Time Sequence Mixing via Probabilistic
 * Latent Routing" (Huang, Raza; arXiv 2606.18283), gist.science summary, section "Core
 * mechanism":
 *   item 1  -- queries and keys are routed to K learned diagonal Gaussians; the
 *              responsibility gamma_{i,k} = p(z=k | x_i) is the standard GMM posterior
 *              with means mu_k, diagonal covariances Sigma_k and mixture priors pi_k,
 *              giving the non-negative maps Gamma_Q, Gamma_K (N x K);
 *   item 2  -- write phase Vt = Gamma_K^T V, Z = Gamma_K^T 1 (a K-slot latent memory),
 *              read phase O = Gamma_Q Vt / (Gamma_Q Z + eps); the N x N affinity
 *              Gamma_Q Gamma_K^T is never formed;
 *   item 3  -- bidirectional and causal variants (the causal one uses prefix sums of
 *              the memory and the normaliser so O_i depends on positions j <= i only);
 *              variances are reparameterised with softplus, priors with softmax.
 *
 * Conventions of this library (the pages leave them open):
 *   var_kd = softplus(var_raw_kd) + var_floor  (softplus acts on the variance);
 *   pi     = softmax(prior_logits) over the K components of a head;
 *   one set of K Gaussians per head, shared by the queries and keys of that head and by
 *   every batch element;
 *   eps is added once per output row after the product Gamma_Q Z;
 *   the causal sum is inclusive: O_i uses keys/values j = 0..i.
 *
 * Layouts (all row-major, contiguous, device memory):
 *   qr, kr        [B, H, N, d_r]  dtype (GMA_F32 or GMA_BF16)
 *   v, out        [B, H, N, d_v]  dtype
 *   mu, var_raw   [H, K, d_r]     float32
 *   prior_logits  [H, K]          float32
 *   gamma_out     [2, B, H, N, K] float32, optional: Gamma_Q then Gamma_K
 *
 * Ownership: the caller owns every buffer, including the workspace; the library never
 * allocates, frees or retains device memory and keeps no mutable global state.  `out`
 * and `gamma_out` must not alias any input or each other.
 *
 * Execution: every call enqueues kernels on `stream` (a hipStream_t; NULL means the
 * legacy default stream) and returns without synchronising.  Results are valid once the
 * stream has been synchronised.  Concurrent calls are safe if they use distinct
 * workspaces and outputs.
 *
 * Errors: every argument is checked on the host before any HIP call; on error nothing is
 * enqueued and a negative status is returned.  Input values are not scanned: NaN or Inf
 * in the inputs propagate.  No C++ exception crosses this interface.
 */
#ifndef GMA_H
#define GMA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GMA_VERSION 10400 /* 1.4.0: backward */

/* Limits of the library (kernel tile and LDS sizes). */
#define GMA_MAX_K 256
#define GMA_MAX_DR 128
#define GMA_MAX_DV 128

typedef enum {
    GMA_OK = 0,
    GMA_ERR_NULL_ARG = -1,    /* a required pointer is NULL                                 */
    GMA_ERR_BAD_SHAPE = -2,   /* B, H or N < 0; d_r, d_v or K < 1; element counts too large  */
    GMA_ERR_UNSUPPORTED = -3, /* K > GMA_MAX_K, d_r > GMA_MAX_DR, d_v > GMA_MAX_DV, unknown
                                 dtype or algorithm, or an algorithm that cannot run this
                                 dtype                                                        */
    GMA_ERR_ALIGN = -4,       /* qr, kr, v, out not 16-byte aligned; parameters or gamma_out
                                 not 4-byte aligned; workspace not 256-byte aligned           */
    GMA_ERR_BAD_SCALAR = -5,  /* eps or var_floor negative or not finite; causal not 0 or 1  */
    GMA_ERR_WORKSPACE = -6,   /* workspace NULL or smaller than gma_workspace_size()         */
    GMA_ERR_ALIAS = -7,       /* out or gamma_out overlaps an input or each other            */
    GMA_ERR_HIP = -8,         /* a kernel launch reported an error                           */
    GMA_ERR_TOO_LARGE = -9    /* gma_forward_noalloc: the call needs more scratch than its
                                 static buffer (GMA_NOALLOC_SCRATCH_BYTES) holds              */
} gma_status;

typedef enum { GMA_F32 = 0, GMA_BF16 = 1 } gma_dtype;

/* Kernel family.  AUTO picks MFMA where it applies and SIMT otherwise.  SIMT is the plain
 * one-thread-per-element fp32 path (any supported shape, both dtypes); MFMA is the fused
 * matrix-core path: bf16 only, d_r and d_v multiples of 8 (rows are read as 16-byte
 * vectors), and shapes whose staging fits in LDS.  An explicit GMA_ALGO_MFMA outside that
 * range gives GMA_ERR_UNSUPPORTED (and gma_workspace_size returns 0). */
typedef enum { GMA_ALGO_AUTO = 0, GMA_ALGO_SIMT = 1, GMA_ALGO_MFMA = 2 } gma_algo;

typedef struct {
    int32_t B, H, N;     /* batch, heads, sequence length (0 gives an empty call)  */
    int32_t d_r, d_v, K; /* routing dim, value dim, number of Gaussian components  */
    int32_t dtype;       /* gma_dtype of qr, kr, v and out                         */
    int32_t algo;        /* gma_algo                                               */
    float var_floor;     /* added to softplus(var_raw); >= 0 and finite            */
} gma_desc;

/*
 * Bytes of device workspace that gma_forward needs for this descriptor and variant
 * (`causal` 0 or 1).  Pure host arithmetic, no HIP call.  Returns 0 when the descriptor
 * is invalid (gma_forward then reports why) or when no workspace is needed.
 */
size_t gma_workspace_size(const gma_desc* desc, int causal);

/*
 * GMA forward (responsibilities, write, read; or the causal prefix form).
 *   qr, kr, v      inputs, layout above, dtype = desc->dtype
 *   mu, var_raw    [H,K,d_r] float32 Gaussian means and pre-softplus variances
 *   prior_logits   [H,K] float32 pre-softmax mixture weights
 *   causal         0 = bidirectional (write/read of "Core mechanism" item 2),
 *                  1 = causal prefix-sum variant (item 3)
 *   eps            normaliser floor, >= 0
 *   out            [B,H,N,d_v] output in desc->dtype (round to nearest even for bf16)
 *   gamma_out      NULL, or [2,B,H,N,K] float32 that receives Gamma_Q and Gamma_K
 *                  (diagnostic; an extra kernel, not part of the fused path)
 *   workspace      device scratch of at least gma_workspace_size(desc, causal) bytes,
 *                  256-byte aligned (may be NULL if that size is 0); contents on entry
 *                  are ignored and on return are unspecified
 *   stream         hipStream_t to enqueue on, NULL for the default stream
 * Returns GMA_OK or a negative gma_status.
 */
int gma_forward(const void* qr, const void* kr, const void* v, const float* mu,
                const float* var_raw, const float* prior_logits, int causal, float eps,
                void* out, float* gamma_out, const gma_desc* desc, void* workspace,
                size_t workspace_bytes, void* stream);

/*
 * Profiling variant of gma_forward: identical arguments and kernels, plus a pair of HIP
 * events recorded on `stream` around every kernel the call launches, so a caller can time
 * each kernel of one forward without a profiler.  `events` holds `n_events` hipEvent_t
 * handles created by the caller (hipEventCreate); kernel i is bracketed by events[2i] and
 * events[2i+1].  On return *n_kernels (if non-NULL) is the number of kernels launched and
 * names[i] (if `names` is non-NULL, room for n_events/2 entries) points to a static name of
 * kernel i.  Kernels beyond n_events/2 run unbracketed.  Nothing is synchronised; read the
 * times with hipEventElapsedTime once the stream is done.
 */
int gma_forward_timed(const void* qr, const void* kr, const void* v, const float* mu,
                      const float* var_raw, const float* prior_logits, int causal, float eps,
                      void* out, float* gamma_out, const gma_desc* desc, void* workspace,
                      size_t workspace_bytes, void* stream, void* const* events, int n_events,
                      const char** names, int* n_kernels);

/*
 * gma_forward without a workspace argument, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).  Same
 * arguments, kernels, results and status codes as gma_forward; the scratch is a static device
 * array of GMA_NOALLOC_SCRATCH_BYTES inside the library, one per GPU, held until the process
 * ends.  The call itself allocates nothing.  A call whose gma_workspace_size(desc, causal)
 * exceeds GMA_NOALLOC_SCRATCH_BYTES returns GMA_ERR_TOO_LARGE before any HIP call.  Every call
 * on one GPU shares that GPU's array: calls that can overlap on one GPU (other streams, other
 * host threads without ordering) race on it and must not be issued; calls in order on one
 * stream are safe.  The first call on a device looks up the array's device address there.
 */
#define GMA_NOALLOC_SCRATCH_BYTES (64u << 20) /* 64 MiB per GPU */

int gma_forward_noalloc(const void* qr, const void* kr, const void* v, const float* mu,
                        const float* var_raw, const float* prior_logits, int causal, float eps,
                        void* out, float* gamma_out, const gma_desc* desc, void* stream);

/*
 * Cross variant (bidirectional only): queries and keys/values of different lengths.  The
 * pages name cross-attention applications as future work (German page, closing paragraph
 * on limitations and future work); this is the plainest reading of that: the write phase
 * of "Core mechanism" item 2 over the N_k key rows, Vt = Gamma_K^T V and Z = Gamma_K^T 1,
 * and its read phase O = Gamma_Q Vt / (Gamma_Q Z + eps) for the N_q query rows, with the
 * same K Gaussians of the head for both sides.
 *   desc->N        N_q: qr [B,H,N_q,d_r], out [B,H,N_q,d_v]
 *   n_k            N_k >= 0: kr [B,H,N_k,d_r], v [B,H,N_k,d_v]
 *   gamma_out      NULL, or float32 Gamma_Q [B,H,N_q,K] followed by Gamma_K [B,H,N_k,K]
 * Every other argument, the alignment, aliasing and workspace rules and the status codes
 * are those of gma_forward (causal = 0).  N_q = 0 (or B = 0, H = 0) is a no-op.  N_k = 0 is
 * an empty memory: every output row is 0 / (0 + eps), i.e. 0 for eps > 0; kr and v are not
 * read then and may be NULL.  With n_k = N and
 * kr, v of the same positions as qr this is gma_forward(causal = 0).
 */
size_t gma_workspace_size_cross(const gma_desc* desc, int32_t n_k);

int gma_forward_cross(const void* qr, const void* kr, const void* v, const float* mu,
                      const float* var_raw, const float* prior_logits, int32_t n_k, float eps,
                      void* out, float* gamma_out, const gma_desc* desc, void* workspace,
                      size_t workspace_bytes, void* stream);

/* Profiling variant of gma_forward_cross, with the event arguments of gma_forward_timed. */
int gma_forward_cross_timed(const void* qr, const void* kr, const void* v, const float* mu,
                            const float* var_raw, const float* prior_logits, int32_t n_k, float eps,
                            void* out, float* gamma_out, const gma_desc* desc, void* workspace,
                            size_t workspace_bytes, void* stream, void* const* events, int n_events,
                            const char** names, int* n_kernels);

/*
 * Causal memory and single-token decode step: the causal variant of "Core mechanism" item
 * 3 written as a recurrence over positions (the pages give the prefix-sum form; the
 * recurrence is the same sums taken one position at a time).  The state of one (b, h)
 * after positions 0..t-1 is the float32 memory [S | z], layout [B,H,K,d_v+1]: row k holds
 * S[k][0..d_v-1] = sum_j gamma_K,j[k] v_j and, last, z[k] = sum_j gamma_K,j[k].
 *
 * gma_memory: the state after the desc->N positions of kr [B,H,N,d_r] and v [B,H,N,d_v]
 *   (a prefill; N = 0 gives zeros; B = 0 or H = 0 is a no-op).  `state` is written.
 * gma_decode_step: one position per (b, h); desc->N must be 1.  qr, kr [B,H,1,d_r],
 *   v [B,H,1,d_v]; `state` is updated in place to include this position (the causal sum
 *   is inclusive) and out [B,H,1,d_v] = gamma_Q S / (gamma_Q . z + eps): row t of the
 *   causal forward when `state` held positions 0..t-1.  One kernel launch; the
 *   workspace size is 0 (workspace may be NULL), the mixture parameters are read raw.
 * Sums over positions are in position order (memory) and per step (decode), so a prefill
 * followed by decode steps matches the causal forward to rounding, not bitwise.  The
 * other rules (alignment: tensors 16 B, parameters and state 4 B, workspace 256 B; no
 * aliasing between outputs, state and inputs; status codes) are those of gma_forward.
 */
size_t gma_memory_workspace_size(const gma_desc* desc);

int gma_memory(const void* kr, const void* v, const float* mu, const float* var_raw,
               const float* prior_logits, float* state, const gma_desc* desc, void* workspace,
               size_t workspace_bytes, void* stream);

size_t gma_decode_workspace_size(const gma_desc* desc);

int gma_decode_step(const void* qr, const void* kr, const void* v, const float* mu,
                    const float* var_raw, const float* prior_logits, float* state, float eps,
                    void* out, const gma_desc* desc, void* workspace, size_t workspace_bytes,
                    void* stream);

/*
 * The decode step on prepared parameters, for callers that decode many positions with the
 * same weights: the same step as gma_decode_step (same recurrence, state layout, update in
 * place and output), with the per-component variance transcendentals of the mixture taken
 * once instead of at every step.
 *
 * gma_decode_prepared_size: bytes of the prepared block for desc (H, K, d_r, dtype; B and N
 *   are not read); 0 for an invalid desc.
 * gma_decode_prepare: writes the prepared block from mu, var_raw [H,K,d_r] and prior_logits
 *   [H,K] (float32) and desc->var_floor.  Its content is opaque (per head: the means and the
 *   precisions 1 / (softplus(var_raw) + var_floor), float64 for float32 inputs, float32 for
 *   bf16, and the constants prior_logit - (1/2) sum log var in float64).  `prepared` is
 *   caller-owned device memory, 256-byte aligned, of at least gma_decode_prepared_size bytes,
 *   not overlapping the parameters; it stays valid until the parameters change.
 * gma_decode_step_prepared: one position per (b, h), desc->N must be 1 and desc must carry the
 *   H, K, d_r and dtype given to gma_decode_prepare (a mismatch is not detectable and gives
 *   wrong results).  qr, kr [B,H,1,d_r], v [B,H,1,d_v] (desc->dtype, 16-byte aligned); `state`
 *   float32 [B,H,K,d_v+1], updated in place; out [B,H,1,d_v].  One kernel launch, no
 *   workspace; `prepared` is only read.  Status codes as gma_decode_step.
 */
size_t gma_decode_prepared_size(const gma_desc* desc);

int gma_decode_prepare(const float* mu, const float* var_raw, const float* prior_logits,
                       void* prepared, size_t prepared_bytes, const gma_desc* desc, void* stream);

int gma_decode_step_prepared(const void* qr, const void* kr, const void* v, const void* prepared,
                             float* state, float eps, void* out, const gma_desc* desc,
                             void* stream);

/*
 * Backward of gma_forward: the pages train the mixture parameters end to end by
 * backpropagation ("Core mechanism" item 3).  Given dout = dL/dO [B,H,N,d_v] (desc->dtype),
 * writes dL/dqr, dL/dkr [B,H,N,d_r] and dL/dv [B,H,N,d_v] (desc->dtype) and, summed over the
 * batch and both sides, dL/dmu, dL/dvar_raw [H,K,d_r] and dL/dprior_logits [H,K] (float32;
 * all outputs are overwritten, not accumulated).  Same inputs, causal flag, eps and layout
 * as gma_forward; the forward is recomputed inside.  The gradients are the chain rule of the
 * forward: see the kernels' source for the formulas.  For bf16 inputs the responsibilities
 * come from the matrix-core responsibilities kernel where it covers the shape (else the SIMT
 * one), and the passes over the rows, the segment partials, dqr/dkr and the parameter sums
 * run on the matrix cores (fp32 products in the causal chunk walks, elsewhere bf16 products
 * of exact two- or three-piece bf16 splits of the fp32 operands; shapes outside the tiles
 * keep SIMT kernels); float32 inputs run SIMT kernels
 * throughout.  algo SIMT only makes bf16 inputs take their responsibilities from the SIMT
 * kernel (double logits); the other kernels are those of AUTO.  An explicit MFMA request
 * returns GMA_ERR_UNSUPPORTED.  Sums accumulate in
 * double for float32 inputs and in float for bf16 (chunk sums of the parameter gradients
 * combined in double); every sum has a fixed order, so results are deterministic.  Every
 * shape within the limits is supported, except 2 B N > INT32_MAX (the row passes index both
 * sides of a head's rows in 32 bits): GMA_ERR_UNSUPPORTED and a workspace size of 0.
 * Alignment, aliasing and status codes as gma_forward (no output may overlap an input, the
 * workspace or another output).  N = 0 gives zero parameter gradients.
 */
size_t gma_backward_workspace_size(const gma_desc* desc, int causal);

int gma_backward(const void* qr, const void* kr, const void* v, const float* mu, const float* var_raw,
                 const float* prior_logits, const void* dout, int causal, float eps, void* dqr,
                 void* dkr, void* dv, float* dmu, float* dvar_raw, float* dprior,
                 const gma_desc* desc, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Responsibility statistics of one set of routing rows: the quantities of the pages'
 * analysis of learned responsibilities (Results, interpretability: components used out of K,
 * usage entropy, hard assignments compared with token categories).  The pages name them
 * without defining them; the readings, per head h pooled over the batch and the positions:
 *   hard    int32 [B,H,N]  argmax_k gamma of row (b, h, n), the lowest k among equal maxima;
 *                          may be NULL (then kept in the workspace)
 *   counts  int32 [H,K]    number of rows whose hard assignment is k
 *   usage   float [H,K]    soft usage: sum over the rows of gamma_k
 *   used    int32 [H]      number of components with counts > 0
 *   entropy float [H]      -sum_k p_k ln p_k / ln K with p_k = counts / (B N): the usage
 *                          entropy normalised to [0, 1] (0 when K = 1 or there are no rows)
 * x [B,H,N,d_r] in desc->dtype (queries or keys; desc->d_v is not used but must be valid).
 * The argmax is taken in the precision of the path's logits (fp32 on the matrix cores for
 * bf16 inputs, double on the SIMT path), so rows whose two best components are closer than
 * that precision may differ from a higher-precision evaluation.  Deterministic: the same
 * call gives bitwise the same results.  Alignment: x 16 B, parameters and outputs 4 B,
 * workspace 256 B; outputs and the workspace may not overlap each other or the inputs.
 * N = 0 gives zero counts, usage, used and entropy; B = 0 or H = 0 is a no-op.
 */
size_t gma_stats_workspace_size(const gma_desc* desc);

int gma_resp_stats(const void* x, const float* mu, const float* var_raw, const float* prior_logits,
                   int32_t* hard, int32_t* counts, float* usage, int32_t* used, float* entropy,
                   const gma_desc* desc, void* workspace, size_t workspace_bytes, void* stream);

/* Static, NUL-terminated description of a status code. */
const char* gma_strerror(int status);

/* GMA_VERSION of the loaded library. */
int gma_version(void);

#ifdef __cplusplus
}
#endif

#endif /* GMA_H */
