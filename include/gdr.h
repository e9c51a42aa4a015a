/*
 * gdr.h -- C ABI of the chunked gated delta-rule backward for AMD MI355X (gfx950).
 *
 * The op.  Per sequence n and head h, with Dv x Dk state S and tokens t:
 *   qn = q / sqrt(|q|^2 + 1e-6), kn likewise, beta = sigmoid(b),
 *   lambda_t = g_t                                   (GDR_GATE_SCALAR, GDN)
 *   lambda_t = -exp(A_log[h]) * softplus(g_t + dt_bias[h])  (GDR_GATE_CHANNEL, KDA)
 *   lambda_t = gate_scale * sigmoid(exp(A_log[h]) * (g_t + dt_bias[h]))
 *                                        (GDR_GATE_CHANNEL_SIGMOID, the bounded KDA
 *                                         gate of the FlashKDA K1 page, section 5.2)
 *   S_t = S_{t-1} Diag(exp(lambda_t)) (I - beta_t kn_t kn_t^T) + beta_t v_t kn_t^T,
 *   o_t = scale * S_t qn_t,  S_0 = h0 (or 0).
 * The backward returns the gradients of L = sum_t <dO_t, o_t> + <dht, S_T> with
 * respect to q, k, v, g, the beta logit, h0, A_log and dt_bias.
 *
 * Citations (the pages describing the method):
 *  - FlashQLA GDN backward overview (lqnn.cn/news/272630), section 1: entry
 *    conventions -- dh0 returned in fp32 while dq/dk/dv are stored in bf16,
 *    dht optional (absent = zero); section 2: the state gradient recursion runs
 *    strictly from the last chunk to the first; section 3: the recursion
 *    dh <- g_last*dh + R^T dO + X^T Y with X = A_beta K.
 *  - FlashKDA backward "K1" page (yuyanqi.com), listing and sections 1-6: the
 *    prepare stage (L2-norm backward, reverse cumsum of the gate gradient plus
 *    the chunk-total term, gate backward, per-head parameter sums by atomics,
 *    beta-logit backward, tail-row masking).
 *
 * Memory and streams.  Every pointer is caller-owned.  Token tensors are
 * row-major [B, T, H, D] (dense) or [1, T_total, H, D] (varlen, B == 1 and
 * T == T_total); per-token scalars are [B, T, H]; states are [N, H, Dv, Dk]
 * fp32.  Device pointers must be 16-byte aligned.  The library never allocates,
 * frees or synchronises, and reads no host memory after a call returns: all
 * work is enqueued on `stream` (a hipStream_t; NULL = the null stream) as kernel
 * launches -- the chunk and sequence tables are written into the workspace by a
 * kernel that receives the sequence lengths as launch arguments -- so a call
 * can be recorded into a HIP graph.  The workspace carries state from
 * gdr_fwd_recompute to gdr_bwd; its layout is internal (gdr_workspace_region
 * exposes it for tests).  Outputs are overwritten, never accumulated.
 *
 * Errors.  All argument checks run before anything is enqueued; a non-OK status
 * means nothing was launched, except GDR_EHIP (a HIP call failed while
 * enqueueing).  gdr_last_error() returns a thread-local message for the last
 * non-OK status of the calling thread.
 */
#ifndef GDR_H_
#define GDR_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  GDR_OK = 0,
  GDR_EINVAL = 1,        /* bad argument: null/misaligned pointer, bad cu_seqlens, gate/param mismatch */
  GDR_EUNSUPPORTED = 2,  /* Dk != Dv, D not in {64, 128}, or a size beyond the int32 index range */
  GDR_EWORKSPACE = 3,    /* workspace smaller than gdr_workspace_bytes() */
  GDR_EHIP = 4           /* a HIP runtime call failed while enqueueing */
} gdr_status;

typedef enum { GDR_GATE_SCALAR = 0, GDR_GATE_CHANNEL = 1, GDR_GATE_CHANNEL_SIGMOID = 2 } gdr_gate;
typedef enum { GDR_BF16 = 0, GDR_F32 = 1 } gdr_dtype;

typedef struct {
  int32_t B, T, H, Dk, Dv;          /* dense: [B,T,H,D]; varlen: B == 1, T == total tokens */
  int32_t N;                        /* sequences: == B when dense, == len(cu_seqlens) - 1 when varlen */
  const int64_t* cu_seqlens_host;   /* host array [N+1], non-decreasing, [0] == 0, [N] == T; NULL = dense.
                                       Read during the call only. */
  int32_t gate;                     /* gdr_gate */
  int32_t dtype;                    /* gdr_dtype of q, k, v, g, b, dO and of dq, dk, dv, dg, dbeta */
  float scale;                      /* readout scale (usually 1/sqrt(Dk)) */
  float gate_scale;                 /* GDR_GATE_CHANNEL_SIGMOID: the bound of the per-token log decay,
                                       finite and <= 0 (natural log: the pages' log2-unit bound times
                                       ln 2); ignored otherwise */
  int32_t Hk;                       /* heads of q and k (grouped heads): 0 means H; else H % Hk == 0 and
                                       value head h reads key head h / (H / Hk), and dq, dk sum over the
                                       H / Hk value heads of each key head (FlashQLA GDN overview,
                                       section 4: hk and hv head counts, GQA tests).  Hk < H needs
                                       workspace for the per-value-head dq, dk before that sum. */
  int32_t seq_split;                /* segments per sequence for the two chunk recursions: 0 = chosen
                                       by the library (a split pays only when few (sequence, head)
                                       pairs leave compute units idle), 1 = never split, n >= 2 = split
                                       every sequence of two or more chunks into min(n, 16, its chunks)
                                       runs of whole chunks.  The split is exact (the chunk recursions
                                       are affine in the carried state; the FlashQLA overview's section
                                       3 splits them across devices with a warm-up approximation
                                       instead): each segment runs from a zero state with its transfer
                                       product, the true boundary states are composed in order, and
                                       every segment then runs again from its true state.  Results
                                       agree with the unsplit recursion up to rounding. */
} gdr_shape;

/* Below, CHANNEL stands for either per-channel gate (GDR_GATE_CHANNEL or
 * GDR_GATE_CHANNEL_SIGMOID): both take the raw gate g, A_log and dt_bias and return
 * dg, dA_log and ddt_bias in the same shapes. */
typedef struct {                    /* device pointers; the token tensors (q, k, v, g, beta_logit) may be
                                       NULL when B * T == 0 */
  const void *q, *k;                /* [B,T,Hk,Dk] dtype (Hk = H unless grouped) */
  const void *v;                    /* [B,T,H,Dv] dtype */
  const void *g;                    /* SCALAR: [B,T,H] log decay; CHANNEL: [B,T,H,Dk] raw gate; dtype */
  const void *beta_logit;           /* [B,T,H] dtype (pre-sigmoid) */
  const float *A_log;               /* CHANNEL: [H]; SCALAR: must be NULL */
  const float *dt_bias;             /* CHANNEL: [H,Dk]; SCALAR: must be NULL */
  const float *h0;                  /* [N,H,Dv,Dk] or NULL (zero initial state) */
} gdr_inputs;

typedef struct {                    /* device pointers, all overwritten; the token gradients (dq, dk, dv,
                                       dg, dbeta) may be NULL when B * T == 0 */
  void *dq, *dk;                    /* [B,T,Hk,Dk] dtype (Hk = H unless grouped) */
  void *dv;                         /* [B,T,H,Dv] dtype */
  void *dg;                         /* SCALAR: [B,T,H]; CHANNEL: [B,T,H,Dk] (w.r.t. the raw gate); dtype */
  void *dbeta;                      /* [B,T,H] dtype, w.r.t. the logit */
  float *dh0;                       /* [N,H,Dv,Dk] or NULL (not returned) */
  float *dA_log, *ddt_bias;         /* CHANNEL: [H], [H,Dk] required; SCALAR: must be NULL */
} gdr_grads;

/* Bytes of workspace the compute calls need for this shape (host only; no
 * device work).  The workspace holds the per-chunk intermediates of the chunked
 * form: the states at chunk starts and the state gradients at chunk ends (the
 * quantities the FlashQLA overview's sections 2-3 carry between its forward
 * and backward passes), the in-chunk UT/WY inverse, the gate cumsum and the
 * chunk/sequence tables.  Returns GDR_EINVAL / GDR_EUNSUPPORTED for a bad shape. */
gdr_status gdr_workspace_bytes(const gdr_shape* shape, size_t* bytes);

/* Forward recompute: the preprocessing that precedes the backward's main
 * kernels (FlashQLA GDN backward overview, section 1: a backward call is a
 * preprocessing stage plus two main kernels, fed the in-chunk cumsum of the
 * gate; section 3: the UT/WY product X = A_beta K).  Per chunk: normalisation,
 * beta, the in-chunk gate cumsum, the UT/WY inverse
 * A = (I + StrictLower(diag(beta) (K K^T o decay)))^-1, U' = A diag(beta) V and
 * W = A diag(beta) K e^Gamma; then the serial state pass storing the state at
 * the start of every chunk and v_new = U' - W S^T.
 * Arguments: shape and inputs as above; ws / ws_bytes a device workspace of at
 * least gdr_workspace_bytes(shape) bytes, 256-byte aligned; o the forward output
 * [B,T,H,Dv] in the input dtype (o_t = scale S_t qn_t, formed chunk-parallel as
 * Qbar S_n^T + P U) or NULL to skip it; ht the final state per sequence
 * [N,H,Dv,Dk] fp32 or NULL.  Leaves what gdr_bwd needs in `ws`; every stage
 * only reads inputs and what earlier stages wrote, so the call may be repeated.
 * Errors: GDR_EINVAL (null required / misaligned pointer, bad shape, gate and
 * parameter mismatch), GDR_EUNSUPPORTED, GDR_EWORKSPACE; nothing is enqueued
 * then.  GDR_EHIP if a launch fails. */
gdr_status gdr_fwd_recompute(const gdr_shape* shape, const gdr_inputs* in, void* ws, size_t ws_bytes, void* o,
                             float* ht, void* stream);

/* The forward pass for training use: gdr_fwd_recompute with the output o
 * required (GDR_EINVAL if NULL while there are tokens).  o = scale S_t qn_t per
 * token, formed per chunk as Qbar S_n^T + P U (Qbar = scale qn e^Gamma,
 * P = scale (Qn Kn^T o decay) on and below the diagonal, U = v_new): the chunked
 * form of the read-out (FlashQLA GDN overview, section 3).  Leaves the same
 * workspace, so gdr_bwd may follow. */
gdr_status gdr_fwd(const gdr_shape* shape, const gdr_inputs* in, void* ws, size_t ws_bytes, void* o, float* ht,
                   void* stream);

/* Backward, after gdr_fwd_recompute on the same shape, inputs and workspace:
 *  - the reverse-chunk state-gradient recursion, run strictly from the last
 *    chunk to the first (FlashQLA overview, section 2; its section 3 gives the
 *    recursion dh <- g_last dh + R^T dO + X^T Y with X = A_beta K), starting
 *    from dht (NULL = zero, section 1) and returning dh0 in fp32 (section 1);
 *  - the chunk-parallel gradients of q, k, v, beta and the gate (section 2: the
 *    compute-bound main backward);
 *  - the prepare-backward of the FlashKDA K1 page: L2-norm backward (section
 *    3.3), reverse cumsum of the gate gradient plus the chunk-total term
 *    (section 5), gate-function backward and the per-head sums dA_log, ddt_bias
 *    (section 5.2), beta-logit backward (section 6), tail rows masked (section 8).
 * dO: [B,T,H,Dv] dtype, required unless there are no tokens; dht: [N,H,Dv,Dk]
 * fp32 or NULL; grads: every token gradient required (dq, dk [B,T,Hk,Dk], dv,
 * dg, dbeta in the input dtype), dh0 optional, dA_log / ddt_bias required for
 * the per-channel gates and NULL for the scalar gate.  Errors as for
 * gdr_fwd_recompute. */
gdr_status gdr_bwd(const gdr_shape* shape, const gdr_inputs* in, const void* dO, const float* dht,
                   void* ws, size_t ws_bytes, gdr_grads* grads, void* stream);

/* The whole backward in one call: the same kernels as gdr_fwd_recompute
 * followed by gdr_bwd, except that the forward state pass and the reverse
 * state-gradient recursion (which do not depend on each other) run side by
 * side in one launch.  Same results, bit for bit; ht may be NULL.  Arguments
 * and errors as gdr_fwd_recompute and gdr_bwd together. */
gdr_status gdr_fwd_bwd(const gdr_shape* shape, const gdr_inputs* in, const void* dO, const float* dht,
                       void* ws, size_t ws_bytes, gdr_grads* grads, float* ht, void* stream);

/* Workspace regions, for tests that inspect intermediates.  Layouts (NC =
 * total chunks of 64 tokens over all sequences, chunk c of sequence n numbered
 * after all chunks of sequences < n; rows past a sequence's end are padding):
 *   GDR_WS_STATE   bf16 [H][NC][Dv][Dk]  state at the start of each chunk
 *   GDR_WS_DSTATE  bf16 [H][NC][Dv][Dk]  gradient w.r.t. the state at the end of each chunk
 *   GDR_WS_U       bf16 [H][NC][Dv][64]  v_new = U' - W S^T, transposed (column v of the chunk is contiguous)
 *   GDR_WS_A       bf16 [H][NC][64][64]  the UT/WY inverse
 *   GDR_WS_GAMMA   fp32 [H][NC][64] (SCALAR) or [H][NC][64][Dk] (CHANNEL): in-chunk gate cumsum
 */
enum { GDR_WS_STATE = 0, GDR_WS_DSTATE = 1, GDR_WS_U = 2, GDR_WS_A = 3, GDR_WS_GAMMA = 4 };
gdr_status gdr_workspace_region(const gdr_shape* shape, int32_t which, size_t* offset, size_t* bytes);

/* One stage of gdr_fwd_bwd enqueued alone, for benchmarks and kernel profiles
 * (same arguments as gdr_fwd_bwd; the workspace must already hold what the
 * earlier stages leave there, e.g. after one gdr_fwd_bwd call).  Stages:
 *   GDR_STAGE_PREP        per-chunk prologue and UT/WY inverse (one launch)
 *   GDR_STAGE_CHAIN_FWD   forward state pass alone
 *   GDR_STAGE_CHAIN_BWD   reverse state-gradient recursion alone
 *   GDR_STAGE_CHAIN_BOTH  both recursions in one launch, as gdr_fwd_bwd runs them
 *   GDR_STAGE_GRADS       chunk-parallel gradients and the prepare-backward (norm,
 *                         sigmoid, gate backward); writes every per-token gradient
 *   GDR_STAGE_FINISH      the per-head reduction of dA_log, ddt_bias (CHANNEL) and the
 *                         dq, dk group sums (grouped heads); enqueues nothing for
 *                         GDR_GATE_SCALAR with Hk = H */
enum { GDR_STAGE_PREP = 0, GDR_STAGE_CHAIN_FWD = 1, GDR_STAGE_CHAIN_BWD = 2, GDR_STAGE_CHAIN_BOTH = 3,
       GDR_STAGE_GRADS = 4, GDR_STAGE_FINISH = 5 };
gdr_status gdr_run_stage(const gdr_shape* shape, const gdr_inputs* in, const void* dO, const float* dht,
                         void* ws, size_t ws_bytes, gdr_grads* grads, float* ht, int32_t stage, void* stream);

/* gdr_fwd_bwd without a caller-supplied workspace, for callers that cannot
 * allocate device memory (code being captured into a HIP graph, tight serving
 * loops, harnesses that forbid allocation).  The workspace is a device array of
 * 128 MiB (134217728 bytes) that the library holds on every GPU it runs on until
 * the process ends; the call itself allocates and
 * frees nothing.  Shapes whose gdr_workspace_bytes() exceed it are rejected with
 * GDR_EWORKSPACE before anything is enqueued.  Every call on one GPU uses that
 * GPU's single array, so calls that overlap in time on one GPU (different
 * streams, threads or processes sharing the array) race; calls in order on one
 * stream are safe.  Inputs, outputs and errors as gdr_fwd_bwd.  The first call
 * on a device looks up that device's copy of the array (hipGetSymbolAddress). */
gdr_status gdr_fwd_bwd_noalloc(const gdr_shape* shape, const gdr_inputs* in, const void* dO, const float* dht,
                               gdr_grads* grads, float* ht, void* stream);

/* Thread-local text for the last non-OK status returned to this thread. */
const char* gdr_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* GDR_H_ */
