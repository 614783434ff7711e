/*
 * libgdn -- chunked-prefill forward of the gated delta rule on MI355X (gfx950).
 *
 * The operation (FlashQLA announcement (Qwen), section "key problems of FLA GDN
 * chunked prefill", the four-step forward for chunk i; GDN-in-FLA notes,
 * forward Steps 1-5):
 *
 *   per sequence, per value head, per chunk of C = 64 tokens (the last chunk of a
 *   sequence may be shorter), with g_c the chunk-local cumsum of the log-gates,
 *   gamma = exp(g_c) and Gamma_ij = gamma_i / gamma_j:
 *     A  = (I + strictLower(diag(beta)(Gamma (.) K K^T)))^{-1}
 *     W  = A diag(beta) diag(gamma) K,      U = A diag(beta) V
 *     V' = U - W S
 *     S <- gamma_C S + K^T diag(gamma_C / gamma) V'        (gamma_C: last valid token)
 *     O  = scale (diag(gamma) Q S + (Lower(Gamma) (.) Q K^T) V')   (mask includes the diagonal)
 *
 *   which equals, token by token, S_t = alpha_t (I - beta_t k_t k_t^T) S_{t-1} + beta_t k_t v_t^T,
 *   o_t = scale S_t^T q_t with alpha_t = exp(g_t) and the [D_k, D_v] state layout.
 *
 *   Per-channel gates (KDA; "KDA源码剖析之FLA", sections 3-5): the log-gate is a
 *   [D_k] vector per token, the decay Diag(exp(gk_t)) is applied to the rows of S
 *   before the read and the erase.  With bf16 inputs the per-channel path multiplies
 *   fp16 operands (the gated q and k rows, the intra-chunk matrix and the inverse),
 *   which requires q and k rows of unit scale (L2-normalised, as the method has them,
 *   or normalised by the prologue's qk_l2norm): larger rows can overflow fp16.
 *   The per-channel log-gates need no lower bound: the pairwise decay factors are split
 *   at a reference row per 16-token block, and a block whose decay in some channel
 *   exceeds what the split factors can hold (2^12 for fp16 operands, 2^64 for fp32 ones)
 *   takes its pairs' factors whole (each at most 1), so no gate value yields inf or NaN.
 *
 * Tensor layouts (row-major, contiguous, device memory):
 *   q, k         [B, T, H_qk, D_k]   dtype
 *   v            [B, T, H_v,  D_v]   dtype
 *   g            [B, T, H_v]         fp32       (GDN_GATE_SCALAR, natural-log gate, <= 0 expected)
 *   g            [B, T, H_v, D_k]    dtype      (GDN_GATE_CHANNEL)
 *   beta         [B, T, H_v]         dtype
 *   o            [B, T, H_v, D_v]    o_dtype    (written)
 *   h0           [N, H_v, D_k, D_v]  fp32       (NULL: zero initial state)
 *   final_state  [N, H_v, D_k, D_v]  fp32       (NULL: not written)
 *   Value head h reads query/key head h / (H_v / H_qk).
 *   Packed variable-length input: B == 1, cu_seqlens holds N + 1 token offsets
 *   (cu[0] = 0, non-decreasing, cu[N] = T); chunks never straddle sequences.
 *
 * Ownership: the caller owns every buffer, including the workspace.  gdn_fwd
 * allocates nothing, enqueues all work on `stream` (a hipStream_t; NULL is the
 * null stream) and returns without synchronising.  Inputs must stay valid and
 * outputs untouched until the enqueued work completes.
 *
 * Errors: all validation happens before any launch; on an error nothing is
 * enqueued and no output is touched.  Faults inside kernels surface at the
 * caller's next synchronisation, as for any HIP launch.
 */
#ifndef GDN_H_
#define GDN_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    GDN_OK = 0,
    GDN_ERR_INVALID_ARG = 1,  /* null required pointer, bad size, bad cu_seqlens, ... */
    GDN_ERR_UNSUPPORTED = 2,  /* valid but not implemented (chunk size, head dim, dtype mix) */
    GDN_ERR_WORKSPACE = 3,    /* workspace NULL or smaller than gdn_fwd_workspace_bytes() */
    GDN_ERR_HIP = 4           /* a HIP launch or query failed */
} gdn_status;

typedef enum { GDN_DTYPE_F32 = 0, GDN_DTYPE_BF16 = 1 } gdn_dtype;
typedef enum { GDN_GATE_SCALAR = 0, GDN_GATE_CHANNEL = 1 } gdn_gate_kind;

/* Context parallelism inside one GPU (FlashQLA announcement, the in-GPU CP
 * pre-process and fix-up): split each sequence into segments of L chunks, run
 * every segment from S = 0 together with its transition matrix M, fix up the
 * segment start states serially, then run all segments in parallel. */
/* GDN_CP_WARMUP (FlashQLA announcement, section "further optimisation through gate decay"): the
 * same segments, but a segment after a sequence's first starts W chunks early from S = 0 instead of
 * from the exact start state (no S*, no M, no fix-up); its warmup chunks write no output.  W is
 * chosen per (segment, value head) by a gate-statistics kernel: the fewest whole chunks right
 * before the segment whose decay bounds multiply to <= cp_warmup_tol (a chunk's bound: the product
 * of its decays; per-channel gates: of each token's largest channel decay), else the whole prefix
 * from h0 (exact).  With unit keys and 0 <= beta <= 2 the state error is at most that product
 * times the norm of the skipped state: an approximation whose error the caller bounds by choosing
 * cp_warmup_tol.  Never chosen by GDN_CP_AUTO. */
typedef enum { GDN_CP_AUTO = 0, GDN_CP_OFF = 1, GDN_CP_ON = 2, GDN_CP_WARMUP = 3 } gdn_cp_mode;

/* Form of the exact CP pre-process (FlashQLA announcement, step 2.1 of the in-GPU CP pre-process):
 * CHAIN runs the recurrence's own three products (K S, A X, K^T V'') over virtual value and
 * identity columns, a workgroup per 32 of them; XYZ forms X^T = -K^T diag(gamma_C / gamma) A
 * diag(beta) once per chunk and updates S* and M with two products (K S, X^T Y), one workgroup per
 * (segment, value head); it applies to bf16 inputs with a scalar gate only (GDN_ERR_UNSUPPORTED
 * otherwise).  AUTO takes XYZ where it applies and the (segment, value head) pairs fill the device's
 * compute units, else CHAIN. */
typedef enum { GDN_CP_FORM_AUTO = 0, GDN_CP_FORM_CHAIN = 1, GDN_CP_FORM_XYZ = 2 } gdn_cp_form;

typedef struct {
    int32_t B, T;             /* batch and tokens per batch row (T = total tokens when packed) */
    int32_t H_qk, H_v;        /* query/key heads, value heads (H_v % H_qk == 0) */
    int32_t D_k, D_v;         /* head dims, each 64 or 128 (independently) */
    int32_t chunk_size;       /* 64 for gdn_fwd, 1 for gdn_fwd_recurrent */
    int32_t dtype;            /* gdn_dtype of q, k, v, beta, o (and a channel gate) */
    int32_t gate_kind;        /* gdn_gate_kind */
    float scale;              /* output scale, usually D_k^-1/2 */
    const void *q, *k, *v, *g, *beta;
    const float *h0;                  /* nullable */
    const int32_t *cu_seqlens_dev;    /* nullable; [N + 1] device copy used by the kernels */
    const int32_t *cu_seqlens_host;   /* required with cu_seqlens_dev; host copy used for planning */
    int32_t N;                        /* sequences: N == B when not packed */
    void *o;
    float *final_state;               /* nullable */
    int32_t cp_mode;                  /* gdn_cp_mode; AUTO decides from the shape */
    int32_t cp_segment_chunks;        /* segment length L in chunks; 0 = choose */
    int32_t o_dtype;                  /* gdn_dtype of o: equal to dtype, or GDN_DTYPE_F32 to receive
                                         the fp32 result before it is rounded to a bf16 output */
    /* In-kernel prologue (zero-initialised fields: the inputs are already processed).  Applied
     * inside the kernels instead of as separate passes over memory (the FLA KDA notes, section
     * "FlashKDA inference backend": l2-norm, sigma(beta) and the gate activation fused into the
     * kernel; the gate activation of the chunked gate cumsum kernel, section 2):
     *   qk_l2norm     1: every q and k row (one token, one head, D_k values) is used as
     *                 x / sqrt(sum x^2 + 1e-6);
     *   beta_sigmoid  1: beta holds logits, sigma(beta) = 1 / (1 + exp(-beta)) is used;
     *   A_log         NULL, or [H_v] fp32: g holds raw gate inputs x and the log-gate is
     *                   -exp(A_log[h]) * softplus(x + dt_bias)               (gate_lower_bound == 0)
     *                   gate_lower_bound * sigmoid(exp(A_log[h]) * (x + dt_bias))   (gate_lower_bound < 0)
     *   dt_bias       NULL (zero) or fp32 [H_v] (scalar gate) / [H_v][D_k] (per-channel gate); only
     *                 with A_log;
     *   gate_lower_bound  0, or a negative bound (only with A_log). */
    int32_t qk_l2norm;
    int32_t beta_sigmoid;
    const float *A_log;
    const float *dt_bias;
    float gate_lower_bound;
    float cp_warmup_tol;      /* GDN_CP_WARMUP: decay bound that ends a warmup, in [0, 1); 0 = 2^-24 */
    int32_t cp_form;          /* gdn_cp_form of the exact CP pre-process; 0 = AUTO */
} gdn_fwd_args;

/* Bytes of device workspace gdn_fwd needs for these arguments (0 on invalid
 * arguments).  Depends on shapes, the packed lengths and the CP decision only. */
size_t gdn_fwd_workspace_bytes(const gdn_fwd_args *a);

/* The schedule gdn_fwd would use for these arguments (in-GPU context parallelism, section
 * "key problems of FLA GDN chunked prefill" of the FlashQLA announcement: sequences split into
 * segments of segment_chunks chunks when too few (sequence, head, column group) chains exist).
 * Host-only: validates like gdn_fwd, launches nothing.  Returns the same status as validation. */
typedef struct {
    int32_t cp;                   /* 1 when sequences are split into segments */
    int32_t segment_chunks;       /* chunks per segment (the longest sequence's count when cp == 0) */
    int64_t total_segments;       /* segments over all sequences (N when cp == 0) */
    int32_t value_cols_per_group; /* D_v columns one recurrence workgroup carries */
    int32_t pieces;               /* chunk ranges of a batched input over which the per-chunk kernel
                                     (on a side stream) and the recurrence are pipelined; 1: none */
    size_t workspace_bytes;       /* as gdn_fwd_workspace_bytes */
    int32_t cp_form;              /* gdn_cp_form the exact CP pre-process runs in (0 without it) */
} gdn_plan_info;
gdn_status gdn_fwd_plan(const gdn_fwd_args *a, gdn_plan_info *info);

/* Validate, plan and enqueue the forward on `stream` (a hipStream_t).  The
 * workspace must be device memory of at least gdn_fwd_workspace_bytes(a)
 * bytes, 256-byte aligned; its contents on entry do not matter. */
gdn_status gdn_fwd(const gdn_fwd_args *a, void *workspace, size_t workspace_bytes, void *stream);

/* Stages of one forward, in launch order, for gdn_fwd_timed. */
enum {
    GDN_STAGE_PLAN = 0,      /* sequence / chunk tables */
    GDN_STAGE_INTRA = 1,     /* kernel (a): gate cumsum, gated beta*K K^T, inverse */
    GDN_STAGE_CP_PRE = 2,    /* in-GPU context parallelism: per-segment S* and M (GDN_CP_WARMUP: the
                                gate statistics that choose each segment's warmup length) */
    GDN_STAGE_CP_FIX = 3,    /* in-GPU context parallelism: serial fix-up of segment starts */
    GDN_STAGE_CHUNK = 4,     /* kernels (b)+(d): state recurrence fused with the output */
    GDN_N_STAGES = 5
};

/* Same as gdn_fwd, and also records caller-created hipEvent_t events on `stream` for
 * measurement: events[0] as the first stage's kernel starts and events[i + 1] as stage i's kernel
 * ends, for the stages that run with these arguments (bit i of *stages_run is set for them).  The
 * events ride in the kernels' own dispatches (hipExtLaunchKernel), so no separate event packets
 * sit between the kernels; a stage that launches no kernel records its events as plain events.  Events of stages that do not run are not
 * recorded, so a stage's duration is the time from the previous recorded event to its own.
 * events must hold GDN_N_STAGES + 1 entries, each a valid event or NULL (that boundary is not
 * recorded); stages_run may be NULL.  A start event in the first kernel's dispatch costs about
 * 5 us per call on MI355X (measured on the Qwen3-Next shape: 158-160 us per step against 154 us
 * without it), so a caller timing back-to-back calls can leave events[0] NULL and measure the
 * first stage from the previous call's last event. */
gdn_status gdn_fwd_timed(const gdn_fwd_args *a, void *workspace, size_t workspace_bytes, void *stream,
                         void *const *events, uint32_t *stages_run);

/* Allocation-free form of gdn_fwd, for callers that cannot allocate device memory or call
 * hipMalloc at the point of the call (code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation).  Same arguments, validation, results and stream semantics as gdn_fwd, but
 * no workspace argument: the workspace gdn_fwd would take is a static device array inside the
 * library of GDN_NOALLOC_SCRATCH_BYTES bytes, one copy per GPU, held from the first call on that
 * GPU until the process ends (its address is looked up on that first call, with the caller's
 * device current).  The call allocates nothing: no device or host memory, no streams, no events
 * (the chunk-range pieces that gdn_fwd may use on a side stream are never used here).
 * Errors: as gdn_fwd; GDN_ERR_WORKSPACE, with nothing enqueued, when the workspace these arguments
 * need (gdn_fwd_workspace_bytes(a)) exceeds GDN_NOALLOC_SCRATCH_BYTES.
 * Concurrency: every call on one GPU uses that GPU's one array, so calls whose work overlaps in
 * time on one GPU (different streams, or different host threads without ordering) race and give
 * undefined results; calls ordered on one stream are safe.  The array keeps the last call's
 * contents; no call depends on them. */
#define GDN_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
gdn_status gdn_fwd_noalloc(const gdn_fwd_args *a, void *stream);

/* Token-by-token forward (the fused recurrent form, chunk size 1; Flash Linear Attention page,
 * section 8): the decode path, for sequences of a few tokens (a chunked forward of fewer than
 * about 64 tokens pays its launch and intra-chunk overheads for nothing).  Same operation,
 * layouts and prologue fields as gdn_fwd; per sequence and value head, token by token,
 *   S <- alpha_t S (per-channel gate: Diag(alpha_t) S),  w = beta_t (v_t - S^T k_t),
 *   S <- S + k_t w^T,  o_t = scale S^T q_t,
 * with the state kept in fp32 and only the final state written.
 * Differences from gdn_fwd: chunk_size must be 1; cp_mode and cp_segment_chunks are ignored;
 * no workspace; h0 and final_state may be the same buffer (each state is read whole before it
 * is written: an in-place decode step).  cu_seqlens_host is still required with cu_seqlens_dev
 * (validation); the kernel reads the device copy, clamped into [0, B*T].
 * Errors and ownership as for gdn_fwd; enqueued on `stream`, not synchronised. */
gdn_status gdn_fwd_recurrent(const gdn_fwd_args *a, void *stream);

/* Backward of the chunked forward (GDN-in-FLA notes, backward Steps 1-7; Flash Linear Attention
 * page, section 7): the gradients of a loss through o and the final state, with the chunk states
 * recomputed (a forward replay), a reverse-time scan of the state gradient, and per chunk the
 * gradients of q, k, v, beta and the gate (dg as the reverse cumsum of the cumulative log-gate's
 * gradient within the chunk; per-channel gates: per channel).  Both gate kinds; no prologue, no
 * context parallelism.
 * Inputs as for gdn_fwd (same layouts and dtype), plus
 *   dout   [B, T, H_v, D_v]  dtype   gradient of o
 *   dht    [N, H_v, D_k, D_v] fp32   gradient of the final state (NULL: zero)
 * Outputs, all fp32 (written, every token of every sequence):
 *   dq, dk [B, T, H_qk, D_k] (summed over the value heads of a group), dv [B, T, H_v, D_v],
 *   dg shaped like g ([B, T, H_v], or [B, T, H_v, D_k] per channel), dbeta [B, T, H_v],
 *   dh0 [N, H_v, D_k, D_v] (NULL: not written).
 * Workspace: gdn_bwd_workspace_bytes(a) bytes of device memory, 256-byte aligned (it holds the
 * recomputed chunk states, the state gradients and the chunks' intra-chunk output matrices,
 * 2 x 4 D_k D_v + 16 KiB per chunk and head).
 * Errors and ownership as for gdn_fwd. */
typedef struct {
    int32_t B, T, H_qk, H_v, D_k, D_v;
    int32_t chunk_size;               /* 64 */
    int32_t dtype;                    /* gdn_dtype of q, k, v, beta and dout */
    int32_t gate_kind;                /* gdn_gate_kind */
    float scale;
    const void *q, *k, *v;
    const void *g;                    /* as for gdn_fwd: fp32 [B, T, H_v] or dtype [B, T, H_v, D_k] */
    const void *beta;
    const float *h0;                  /* nullable */
    const int32_t *cu_seqlens_dev;    /* nullable, as for gdn_fwd */
    const int32_t *cu_seqlens_host;
    int32_t N;
    const void *dout;
    const float *dht;                 /* nullable */
    float *dq, *dk, *dv, *dg, *dbeta;
    float *dh0;                       /* nullable */
} gdn_bwd_args;
size_t gdn_bwd_workspace_bytes(const gdn_bwd_args *a);
gdn_status gdn_bwd(const gdn_bwd_args *a, void *workspace, size_t workspace_bytes, void *stream);

/* Static, human-readable name of a status code. */
const char *gdn_status_string(gdn_status s);

/* Last validation message of this thread (empty when the last call succeeded). */
const char *gdn_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* GDN_H_ */
