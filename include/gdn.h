/*
 * gdn.h -- C ABI of the MI355X (gfx950) Gated DeltaNet layer forward.
 *
 * The operation.  The LinMorph project page ("Abstract" and "Why learn the
 * initialization?") replaces the softmax self-attention of a video diffusion
 * transformer with a Gated DeltaNet (GDN) token mixer whose parameter groups
 * are update gates, decay terms, short convolutions and normalisation
 * parameters; the VMonarch page (section 2, "Efficient Attention
 * Mechanisms", ref. [57]) files GDN under linear attention with an expanded
 * recurrent state.  One call computes, for every batch row b and head h of a
 * flattened video token sequence of length T:
 *
 *   1. short convolution + SiLU on q, k and v, per channel c:
 *        x~_t[c] = SiLU( sum_{j=0..3} w[c][j] * x_{t-3+j}[c] ),  x_{<0} = 0
 *   2. unit-L2 queries and keys:  q^_t = q~_t / sqrt(|q~_t|^2 + eps_l2),
 *      likewise k^_t;  v^_t = v~_t
 *   3. the gated delta rule with state S in R^{Dv x Dk} (S_{-1} = S0):
 *        S_t = a_t S_{t-1} (I - b_t k^_t k^_t^T) + b_t v^_t k^_t^T,
 *        o_t = S_t q^_t,   a_t = exp(log_a_t)
 *   4. gated RMS normalisation over the Dv channels:
 *        y_t = o_t / sqrt(mean(o_t^2) + eps_norm) * norm_w * SiLU(gate_t)
 *   5. S_T = the state after the last token.
 *
 * Layouts (row-major, contiguous, no strides):
 *   q, k          [B, T, H, Dk]   io_dtype
 *   v, gate, o    [B, T, H, Dv]   io_dtype
 *   log_a, beta   [B, T, H]       float32  (log_a <= 0 expected, beta in [0,1])
 *   conv_q, conv_k [H*Dk, 4], conv_v [H*Dv, 4]  float32; tap 3 multiplies
 *                 the current token, tap j the token 3-j steps earlier
 *   norm_w        [H, Dv]         float32, or NULL for all ones
 *   S0, S_T       [B, H, Dv, Dk]  float32, S0 NULL means zeros,
 *                 S_T NULL means not written
 *
 * Ownership.  Every pointer is a device pointer owned by the caller, except
 * the params struct itself (host memory, read during the call only).  The
 * library allocates and frees nothing and keeps no pointer after return; the
 * caller supplies a device workspace of at least gdn_fwd_workspace_bytes()
 * (or gdn_fwd_bidir_workspace_bytes()) bytes, 256-byte aligned, which the
 * call may overwrite entirely.
 *
 * Execution.  A call is ordered on `stream` (NULL = the null stream) like a
 * single operation and returns without waiting: its kernels run on `stream`
 * and on up to three library streams per device (created on first use and
 * kept, default priority), which wait for `stream` at the start of the call
 * and which `stream` waits for at its end.  Calls from several host threads
 * are enqueued one at a time (a lock); their work may then share the library
 * streams.  Two in-flight calls must not share a workspace.  A call can be
 * captured into a HIP graph on `stream` (the fork onto the library streams
 * and the join back are captured with it; the first call on a device, which
 * creates those streams and events, should run before capturing); a replay
 * repeats the call exactly.  gdn_fwd_varlen copies its table from host
 * memory and is not meant for capture.
 *
 * Graph cache.  Outside a capture, on a stream other than the null stream,
 * gdn_fwd, gdn_fwd_varlen and gdn_mixer_fwd (its layer and out-projection)
 * record their launches as a HIP graph (a capture of `stream`, in thread-local mode,
 * inside the call) the second time a call has the same launches (the same
 * sizes, pointers and scalars; the first such call launches directly), and
 * replay the graph for every later such call.  The result is the same as
 * launching directly, bit for bit; the graph removes the gaps between
 * dependent kernels on different streams.  Callers whose buffers move from
 * call to call simply keep launching directly.  The library keeps the most
 * recently used graphs per process (8 by default), each holding only the
 * recorded launches, no memory of its own.  gdn_fwd_bidir, the timed calls
 * and calls on the null stream or on a stream being captured always launch
 * directly.
 *   gdn_set_graph_cache_limit(n): keep at most n graphs (0 <= n <= 64;
 *     0 turns the cache off and frees it); GDN_ERR_INVALID_ARG otherwise.
 *     Graphs past the new limit are destroyed at once, so call it with no
 *     library call in flight on any stream.
 *   gdn_graph_cache_count(): the number of graphs held.
 *
 * Errors.  All checks run on the host before anything is enqueued; on any
 * error nothing is launched and no output is touched.  Launch failures
 * return GDN_ERR_HIP.  Faults inside kernels surface at the caller's next
 * synchronisation, as usual in HIP.  No C++ exception crosses this ABI.
 */
#ifndef GDN_H_
#define GDN_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

struct ihipStream_t; /* hipStream_t is `struct ihipStream_t *` */

typedef enum {
    GDN_OK = 0,
    GDN_ERR_INVALID_ARG = 1, /* NULL required pointer, bad size, non-finite or negative eps, aliasing */
    GDN_ERR_UNSUPPORTED = 2, /* a valid request this build has no kernel for (see gdn_fwd) */
    GDN_ERR_ALIGNMENT = 3,   /* tensors not 16-byte aligned, workspace not 256-byte aligned */
    GDN_ERR_WORKSPACE = 4,   /* workspace NULL or smaller than required */
    GDN_ERR_HIP = 5          /* a HIP runtime call or kernel launch failed */
} gdn_status;

typedef enum { GDN_F32 = 0, GDN_BF16 = 1 } gdn_dtype;

typedef struct gdn_fwd_params {
    int B, T, H, Dk, Dv;      /* B, T, H >= 1; Dk == Dv */
    gdn_dtype io_dtype;       /* dtype of q, k, v, gate and o */
    const void *q, *k, *v;
    const float *log_a;       /* the decay a_t in log space */
    const float *beta;        /* the update gate b_t */
    const void *gate;         /* output gate, SiLU-activated */
    const float *conv_q, *conv_k, *conv_v;
    const float *norm_w;      /* NULL: ones */
    float eps_l2, eps_norm;   /* >= 0 and finite; 1e-6 in the shipped workloads */
    const float *S0;          /* NULL: zero initial state */
    void *o;                  /* output y, overwritten */
    float *S_T;               /* final state, or NULL */
    int reverse;              /* 0: scan t = 0..T-1; 1: scan t = T-1..0, i.e. the
                                 layer applied to the time-reversed sequence with
                                 its output written back in input order */
    void *workspace;
    size_t workspace_bytes;
} gdn_fwd_params;

/*
 * Device workspace gdn_fwd needs for these sizes (only B, T, H, Dk, Dv and
 * io_dtype are read).  Returns 0 if the sizes are invalid.
 */
size_t gdn_fwd_workspace_bytes(const gdn_fwd_params *p);

/*
 * One GDN layer forward (steps 1-5 above), in scan order given by p->reverse.
 * Supported: io_dtype GDN_BF16 or GDN_F32 with Dk = Dv in {64, 128}; other
 * sizes return GDN_ERR_UNSUPPORTED.  With bf16 I/O the matrix products take
 * bf16 operands with fp32 accumulation and an fp32 master state; with fp32
 * I/O they run in fp32 throughout.
 */
gdn_status gdn_fwd(const gdn_fwd_params *p, struct ihipStream_t *stream);

/*
 * gdn_fwd for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same operation, results equal to gdn_fwd's bit for bit, but p->workspace
 * and p->workspace_bytes are ignored.  The workspace is instead a 64 MiB
 * array the library holds in device memory (one per GPU, for the life of the
 * process).  The call allocates nothing and creates nothing (no memory,
 * streams, events or graphs): its kernels run one after another on
 * `stream`.  Sizes whose workspace (gdn_fwd_workspace_bytes) exceeds 64 MiB
 * return GDN_ERR_WORKSPACE before any device call; for example B = 1,
 * H = 8, D = 128 bf16 fits up to T = 4544.  All calls on one GPU share the
 * array: calls that may overlap on that GPU (on different streams, or from
 * different threads without ordering) race and must not be issued.  Every
 * other rule is gdn_fwd's.
 */
gdn_status gdn_fwd_noalloc(const gdn_fwd_params *p, struct ihipStream_t *stream);

/* Workspace for gdn_fwd_bidir (two scans' partial results at once). */
size_t gdn_fwd_bidir_workspace_bytes(const gdn_fwd_params *p);

/*
 * Bidirectional stress variant: the whole layer run forward in time and on
 * the time-reversed sequence (each scan with its own causal convolution and
 * its own output normalisation, both from S0), the two outputs added in fp32
 * and stored once into p->o.  p->reverse must be 0.  p->S_T receives the
 * forward scan's final state and S_T_rev the reversed scan's (either may be
 * NULL).
 */
gdn_status gdn_fwd_bidir(const gdn_fwd_params *p, float *S_T_rev,
                         struct ihipStream_t *stream);

/*
 * Variable-length batch: p->B sequences of different lengths packed along
 * the token axis, each its own scan with its own initial and final state
 * (classifier-free-guidance pairs of equal length can also use gdn_fwd with
 * B = 2).  cu_seqlens is a HOST array of p->B + 1 ints: cu_seqlens[0] = 0,
 * sequence b is token rows cu_seqlens[b] .. cu_seqlens[b+1] - 1, every length
 * >= 1 (else GDN_ERR_INVALID_ARG).  The table is read during the call and
 * copied into the workspace on `stream`; the caller may release it when the
 * call returns.  p->T is ignored (the library uses the longest length).
 * Layouts: q, k, v, gate, o [total, H, D] and log_a, beta [total, H] with
 * total = cu_seqlens[p->B]; S0, S_T [p->B, H, Dv, Dk].  Everything else
 * (dtypes, supported sizes, reverse, errors, execution) is as for gdn_fwd;
 * the workspace is gdn_fwd_varlen_workspace_bytes(p, cu_seqlens) bytes (0 for
 * an invalid table).  Each sequence's result equals gdn_fwd on that sequence
 * alone.
 */
size_t gdn_fwd_varlen_workspace_bytes(const gdn_fwd_params *p, const int *cu_seqlens);
gdn_status gdn_fwd_varlen(const gdn_fwd_params *p, const int *cu_seqlens, struct ihipStream_t *stream);

/*
 * Measurement aids.  A call is a fixed sequence of kernel launches (a range
 * of chunks per launch, spread over the streams above);
 * gdn_fwd_launch_count() says how many (bidirectional != 0 for
 * gdn_fwd_bidir), or -1 for invalid or unsupported sizes, and
 * gdn_fwd_launch_name() names launch i (static string, NULL if out of range).
 * gdn_fwd_timed() does exactly what gdn_fwd (bidirectional == 0) or
 * gdn_fwd_bidir (bidirectional != 0; S_T_rev as there) does, and in addition
 * records events[2i] right before launch i and events[2i+1] right after it,
 * on the stream that launch runs on, so launch i's duration is the elapsed
 * time between those two events.  events: n_events >= 2 * count
 * caller-created HIP events with timing enabled (hipEvent_t is
 * `struct ihipEvent_t *`); otherwise GDN_ERR_INVALID_ARG and nothing is
 * launched.
 */
struct ihipEvent_t;
int gdn_fwd_launch_count(const gdn_fwd_params *p, int bidirectional);
const char *gdn_fwd_launch_name(const gdn_fwd_params *p, int bidirectional, int i);
gdn_status gdn_fwd_timed(const gdn_fwd_params *p, float *S_T_rev, int bidirectional,
                         struct ihipEvent_t **events, int n_events,
                         struct ihipStream_t *stream);

/*
 * Token mixer projections.  The GDN layer's per-token inputs come from the
 * hidden states x through linear projections, and its output goes back
 * through one (LinMorph project page, "Why learn the initialization?": the
 * GDN parameters are built from the pretrained query, key, value and output
 * projections; the T3-Video page, Table 1, counts the "QKV proj." and
 * "O proj." MACs of Wan2.1-T2V-1.3B).  Weights use the layout of a linear
 * layer, [out_features, in_features], bf16; products take bf16 operands with
 * fp32 accumulation on MFMA.
 *
 * gdn_in_proj computes, per token row m of x [B*T, C]:
 *   z = x_m W_in^T + b_in,  W_in = [W_q; W_k; W_v; W_g; W_b; W_a]
 *   q, k, v, gate = bf16(z[part])     (H*D columns each, [B, T, H, D])
 *   beta[h]  = sigmoid(z_b[h])                    ([B, T, H] float32)
 *   log_a[h] = -exp(A_log[h]) * softplus(z_a[h])  ([B, T, H] float32)
 * i.e. the update gate b in (0, 1) and the decay a = exp(log_a) in (0, 1]
 * that gdn_fwd takes, with softplus(z) = log(1 + e^z).
 *
 * Layouts (row-major, contiguous):
 *   x      [B, T, C]             bf16, 16-byte aligned
 *   w_in   [4*H*D + 2*H, C]      bf16, 16-byte aligned; rows in the order
 *                                q (H*D), k (H*D), v (H*D), gate (H*D),
 *                                b (H), a (H); within a block, row h*D + i
 *                                is head h, channel i
 *   b_in   [4*H*D + 2*H]         float32, 16-byte aligned, or NULL (no bias)
 *   A_log  [H]                   float32
 * Requirements: C % 64 == 0, (H*D) % 16 == 0, B*T*C and (4*H*D+2*H)*C below
 * 2^31; otherwise GDN_ERR_UNSUPPORTED.  Ownership, ordering and errors as for
 * gdn_fwd: device buffers owned by the caller, no allocation, one launch on
 * `stream`, all checks on the host first (outputs must not overlap inputs or
 * each other).
 */
typedef struct gdn_in_proj_params {
    int B, T, H, D, C;
    const void *x;
    const void *w_in;
    const float *b_in;        /* NULL: no bias */
    const float *A_log;
    void *q, *k, *v, *gate;   /* [B, T, H, D] bf16 outputs */
    float *beta, *log_a;      /* [B, T, H] float32 outputs */
} gdn_in_proj_params;

gdn_status gdn_in_proj(const gdn_in_proj_params *p, struct ihipStream_t *stream);

/*
 * gdn_out_proj:  out = y W_out^T + b_out  per token row, y being the layer
 * output [B, T, H, D] viewed as [B*T, H*D].
 *   y      [B, T, H, D]   bf16, 16-byte aligned
 *   w_out  [C, H*D]       bf16, 16-byte aligned
 *   b_out  [C]            float32, 16-byte aligned, or NULL
 *   out    [B, T, C]      bf16 output
 * Requirements: (H*D) % 64 == 0, C % 8 == 0, B*T*H*D and C*H*D below 2^31;
 * otherwise GDN_ERR_UNSUPPORTED.  Conventions as for gdn_in_proj.
 */
typedef struct gdn_out_proj_params {
    int B, T, H, D, C;
    const void *y;
    const void *w_out;
    const float *b_out;       /* NULL: no bias */
    void *out;
} gdn_out_proj_params;

gdn_status gdn_out_proj(const gdn_out_proj_params *p, struct ihipStream_t *stream);

/*
 * The whole token mixer: gdn_in_proj, then the layer (gdn_fwd, forward scan,
 * bf16), then gdn_out_proj, as one call ordered on `stream`:
 *   out = out_proj( GDN layer( in_proj(x) ) )
 * The out-projection runs in parts, one per chunk range of the layer's launch
 * plan, each on a library stream right after the layer's output kernel of
 * that range (so beside the layer's later ranges); the result is the same,
 * bit for bit, as the three stages called one after another.
 * The intermediates (q, k, v, gate, b, log a and the layer output y) live in
 * the caller's workspace, of at least gdn_mixer_workspace_bytes() bytes,
 * 256-byte aligned (that function reads B, T, H, D, C only and returns 0 for
 * invalid sizes).  D must be 64 or 128 and every requirement of the three
 * stages holds; all checks of all stages run before the first launch.
 *   x [B, T, C], w_in, b_in, A_log as for gdn_in_proj; conv_*, norm_w, eps,
 *   S0, S_T as for gdn_fwd; w_out, b_out as for gdn_out_proj; out [B, T, C]
 *   bf16.  No caller buffer may overlap the workspace; out may not overlap
 *   any input.
 * gdn_mixer_fwd_timed does the same and records events[0] / events[1] around
 * the in-projection launch, events[2] / events[3] around the output
 * projection, and events[4 + 2i] / events[5 + 2i] around launch i of the
 * layer (gdn_fwd_launch_count of the layer's sizes), on the stream each runs
 * on; n_events >= 4 + 2 * that count, else GDN_ERR_INVALID_ARG.
 */
typedef struct gdn_mixer_params {
    int B, T, H, D, C;
    const void *x;
    const void *w_in;
    const float *b_in;        /* NULL: no bias */
    const float *A_log;
    const float *conv_q, *conv_k, *conv_v;
    const float *norm_w;      /* NULL: ones */
    float eps_l2, eps_norm;
    const float *S0;          /* NULL: zero initial state */
    float *S_T;               /* final state, or NULL */
    const void *w_out;
    const float *b_out;       /* NULL: no bias */
    void *out;
    void *workspace;
    size_t workspace_bytes;
} gdn_mixer_params;

size_t gdn_mixer_workspace_bytes(const gdn_mixer_params *p);
gdn_status gdn_mixer_fwd(const gdn_mixer_params *p, struct ihipStream_t *stream);
gdn_status gdn_mixer_fwd_timed(const gdn_mixer_params *p, struct ihipEvent_t **events, int n_events,
                               struct ihipStream_t *stream);

/* The graph cache of gdn_fwd, gdn_fwd_varlen and gdn_mixer_fwd (see "Graph
 * cache" at the top of this header). */
gdn_status gdn_set_graph_cache_limit(int max_graphs);
int gdn_graph_cache_count(void);

/*
 * The layer's backward pass: the gradients of steps 1-5 (gdn_fwd with the
 * same reverse flag) with respect to every input, for equal-length batch
 * rows.  The bidirectional variant's gradients are the sums of the calls with
 * reverse = 0 and reverse = 1 (each with its own dS_T).
 * The pages train the converted GDN blocks (LinMorph project page,
 * "Abstract": progressive distillation and joint recovery), which needs
 * them; they are taken through the forward's chunked form (the delta rule
 * unrolled inside 64-token chunks).  Given dy = dL/dy and dS_T = dL/dS_T, one call
 * writes
 *   dq, dk, dv, dgate   [B, T, H, D]   io_dtype
 *   dlog_a, dbeta       [B, T, H]      float32
 *   dconv_q, dconv_k, dconv_v [H*D, 4] float32 (sums over batch rows and tokens)
 *   dnorm_w             [H, Dv]        float32, the gradient at norm_w (ones
 *                                      when norm_w is NULL); NULL: not written
 *   dS0                 [B, H, Dv, Dk] float32, also when S0 is NULL (the
 *                                      gradient at the zero state); NULL: not written
 * The inputs have the layouts of gdn_fwd; dy is [B, T, H, Dv] in io_dtype,
 * dS_T [B, H, Dv, Dk] float32 or NULL (zero).  The forward is recomputed
 * inside the call (nothing is kept from a gdn_fwd call).
 * Supported: Dk = Dv in {64, 128}, io_dtype GDN_BF16 or GDN_F32.  All
 * arithmetic is fp32 (fp32 MFMA); bf16 inputs are read exactly and bf16
 * outputs rounded to nearest even once.
 * Execution: as for gdn_fwd, the call is ordered on `stream` like a single
 * operation.  The two chains run over ranges of chunks on `stream`, and the
 * kernels that follow each range run on one library stream per device
 * (created on first use and kept, default priority), which waits for
 * `stream` at the start of the call and which `stream` waits for at its end;
 * enqueueing is serialised by a lock.  gdn_bwd_timed runs the 7 kernels once
 * each, in order, on `stream` alone (same results, bit for bit).
 * The workspace (gdn_bwd_workspace_bytes(), 256-byte aligned) holds the
 * recomputed chunk quantities in fp32: about (909 D + 12416 + 2 D^2) * 4
 * bytes per (batch row, head, 64-token chunk), 4.0 GB at B = 1, T = 32760,
 * H = 12, D = 128.
 * Errors: as for gdn_fwd.  GDN_ERR_INVALID_ARG for a NULL required pointer,
 * bad sizes, eps < 0 or not finite, reverse not 0 or 1, or an output that
 * overlaps an input, another output or the workspace; GDN_ERR_ALIGNMENT for
 * q, k, v or a conv weight not 16-byte aligned, another tensor not aligned
 * to its element size, or a workspace not 256-byte aligned;
 * GDN_ERR_UNSUPPORTED for other D.
 */
typedef struct gdn_bwd_params {
    int B, T, H, Dk, Dv;
    gdn_dtype io_dtype;
    const void *q, *k, *v;
    const float *log_a, *beta;
    const void *gate;
    const float *conv_q, *conv_k, *conv_v;
    const float *norm_w;      /* NULL: ones */
    float eps_l2, eps_norm;
    const float *S0;          /* NULL: zero initial state */
    const void *dy;           /* gradient of the output y */
    const float *dS_T;        /* gradient of the final state, or NULL */
    void *dq, *dk, *dv, *dgate;
    float *dlog_a, *dbeta;
    float *dconv_q, *dconv_k, *dconv_v;
    float *dnorm_w;           /* or NULL */
    float *dS0;               /* or NULL */
    int reverse;              /* 0 or 1, as for gdn_fwd */
    void *workspace;
    size_t workspace_bytes;
} gdn_bwd_params;

/* Workspace gdn_bwd needs (only B, T, H, Dk, Dv and io_dtype are read); 0 if
 * the sizes are invalid. */
size_t gdn_bwd_workspace_bytes(const gdn_bwd_params *p);
gdn_status gdn_bwd(const gdn_bwd_params *p, struct ihipStream_t *stream);
/* As gdn_bwd, with events[2 i] and events[2 i + 1] recorded on `stream`
 * around kernel i (n_events >= 2 * gdn_bwd_launch_count()). */
gdn_status gdn_bwd_timed(const gdn_bwd_params *p, struct ihipEvent_t **events, int n_events,
                         struct ihipStream_t *stream);
/*
 * The backward of gdn_fwd_varlen: p->B sequences packed along the token axis
 * (cu_seqlens: a HOST array of p->B + 1 ints, as for gdn_fwd_varlen; p->T is
 * ignored).  q, k, v, gate, dy and dq, dk, dv, dgate are [total, H, D];
 * log_a, beta, dlog_a, dbeta [total, H]; S0, dS_T, dS0 [p->B, H, D, D]; the
 * weight gradients are sums over all sequences.  The table is copied into the
 * workspace (gdn_bwd_varlen_workspace_bytes(p, cu_seqlens) bytes; 0 for an
 * invalid table) on `stream`.  Each sequence's per-token and per-sequence
 * gradients equal gdn_bwd on that sequence alone.
 */
size_t gdn_bwd_varlen_workspace_bytes(const gdn_bwd_params *p, const int *cu_seqlens);
gdn_status gdn_bwd_varlen(const gdn_bwd_params *p, const int *cu_seqlens, struct ihipStream_t *stream);
/* The number of kernels of a gdn_bwd call, and the name of kernel i
 * (NULL out of range). */
int gdn_bwd_launch_count(void);
const char *gdn_bwd_launch_name(int i);

/* Static, human-readable text for a status code. */
const char *gdn_status_string(gdn_status s);

#ifdef __cplusplus
}
#endif

#endif /* GDN_H_ */
