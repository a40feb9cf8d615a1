/*
 * switch_ffn.h -- C-ABI of the SwitchFFN forward pass on one MI355X (gfx950).
 *
 * The layer (one Switch layer's sparse FFN, forward only):
 *   router   z[t,i] = sum_k x[t,k] Wr[i,k] in fp32; p[t,:] = softmax(z[t,:]);
 *            e_t = argmax_i z[t,i] (ties -> lowest index); gate g_t = p[t,e_t]
 *            ("Switch Transformers: Scaling to Trillion Parameter Models with
 *            Simple and Efficient Sparsity", section 3.4, "Switch Routing: The
 *            k=1 Simplification"; float32 router per "Selective Precision
 *            Training" in the same section).
 *   capacity C = floor(CF * T / N) (same page, "Distributed Implementation and
 *            Expert Capacity"; the pages round differently, this is the reading
 *            used throughout).  The first C tokens of an expert in token order
 *            are accepted; the rest are dropped (that section's overflow
 *            handling: a running count per expert, positions past C masked out).
 *   experts  E_e(v) = W2[e] ReLU(W1[e] v + b1[e]) + b2[e] ("Switch Transformer"
 *            paper note, section "Expert FFN Layer").
 *   combine  y_t = x_t + g_t E_{e_t}(x_t) for accepted tokens, y_t = x_t for
 *            dropped ones (section 3.2 "Big-Picture Architecture", information
 *            flow: scaled by the gate, added through the residual; overflow
 *            tokens pass through unchanged).
 *   aux      aux = N sum_i f_i P_i with f_i = #{t : e_t = i}/T (before capacity)
 *            and P_i = (1/T) sum_t p[t,i] (section 3.4, "The Load-Balancing
 *            Auxiliary Loss"); returned without the alpha factor.
 *
 * Layouts (row-major, all device memory):
 *   x [T, d]   Wr [N, d] (fp32)   W1 [N, F, d]   b1 [N, F]   W2 [N, d, F]
 *   b2 [N, d]  y [T, d]  expert_idx [T] (int32)  slot [T] (int32)
 *   gate [T] (fp32)  aux_loss [1] (fp32)
 * x, W1, b1, W2, b2 and y share `dtype` (SFFN_FP32 or SFFN_BF16); Wr, gate and
 * aux_loss are always fp32.  Every GEMM operand is contiguous along its
 * reduction axis.  b1 and b2 may be NULL (zero bias).
 *
 * Outputs for a dropped token t: expert_idx[t] = its routed expert,
 * slot[t] = -1, gate[t] = p[t, e_t], y[t] = x[t].  Accepted tokens have
 * slot[t] in [0, C): their position in the expert's buffer.
 *
 * Ownership and ordering: every pointer is owned by the caller.  The library
 * allocates nothing, keeps no state between calls (apart from loading its code
 * object once) and enqueues all work on `stream` (a hipStream_t; NULL = the
 * default stream) without synchronising the host: outputs are valid once the
 * stream reaches the end of the call, and inputs must stay unchanged until
 * then.  Calls on different streams are independent when each has its own
 * workspace and outputs.
 *
 * Errors: arguments are validated before anything is enqueued; on an error
 * nothing is launched and no output is touched.  SFFN_EHIP reports a launch
 * failure; the HIP error text is then available from
 * switch_ffn_status_string(SFFN_EHIP) on the same thread.
 *
 * Non-finite inputs are not checked and give non-finite results, but never an
 * access outside the buffers: the routing order treats a NaN logit as larger
 * than every number (ties and NaNs to the lowest index, numpy's argmax order),
 * so every token is routed to an expert in [0, N); its gate and the aux loss
 * then come out NaN.
 */
#ifndef SWITCH_FFN_H
#define SWITCH_FFN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
#define SFFN_OK 0
#define SFFN_EINVAL (-1)       /* null required pointer, T/d/F/N <= 0, CF < 0 or not finite */
#define SFFN_EDTYPE (-2)       /* dtype is neither SFFN_FP32 nor SFFN_BF16 */
#define SFFN_EWORKSPACE (-3)   /* workspace NULL or smaller than switch_ffn_workspace_bytes() */
#define SFFN_EUNSUPPORTED (-4) /* shape or alignment outside this library's limits (see below) */
#define SFFN_EHIP (-5)         /* a HIP launch failed */
#define SFFN_ESCRATCH (-6)     /* switch_ffn_forward_noalloc: the shape needs more than its scratch */

/* Element types of x, W1, b1, W2, b2 and y.  SFFN_BF16 is the performance path
 * (matrix-core GEMMs).  SFFN_FP32 computes the same layer in fp32 with
 * fp32 FMA kernels of one thread per output element, made for exactness on
 * small layers (the reference-precision check of the method): correct at
 * every supported shape, but far below the bf16 path's throughput on large
 * ones. */
#define SFFN_FP32 0
#define SFFN_BF16 1

/* forward_ex flags. */
#define SFFN_NO_RESIDUAL 1u /* y = g*E(x) for accepted tokens and 0 for dropped ones */
/* No-Token-Left-Behind rerouting ("Switch Transformers" summary, section 3.4,
 * "Distributed Implementation and Expert Capacity": the No-Token-Left-Behind
 * experiment of Appendix B, the two-stage process of Figure 11).  k = 1 only,
 * N >= 2 (else SFFN_EINVAL).  Stage 1 is the plain top-1 dispatch.  Stage 2
 * takes the tokens stage 1 refused, in token order, and places each in the
 * next free position of its second choice e2 (the largest fp32 logit other
 * than the first choice, ties -> lowest index) after e2's stage-1 tokens; a
 * position below C is accepted, and the token then uses e2 with gate
 * p[t, e2].  A token refused by both passes through (y = x).  Outputs:
 * expert_idx[t] is the expert t ends in (its first choice if refused by both),
 * gate[t] = p[t, expert_idx[t]], slot[t] its position or -1; the aux loss and
 * stats.expert_count count first choices, accepted_count = rows each expert
 * holds after both stages, n_dropped = tokens refused by both.  The
 * dispatch_scan stage also holds the second stage's count and scan.  The
 * workspace of switch_ffn_workspace_bytes() covers this flag. */
#define SFFN_REROUTE_OVERFLOW 2u
/* GEGLU experts ("Switch Transformers" summary, section 3.2, "Expert FFNs",
 * which names GEGLU beside ReLU): W1 is [N, 2F, d] and b1 [N, 2F]; rows
 * 0..F-1 of W1[e] are the gate projection W, rows F..2F-1 the linear
 * projection V, and the hidden activation is
 *   h = GELU(W x + b1[0..F)) * (V x + b1[F..2F)),  GELU(a) = a Phi(a)
 * (the exact GELU, Phi the standard normal CDF).  W2, b2, the workspace and
 * every other argument keep their meaning.  Any k, with or without the other
 * flags. */
#define SFFN_GEGLU 4u

/* Limits of this library (SFFN_EUNSUPPORTED beyond them):
 *   N <= 4096;  T * max(N, d, F) < 2^29;  d * F < 2^29 (byte offsets of every
 *   fp32 and bf16 tensor, the fp32 router logits [T, N] included, below 2^31);
 *   SFFN_BF16: d % 8 == 0, F % 8 == 0, and x, W1, W2, y 16-byte aligned. */
#define SFFN_MAX_EXPERTS 4096

/* Optional routing statistics of forward_ex (each pointer device memory, nullable):
 *   expert_count[N]   tokens whose top-1 is expert i (before capacity)
 *   accepted_count[N] tokens expert i processes: min(expert_count[i], C)
 *   n_dropped[1]      tokens dropped by the capacity limit */
typedef struct sffn_stats {
  int32_t* expert_count;
  int32_t* accepted_count;
  int32_t* n_dropped;
} sffn_stats;

/* Expert capacity C = floor((CF * T) / N), evaluated in IEEE double in that
 * order.  Returns -1 if T < 0, N <= 0, or CF is negative or not finite.
 * Host only; touches no device. */
int64_t switch_ffn_capacity(int64_t T, int64_t N, double CF);

/* Bytes of device workspace switch_ffn_forward needs for this shape (0 on bad
 * arguments).  Host only.  The workspace holds, from its start, a layout tag
 * of 16 uint32 words (magic 0x4E464653, version 1, k, flags, T, d, F, N, C,
 * dtype, then zeros) in a 256-byte region, so that the backward pass can tell
 * which form of the layer wrote the rest; from byte 256 the fp32 router logits
 * z [T, N] (row-major; a forward call leaves them there for the backward
 * pass), then per-block probability sums, dispatch counts and offsets, the
 * row-to-token map and the expert hidden activations [min(T, N*C), F]. */
size_t switch_ffn_workspace_bytes(int64_t T, int64_t d, int64_t F, int64_t N, double CF,
                                  int dtype);

/* The SwitchFFN forward pass (see the top of this file).  `workspace` is a
 * device buffer of at least switch_ffn_workspace_bytes() bytes, 256-byte
 * aligned; its contents on entry do not matter and are garbage afterwards.
 * `stream` is a hipStream_t.  Returns SFFN_OK or a negative status. */
int switch_ffn_forward(const void* x, const float* Wr, const void* W1, const void* b1,
                       const void* W2, const void* b2, int64_t T, int64_t d, int64_t F,
                       int64_t N, double CF, int dtype, void* y, int32_t* expert_idx,
                       int32_t* slot, float* gate, float* aux_loss, void* workspace,
                       size_t workspace_bytes, void* stream);

/* switch_ffn_forward plus:
 *   flags         0 or an OR of SFFN_NO_RESIDUAL (a diagnostic: the bare expert
 *                 term), SFFN_REROUTE_OVERFLOW (No-Token-Left-Behind) and
 *                 SFFN_GEGLU (GEGLU experts); other bits: SFFN_EINVAL
 *   stats         optional routing statistics (NULL = none)
 * Per-stage timing events: switch_ffn_forward_topk with k = 1. */
int switch_ffn_forward_ex(const void* x, const float* Wr, const void* W1, const void* b1,
                          const void* W2, const void* b2, int64_t T, int64_t d, int64_t F,
                          int64_t N, double CF, int dtype, void* y, int32_t* expert_idx,
                          int32_t* slot, float* gate, float* aux_loss, void* workspace,
                          size_t workspace_bytes, void* stream, uint32_t flags,
                          const sffn_stats* stats);

/* Top-k routing, k = 1 or 2 (k = 2: the MoE top-2 baseline the Switch summary
 * contrasts with, section "Why Top-1 Routing Matters" and its top-2 routing
 * formula y = sum over the two largest p[t,i] of p[t,i] E_i(x); section 3.4
 * gives the capacity k x tokens / N x capacity factor).  With k = 2:
 *   choices  e[t,0] = argmax_i z[t,i], e[t,1] = argmax over i != e[t,0]
 *            (fp32 logits, ties -> lowest index)
 *   gates    gate[t,c] = p[t, e[t,c]] (raw, not renormalised)
 *   capacity C = floor(CF * (k*T) / N) = switch_ffn_capacity(k*T, N, CF); each
 *            expert's buffer is filled in token order (a token holds at most
 *            one position per expert), the first C accepted, the rest dropped
 *   combine  y_t = x_t + sum over t's accepted choices of gate[t,c] E_{e[t,c]}(x_t)
 *            (y_t = x_t when both are dropped); SFFN_NO_RESIDUAL drops the x_t term
 *   aux      as for k = 1: f_i counts the top-1 choices
 *   outputs  expert_idx, slot, gate are [T, k], row-major (choice minor);
 *            stats: expert_count[i] = tokens with i among their k choices,
 *            accepted_count = min(expert_count, C), n_dropped = dropped choices.
 * k = 1 is exactly switch_ffn_forward_ex.  k = 2 needs N >= 2 and
 * min(2T, N*C) * max(d, F) * 4 < 2^31 (else SFFN_EUNSUPPORTED); k outside
 * {1, 2} or N < k is SFFN_EINVAL.
 * stage_events: NULL, or a host array of switch_ffn_num_stages()+1 hipEvent_t
 * handles created by the caller; event i is recorded on `stream` before stage
 * i and the last one after the final stage, so the caller can time each stage
 * (with k = 2 the ffn2 stage also holds the combine). */
size_t switch_ffn_workspace_bytes_topk(int64_t T, int64_t d, int64_t F, int64_t N, double CF,
                                       int k, int dtype);
int switch_ffn_forward_topk(const void* x, const float* Wr, const void* W1, const void* b1,
                            const void* W2, const void* b2, int64_t T, int64_t d, int64_t F,
                            int64_t N, double CF, int k, int dtype, void* y, int32_t* expert_idx,
                            int32_t* slot, float* gate, float* aux_loss, void* workspace,
                            size_t workspace_bytes, void* stream, uint32_t flags,
                            const sffn_stats* stats, void* const* stage_events);

/* Backward pass of the top-1 layer with ReLU experts (forward flags 0: k = 1,
 * residual on, no rerouting, no GEGLU).  The routing is a piecewise-constant
 * choice without a gradient; the router learns through the gate p[t, e_t]
 * ("Switch Transformers" summary, section 3.4, "Switch Routing: The k=1
 * Simplification") and through P_i of the aux loss, f_i being a count with no
 * gradient ("Switch Transformer, explained.", the symbols under "Why one
 * expert is enough"; the summary's "The Load-Balancing Auxiliary Loss").
 * For an accepted token t of expert e (a = W1 x + b1, h = ReLU(a),
 * o = W2 h + b2, g = gate):
 *   dW2_e += g dy h^T,  db2_e += g dy,  da = (W2^T g dy) * [h > 0],
 *   dW1_e += da x^T,  db1_e += da,  dx_t = dy_t + W1^T da + Wr^T dz_t,
 *   dz_t = p_t * (u_t - p_t . u_t),  u_{t,i} = d_aux N f_i / T + [i = e] dy . o
 * (dropped tokens: dx_t = dy_t + Wr^T dz_t with the aux term of u alone);
 * dWr = sum_t dz_t x_t^T.  ReLU'(0) = 0; the mask uses the forward's H.
 * Arguments:
 *   x, Wr, W1, b1, W2, b2, T, d, F, N, CF, dtype  exactly as in the forward call
 *   expert_idx, slot  [T] the forward's outputs (device)
 *   fwd_workspace     the forward's workspace (device), as that call left it:
 *                     it holds the layout tag, the fp32 router logits, the
 *                     dispatch (offsets, row maps, gates, counts) and the
 *                     hidden activations H; only read here.  Its tag must name
 *                     a forward with k = 1, without SFFN_REROUTE_OVERFLOW or
 *                     SFFN_GEGLU, of the same T, d, F, N, C and dtype
 *                     (SFFN_NO_RESIDUAL does not matter).  While `stream` is
 *                     not being captured into a graph, the tag is read on the
 *                     host before anything is enqueued (the call then waits
 *                     for the stream's earlier work) and any other tag returns
 *                     SFFN_EINVAL.  Under capture the forward has not run yet:
 *                     the first kernel checks the tag on the device, together
 *                     with the expert offsets, and on a mismatch the call
 *                     reads none of the forward's row maps and every gradient
 *                     comes out NaN.
 *   dy                [T, d] dL/dy (device, dtype)
 *   d_aux             dL/d(aux_loss) (host value; the alpha factor goes here)
 * Outputs (device, caller-allocated, overwritten): dx [T, d] (dtype),
 * dWr [N, d] fp32, dW1 [N, F, d], dW2 [N, d, F] (dtype), db1 [N, F] and
 * db2 [N, d] (dtype; each nullable: then not computed).  Experts without
 * tokens get zero gradients.  `workspace`: a device buffer of at least
 * switch_ffn_backward_workspace_bytes() bytes, 256-byte aligned, separate
 * from fwd_workspace.  stage_events: NULL or switch_ffn_backward_num_stages()+1
 * events, recorded like forward_topk's.  expert_idx[t] outside [0, N) or
 * slot[t] >= C reads as a dropped token.  Returns SFFN_OK, SFFN_EINVAL (a null
 * required pointer, d_aux not finite, the shape checks of the forward, or a
 * forward workspace whose tag names another form of the layer),
 * SFFN_EWORKSPACE (either workspace too small), SFFN_EUNSUPPORTED (alignment,
 * limits) or SFFN_EHIP. */
size_t switch_ffn_backward_workspace_bytes(int64_t T, int64_t d, int64_t F, int64_t N, double CF,
                                           int dtype);
int switch_ffn_backward(const void* x, const float* Wr, const void* W1, const void* b1,
                        const void* W2, const void* b2, int64_t T, int64_t d, int64_t F,
                        int64_t N, double CF, int dtype, const int32_t* expert_idx,
                        const int32_t* slot, const void* fwd_workspace,
                        size_t fwd_workspace_bytes, const void* dy, float d_aux, void* dx,
                        float* dWr, void* dW1, void* db1, void* dW2, void* db2, void* workspace,
                        size_t workspace_bytes, void* stream, void* const* stage_events);
int switch_ffn_backward_num_stages(void);
const char* switch_ffn_backward_stage_name(int stage);

/* Number of stages forward_ex reports events around, and their names
 * ("router_logits", "softmax_route", ...); NULL for an index out of range. */
int switch_ffn_num_stages(void);
const char* switch_ffn_stage_name(int stage);

/* Allocation-free forward, for callers that cannot allocate device memory
 * (code under stream capture, tight serving loops, harnesses that forbid
 * allocation).  switch_ffn_forward with the same arguments minus the
 * workspace: the workspace is a file-scope device array of
 * SFFN_NOALLOC_SCRATCH_MIB MiB inside the library (each GPU the library runs
 * on holds its own copy from the first call there until the process ends),
 * looked up once per device with that device current.  The call allocates
 * nothing.  Shapes whose switch_ffn_workspace_bytes() exceeds
 * switch_ffn_noalloc_scratch_bytes() return SFFN_ESCRATCH before anything is
 * enqueued (64 MiB covers the Switch-Base-like layer: T = 8192, d = 768,
 * F = 3072, N = 64); other errors are switch_ffn_forward's.  Every call on one
 * GPU uses that GPU's one array, which keeps the last call's contents (the
 * forward needs nothing cleared): calls that overlap on one GPU -- on
 * different streams, or from different threads, without ordering between
 * them -- race on it, and a backward pass cannot use this forward's
 * workspace.  Outputs as switch_ffn_forward's. */
#define SFFN_NOALLOC_SCRATCH_MIB 64
size_t switch_ffn_noalloc_scratch_bytes(void);
int switch_ffn_forward_noalloc(const void* x, const float* Wr, const void* W1, const void* b1,
                               const void* W2, const void* b2, int64_t T, int64_t d, int64_t F,
                               int64_t N, double CF, int dtype, void* y, int32_t* expert_idx,
                               int32_t* slot, float* gate, float* aux_loss, void* stream);

/* Static description of a status code; for SFFN_EHIP, the text of the last
 * HIP error seen on this thread. */
const char* switch_ffn_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* SWITCH_FFN_H */
