/*
 * linattn.h — C ABI of the MI355X (gfx950) library for causal linear-attention
 * sequence mixing with a fixed d_k x d_v fp32 state per head.
 *
 * The operation (page titles as published):
 *   "Linear Attention, Visualized" — sections "Naive linear attention" (state
 *   S_t, inclusive causal read-out), "Mamba-2: input-dependent scalar decay",
 *   "Gated Linear Attention (GLA)" (per-key-channel decay), "DeltaNet:
 *   correcting memory collisions" (recurrent form with the scaled correction),
 *   "Gated DeltaNet (GDN)" and "Kimi Delta Attention (KDA)" (decay first, then
 *   the delta correction), and "Chunkwise algorithm" (the exact chunk
 *   regrouping that the prefill kernels use);
 *   "Beyond attention" — "Three ways to update the state".
 *
 * Per (batch b, head h), for t = 1..T, row-vector convention (q_t, k_t are
 * 1 x dk, v_t is 1 x dv, S is dk x dv; key channel i is row i of S):
 *   a_t = exp(g_t)                       (g is the log of the forget gate)
 *   S'  = S_{t-1}                        LINATTN_GATE_NONE
 *       = a_t S_{t-1}                    LINATTN_GATE_SCALAR  (one g per token)
 *       = Diag(a_t) S_{t-1}              LINATTN_GATE_CHANNEL (one g per token and key channel)
 *   LINATTN_RULE_ADD  : S_t = S' + k_t^T v_t
 *   LINATTN_RULE_DELTA: S_t = S' + k_t^T beta_t (v_t - k_t S')
 *   o_t = q_t S_t                        (after the write; no query scale, no normaliser)
 *
 * Conventions shared by every entry point
 *   - Tensor pointers are DEVICE pointers to contiguous row-major arrays; the
 *     caller allocates and owns every buffer.  The library never allocates,
 *     frees or keeps device memory, and holds no mutable global state.
 *   - Token tensors (q, k, v, g, beta, o) share one dtype (linattn_dtype); the
 *     state is always fp32.  Every pointer must be 16-byte aligned.
 *   - Calls only validate arguments and enqueue kernels on `stream` (a
 *     hipStream_t; NULL = the default stream); they return before the work
 *     finishes.  Device faults surface at the caller's next synchronisation.
 *   - A nonzero status means nothing was enqueued (argument errors are found
 *     before any launch) or, for LINATTN_ERR_LAUNCH, that a launch failed.
 *   - Thread-safe for distinct buffers; no exception crosses the ABI.
 */
#ifndef LINATTN_H
#define LINATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define LINATTN_ABI_VERSION 1

typedef enum {
    LINATTN_OK = 0,
    LINATTN_ERR_NULL = 1,        /* a required pointer is NULL */
    LINATTN_ERR_SHAPE = 2,       /* negative or overflowing sizes */
    LINATTN_ERR_UNSUPPORTED = 3, /* valid but not built: head size, chunk, dtype, alignment */
    LINATTN_ERR_WORKSPACE = 4,   /* workspace missing or smaller than required */
    LINATTN_ERR_LAUNCH = 5,      /* the HIP runtime refused a launch */
    LINATTN_ERR_ARG = 6          /* inconsistent arguments (rule/gate/pointer mismatch) */
} linattn_status;

typedef enum { LINATTN_RULE_ADD = 0, LINATTN_RULE_DELTA = 1 } linattn_rule;
typedef enum { LINATTN_GATE_NONE = 0, LINATTN_GATE_SCALAR = 1, LINATTN_GATE_CHANNEL = 2 } linattn_gate;
typedef enum { LINATTN_F32 = 0, LINATTN_BF16 = 1 } linattn_dtype;

/* Chunk-forward problem description.  rule/gate/dtype hold the enum values. */
typedef struct {
    int64_t B, H, T;   /* batch, heads, tokens per sequence (T >= 0) */
    int32_t dk, dv;    /* key and value head sizes */
    int32_t chunk;     /* tokens per chunk C; 0 selects the default (64) */
    int32_t rule, gate, dtype;
} linattn_chunk_args;

/* Decode problem description: N sequences x H heads, one token each. */
typedef struct {
    int64_t N, H;
    int32_t dk, dv;
    int32_t rule, gate, dtype;
} linattn_decode_args;

/* ABI version the library was built with (LINATTN_ABI_VERSION). */
int linattn_abi_version(void);

/* Static description of a status code; never NULL. */
const char *linattn_status_string(int status);

/*
 * Device workspace, in bytes, that linattn_chunk_fwd needs for this problem:
 * 0 when the single-pass kernel serves it, else the size of the per-chunk
 * operand tiles the two-kernel path stages in HBM.  Returns 0 for invalid
 * arguments as well (linattn_chunk_fwd reports those).
 */
size_t linattn_chunk_workspace_bytes(const linattn_chunk_args *a);

/*
 * Chunkwise-parallel forward over whole sequences (prefill / training
 * forward).  "Linear Attention, Visualized", "Chunkwise algorithm": within a
 * chunk the parallel (masked, decay-weighted) form, between chunks the state
 * recurrence; for the delta rule the per-chunk triangular system
 * (I + diag(beta) L) is solved once ("Optional: Use UT to share the triangular
 * transform") and the incoming state corrects the chunk's writes ("Correct the
 * incoming state").  The result equals the token recurrence above up to
 * rounding for every chunk size.
 *
 *   q, k     [B,H,T,dk]              token dtype
 *   v        [B,H,T,dv]              token dtype
 *   g        [B,H,T] (SCALAR) | [B,H,T,dk] (CHANNEL) | NULL (NONE); log-gate, token dtype
 *   beta     [B,H,T] (DELTA) | NULL (ADD); token dtype
 *   s0       [B,H,dk,dv] fp32 initial state, or NULL for zero
 *   o        [B,H,T,dv] output, token dtype (fp32 accumulation)
 *   s_final  [B,H,dk,dv] fp32 final state, or NULL; may alias s0 exactly
 *   workspace, workspace_bytes: device scratch of at least
 *            linattn_chunk_workspace_bytes(a) bytes (may be NULL when that is 0)
 *   stream   hipStream_t
 * Supported: dk, dv in {64, 128}; chunk in {16, 32, 64, 128} (0 = 64); bf16
 * or fp32 tokens; every rule and gate; one head's output under 2 GiB
 * (T * dv * element size < 2^31, else LINATTN_ERR_UNSUPPORTED).  T need not
 * be a multiple of the chunk size.  Chunk 64 with bf16 tokens (and fp32
 * tokens at dk = 64 without the per-channel gate) runs the tuned kernels;
 * other chunk sizes, fp32 tokens at dk = 128 and fp32 tokens with the
 * per-channel gate run a generic two-kernel path; both need the workspace
 * linattn_chunk_workspace_bytes reports (0 for the single-pass kernels).
 */
linattn_status linattn_chunk_fwd(const linattn_chunk_args *a,
                                 const void *q, const void *k, const void *v,
                                 const void *g, const void *beta,
                                 const float *s0, void *o, float *s_final,
                                 void *workspace, size_t workspace_bytes, void *stream);

/* Input preparation from raw projections, fused into the chunk forward
 * (linattn_chunk_fwd_prep): "All sorts of famous Attention Layers", "DeltaNet"
 * (keys and queries L2-normalised per token, x / max(|x|, 1e-6); beta a
 * sigmoid) and "Linear Magic" (the positive feature map elu(x) + 1); "Linear
 * Attention, Visualized", "Mamba-2" / "Gated DeltaNet (GDN)" (forget gate
 * exp(-softplus(x)) in (0, 1), i.e. log-gate -softplus(x)).  The maps run in
 * fp32 on the raw values as the kernel stages them; the prepared q and k are
 * then rounded to the token dtype once. */
typedef enum { LINATTN_QK_AS_IS = 0, LINATTN_QK_L2 = 1, LINATTN_QK_ELU1 = 2 } linattn_qk_map;
typedef enum { LINATTN_GMAP_AS_IS = 0, LINATTN_GMAP_NEG_SOFTPLUS = 1 } linattn_gate_map;
typedef enum { LINATTN_BMAP_AS_IS = 0, LINATTN_BMAP_SIGMOID = 1 } linattn_beta_map;
typedef struct {
    int32_t qk_map;     /* applied to q and to k (linattn_qk_map) */
    int32_t gate_map;   /* linattn_gate_map; needs a gate (scalar or per channel) */
    int32_t beta_map;   /* linattn_beta_map; needs the delta rule */
} linattn_prep_args;

/*
 * linattn_chunk_fwd with q, k, g and beta given as raw projections and mapped
 * inside the kernel as prep says (NULL prep: no maps, same as
 * linattn_chunk_fwd).  A map the problem has no operand for (a gate map without
 * a gate, a beta map for the add rule) or an unknown map value is
 * LINATTN_ERR_ARG.  Every path applies the maps (the per-channel gate map
 * element by element, -softplus of each key channel's logit).  Same
 * arguments, layouts and workspace as linattn_chunk_fwd otherwise.
 */
linattn_status linattn_chunk_fwd_prep(const linattn_chunk_args *a, const linattn_prep_args *prep,
                                      const void *q, const void *k, const void *v,
                                      const void *g, const void *beta,
                                      const float *s0, void *o, float *s_final,
                                      void *workspace, size_t workspace_bytes, void *stream);

/*
 * Device workspace, in bytes, that linattn_chunk_fwd_normalized needs (a block
 * of ones, the denominator pass's output and states, and the chunk path's
 * workspace); 0 for invalid arguments.
 */
size_t linattn_normalized_workspace_bytes(const linattn_chunk_args *a);

/*
 * Normalised linear attention ("All sorts of famous Attention Layers",
 * "Linear Magic" and its normaliser): the add rule (a->rule must be
 * LINATTN_RULE_ADD, else LINATTN_ERR_ARG) with a second state z_t = a_t
 * z_{t-1} + k_t (the decayed running sum of the keys; Diag(a_t) for the
 * channel gate) and the read-out o_t = (q_t S_t) / (q_t . z_t).  The
 * denominator is only well defined for positive feature maps (elu + 1, e.g.
 * prep->qk_map = LINATTN_QK_ELU1 on raw projections).
 *
 *   q, k, v, g, s0, o, s_final: as for linattn_chunk_fwd_prep (no beta)
 *   z0       [B,H,dk] fp32 initial key sum, or NULL for zero
 *   z_final  [B,H,dk] fp32 final key sum, or NULL; may alias z0 exactly (the
 *            key sum carried in place), a partial overlap is LINATTN_ERR_ARG
 *   workspace: at least linattn_normalized_workspace_bytes(a) bytes,
 *            16-byte aligned; always required (the per-channel gate runs a
 *            second, denominator pass that writes to it; no gate and the
 *            scalar gate run one pass that carries z beside S and use it only
 *            to hold a copy of z0 when z_final aliases it)
 */
linattn_status linattn_chunk_fwd_normalized(const linattn_chunk_args *a, const linattn_prep_args *prep,
                                            const void *q, const void *k, const void *v,
                                            const void *g, const float *s0, const float *z0,
                                            void *o, float *s_final, float *z_final,
                                            void *workspace, size_t workspace_bytes, void *stream);

/* Gated DeltaProduct problem description: n_h delta-rule substeps per token.
 * gate holds LINATTN_GATE_NONE or LINATTN_GATE_SCALAR; dtype as above. */
typedef struct {
    int64_t B, H, T;   /* batch, heads, tokens per sequence (T >= 0) */
    int32_t nh;        /* substeps per token (>= 1) */
    int32_t dk, dv;    /* key and value head sizes */
    int32_t chunk;     /* tokens per chunk of the virtual sequence; 0 = 64 */
    int32_t gate, dtype;
} linattn_deltaproduct_args;

/*
 * Device workspace, in bytes, that linattn_deltaproduct_fwd needs: for n_h > 1
 * the expanded queries and log-gates and the n_h T virtual outputs (plus what
 * the chunk path needs for them); for n_h = 1 what linattn_chunk_fwd needs.
 * Returns 0 for invalid arguments as well.
 */
size_t linattn_deltaproduct_workspace_bytes(const linattn_deltaproduct_args *a);

/*
 * Gated DeltaProduct forward ("Linear Attention, Visualized", "Gated Delta
 * Product (GDP)"): token t decays the state once by a_t = exp(g_t), then
 * applies n_h delta-rule substeps in order, substep j with key k_{t,j}, value
 * v_{t,j} and correction gate beta_{t,j}; the query reads the state after the
 * last substep.  Computed as Gated DeltaNet over the virtual sequence of n_h T
 * steps ("GDP as GDN over a virtual sequence") by the chunk kernels.
 *
 *   q        [B,H,T,dk]              token dtype
 *   k        [B,H,T,nh,dk]           token dtype
 *   v        [B,H,T,nh,dv]           token dtype
 *   g        [B,H,T] (SCALAR) | NULL (NONE); log-gate, token dtype
 *   beta     [B,H,T,nh]              token dtype
 *   s0, o, s_final, stream: as for linattn_chunk_fwd
 *   workspace, workspace_bytes: at least
 *            linattn_deltaproduct_workspace_bytes(a) bytes, 16-byte aligned
 * Supported: as linattn_chunk_fwd for the delta rule with the virtual length
 * n_h T (so one head's virtual output must stay under 2 GiB); the channel
 * gate is not supported (LINATTN_ERR_UNSUPPORTED).
 */
linattn_status linattn_deltaproduct_fwd(const linattn_deltaproduct_args *a,
                                        const void *q, const void *k, const void *v,
                                        const void *g, const void *beta,
                                        const float *s0, void *o, float *s_final,
                                        void *workspace, size_t workspace_bytes, void *stream);

/*
 * Chunk forward that also keeps, for the backward pass, the state entering
 * every chunk ("Linear Attention, Visualized", "Update the state": in the
 * chunkwise form autograd keeps one boundary state per chunk instead of one
 * state per token).  Same arguments and results as
 * linattn_chunk_fwd, plus
 *   states   [B,H,N,dk,dv] in the token dtype, N = ceil(T / 64):
 *            states[b,h,r] is the state before chunk r (states[b,h,0] = s0,
 *            or zero), rounded once from the fp32 state the forward carries
 *            (the backward uses it as matrix-core operands of that dtype);
 *            caller-owned.
 *   workspace: at least linattn_chunk_workspace_bytes(a) bytes, 16-byte
 *            aligned, for the per-channel gate (the two-kernel path's staged
 *            chunk operands); not read otherwise (NULL allowed).
 * Supported: chunk 64; bf16 tokens with dk, dv in {64, 128} (every gate);
 * fp32 tokens with dk = 64 and dv in {64, 128}, gate NONE or SCALAR
 * (LINATTN_ERR_UNSUPPORTED otherwise); the same 2 GiB limit.
 */
linattn_status linattn_chunk_fwd_save(const linattn_chunk_args *a,
                                      const void *q, const void *k, const void *v,
                                      const void *g, const void *beta,
                                      const float *s0, void *o, float *s_final,
                                      void *states, void *workspace, size_t workspace_bytes,
                                      void *stream);

/*
 * Device workspace, in bytes, of linattn_chunk_bwd: the per-chunk operands of
 * its reverse state pass and the gradients of every chunk's outgoing state,
 * plus, when states_given is 0, room for the recomputed chunk states and a
 * forward output.  0 for invalid or unsupported arguments.
 */
size_t linattn_chunk_bwd_workspace_bytes(const linattn_chunk_args *a, int states_given);

/*
 * Backward pass of the chunkwise forward: the gradients of a loss with
 * respect to q, k, v, g, beta and s0, given its gradients with respect to
 * every output (dout) and the final state (dsT).  "Linear Attention,
 * Visualized", "Update the state" (the chunk form is how these layers train,
 * saving one state per chunk for the backward pass) and "Beyond attention",
 * "Chunkwise parallel training", with the per-chunk quantities of "Linear Attention, Visualized", "Chunkwise
 * algorithm", the GDN table and "The triangular correction system"
 * differentiated: a reverse pass over the chunks carries the gradient of the
 * state, and every chunk's gradients then follow from its incoming state and
 * the gradient of its outgoing state.
 *
 *   q, k, v, g, beta, s0: the forward's inputs (as linattn_chunk_fwd)
 *   states   [B,H,N,dk,dv] from linattn_chunk_fwd_save, or NULL to
 *            recompute them (then s0 is read; with states given it is not)
 *   dout     [B,H,T,dv] token dtype
 *   dsT      [B,H,dk,dv] fp32, or NULL for zero
 *   dq, dk   [B,H,T,dk] token dtype (written)
 *   dv       [B,H,T,dv] token dtype (written)
 *   dg       [B,H,T] token dtype for the SCALAR gate, [B,H,T,dk] for the
 *            CHANNEL gate, NULL for NONE (written)
 *   dbeta    [B,H,T] token dtype for DELTA, NULL for ADD (written)
 *   ds0      [B,H,dk,dv] fp32, or NULL (written)
 *   workspace: at least linattn_chunk_bwd_workspace_bytes(a, states != NULL)
 *            bytes, 16-byte aligned
 * Supported: as linattn_chunk_fwd_save.  For the CHANNEL gate ("Gated
 * Linear Attention (GLA)" and "Kimi Delta Attention (KDA)" on the same page:
 * the decay is diagonal, one factor per key channel) the per-channel decay
 * stays inside every score's sum over key channels, and dg is per channel.
 * Accumulation is fp32; matrix-core operands are in the token dtype.  Inputs are not normalised or mapped here:
 * these are the gradients with respect to the values the kernels received.
 */
linattn_status linattn_chunk_bwd(const linattn_chunk_args *a,
                                 const void *q, const void *k, const void *v,
                                 const void *g, const void *beta, const float *s0,
                                 const void *states, const void *dout, const float *dsT,
                                 void *dq, void *dk, void *dv, void *dg, void *dbeta,
                                 float *ds0, void *workspace, size_t workspace_bytes,
                                 void *stream);

/*
 * Device workspace, in bytes, of linattn_deltaproduct_bwd (the expanded
 * queries and gates, the virtual dO, dq and dg, and linattn_chunk_bwd's
 * workspace for the virtual sequence); 0 for invalid or unsupported arguments.
 */
size_t linattn_deltaproduct_bwd_workspace_bytes(const linattn_deltaproduct_args *a);

/*
 * Backward pass of Gated DeltaProduct ("Linear Attention, Visualized", "Gated
 * Delta Product (GDP)"): the gradients with respect to q, k, v, g, beta and s0
 * given dout and dsT, computed as the Gated DeltaNet backward over the
 * virtual sequence ("GDP as GDN over a virtual sequence": the query on the
 * last substep of each token, the gate on the first), so dk, dv and dbeta come
 * out in the [B,H,T,nh,...] layout and dq, dg are the virtual ones at those
 * substeps.  The forward's states are recomputed.
 *
 *   q, k, v, g, beta, s0: as linattn_deltaproduct_fwd
 *   dout     [B,H,T,dv] token dtype;  dsT [B,H,dk,dv] fp32 or NULL
 *   dq [B,H,T,dk], dk [B,H,T,nh,dk], dv [B,H,T,nh,dv], dg [B,H,T] (SCALAR gate,
 *   else NULL), dbeta [B,H,T,nh]: token dtype;  ds0 [B,H,dk,dv] fp32 or NULL
 *   workspace: at least linattn_deltaproduct_bwd_workspace_bytes(a) bytes,
 *            16-byte aligned
 * Supported: as linattn_chunk_bwd for the virtual length n_h T.
 */
linattn_status linattn_deltaproduct_bwd(const linattn_deltaproduct_args *a,
                                        const void *q, const void *k, const void *v,
                                        const void *g, const void *beta, const float *s0,
                                        const void *dout, const float *dsT,
                                        void *dq, void *dk, void *dv, void *dg, void *dbeta,
                                        float *ds0, void *workspace, size_t workspace_bytes,
                                        void *stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc):
 * linattn_chunk_fwd_prep without a workspace argument.  Where the chosen path
 * stages per-chunk operands (the per-channel gate, chunk sizes other than 64,
 * fp32 tokens at dk = 128 or with the per-channel gate) they go to a static
 * device array of LINATTN_NOALLOC_SCRATCH_BYTES owned by the library, one per
 * GPU, held until the process ends; its address is looked up once per device
 * (the device current at the call, which must own `stream`).  The call makes
 * no allocation.  Problems whose workspace (linattn_chunk_workspace_bytes)
 * exceeds the array return LINATTN_ERR_WORKSPACE before anything is enqueued.
 * Every call on one GPU shares that GPU's array: calls that overlap in time on
 * one GPU (different streams, or threads) race and must be serialised by the
 * caller.  The array needs no clearing between calls (every byte a call reads
 * was written by the same call).  Arguments otherwise as
 * linattn_chunk_fwd_prep (prep may be NULL).
 */
#define LINATTN_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
linattn_status linattn_chunk_fwd_noalloc(const linattn_chunk_args *a, const linattn_prep_args *prep,
                                         const void *q, const void *k, const void *v,
                                         const void *g, const void *beta,
                                         const float *s0, void *o, float *s_final, void *stream);

/*
 * One recurrent decode step for N sequences x H heads, updating the state in
 * place ("Linear Attention, Visualized", "Optional: Linear attention as an
 * RNN" and the DeltaNet recurrent form; "All sorts of famous Attention
 * Layers", "DeltaNet": read at the key, write the beta-scaled difference, then
 * read with the query).  Memory-bound: each state is read and written once.
 *
 *   q, k   [N,H,dk]                 token dtype
 *   v      [N,H,dv]                 token dtype
 *   g      [N,H] | [N,H,dk] | NULL  log-gate (SCALAR | CHANNEL | NONE)
 *   beta   [N,H] | NULL             (DELTA | ADD)
 *   state  [N,H,dk,dv] fp32, read and overwritten in place
 *   o      [N,H,dv] token dtype
 * Supported: dk, dv in {64, 128}; bf16 or fp32 tokens; every rule and gate.
 */
linattn_status linattn_decode_step(const linattn_decode_args *a,
                                   const void *q, const void *k, const void *v,
                                   const void *g, const void *beta,
                                   float *state, void *o, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* LINATTN_H */
