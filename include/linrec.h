/*
 * linrec.h -- C ABI of the MI355X (gfx950) chunkwise linear-recurrence layer.
 *
 * The layer (per batch b and head h, one sub-sequence of T tokens):
 *
 *     S_0 = S_in,   S_t = a_t S_{t-1} + k_t^T v_t,   o_t = q_t S_t,   S_out = S_T
 *
 * with a d_k x d_v state per head.  A long sequence is processed as a chain
 * of sub-sequences: S_out of one piece is S_in of the next, and in the
 * backward pass dS_in of one piece is dS_out of the previous one, so any
 * split gives the result of one pass over the whole sequence.  Sources: the
 * d x d memory state accumulated over sub-sequences processed one after
 * another, with the backward pass over stored states (Sequence Accumulation
 * and Beyond, "Approach"); boundary states and gradients propagated across
 * chunks (StateFlow, Abstract; the gptget summary's method details: a linear
 * recurrence kernel inside each chunk, chunks joined by boundary states);
 * the right-product form of linear attention with cached intermediate
 * states (Linear Attention Sequence Parallelism, abstract).
 *
 * Inside a piece the work is done chunkwise with C = 64 tokens per chunk,
 * chunks grouped into segments of 4:
 *   - the state transition (a parallel segment-sum kernel and a serial fold
 *     kernel) carries S across the piece in fp32 and stores the state
 *     entering every segment ("states");
 *   - a segment kernel walks each segment's chunks with the state in
 *     registers and computes, per chunk,
 *         O_n = [(Q_n K_n^T) .* D_n] V_n + (Q_n .* gamma) S_{n-1}
 *     where gamma_i is the chunk-local cumulative decay of token i and
 *     D_ij = gamma_i / gamma_j for j <= i (0 above the diagonal).
 *   The backward mirrors this: the reverse transition carries dS from
 *   dS_out back to dS_in and stores the gradient leaving every segment; a
 *   segment kernel rebuilds the per-chunk states and gradients from the
 *   stored ones and computes dQ, dK, dV.
 *
 * ---------------------------------------------------------------- layouts
 *   Activations q, k (d_k wide), v, o, dO, dq, dk, dv (d_v or d_k wide) are
 *   [B, H, T, d] with element strides (sb, sh, st); the feature index is
 *   contiguous (stride 1).  A piece of a longer tensor is passed as a
 *   strided view (pointer advanced to the piece's first token), no copy.
 *   decay:  LINREC_DECAY_NONE  -> a_t = 1, decay.ptr ignored;
 *           LINREC_DECAY_HEAD  -> fp32 [H] (a_h itself, not its log), element
 *                                 stride decay.sh (sb, st ignored);
 *           LINREC_DECAY_TOKEN -> fp32 [B, H, T] with strides (sb, sh, st).
 *           Values must lie in (0, 1].
 *   S_in, S_out, dS_out, dS_in: contiguous fp32 [B, H, d_k, d_v].
 *   states: opaque, linrec_states_bytes() bytes, 16-byte aligned.
 *   workspace: opaque, linrec_bwd_workspace_bytes() bytes, 16-byte aligned.
 *
 * ---------------------------------------------------------------- dtypes
 *   dtype (inputs q, k, v, dO):
 *     LINREC_BF16: products run on bf16 MFMA with fp32 accumulation.  Every
 *                  operand the kernels compute (the masked score matrix, the
 *                  decay-scaled keys/queries, the carried state) enters the
 *                  MFMA as a hi + lo pair of bf16 values, so its rounding
 *                  costs ~2^-17 rather than 2^-9 of relative accuracy.
 *     LINREC_F32:  fp32 MFMA; only d_k = d_v = 64.
 *   out_dtype (outputs o, dq, dk, dv): LINREC_BF16 (round to nearest even
 *     from the fp32 result) or LINREC_F32; must be LINREC_F32 when dtype is.
 *   S_*, dS_*, decay, the per-chunk state store and the workspace are fp32.
 *
 * ---------------------------------------------------------------- shapes
 *   chunk == 64; 0 <= T <= LINREC_MAX_T (the last chunk of a piece may be
 *   partial: its missing tokens are neither read nor written; the
 *   delta-rule buffers count it whole); d_k, d_v in {64, 128};
 *   1 <= B <= 32767, 1 <= H <= 65535.  Offsets into every tensor are 64-bit, so a tensor
 *   may hold more than 2^31 elements (one head's T * d included).  Activation
 *   pointers and their strides sb, sh, st must keep every token row 16-byte
 *   aligned.
 *   T == 0 (per-piece calls only; every piece of a sequence call has at
 *   least one token): the piece is empty and the recurrence is the
 *   identity on its carry, so the call copies S_in to S_out (dS_out to
 *   dS_in, da_carry_in to da_carry_out; zeros for a NULL input) on `stream`
 *   and nothing else.  Activations, decay, beta, states, saved and the
 *   workspace are then not read, written or checked and may be NULL; the
 *   size functions return 0 for them.
 *
 * ---------------------------------------------------------------- semantics
 *   Ownership: the caller owns all device memory; the library keeps no
 *   pointer after a call returns and allocates no device memory (a context
 *   owns one auxiliary HIP stream and a few events).
 *   Ordering: work is enqueued on `stream` (a hipStream_t; NULL is the null
 *   stream) and the call returns at once.  Inputs must be ready on `stream`;
 *   outputs are ready on `stream` when it reaches the call's end.
 *   Errors: every argument is checked on the host before anything is
 *   enqueued; on error nothing runs and no output is touched.  A failed
 *   launch returns LINREC_E_LAUNCH (linrec_last_hip_error() gives the HIP
 *   code).  Faults inside kernels surface at the caller's next
 *   synchronisation.  Nothing is printed and no exception crosses the ABI.
 *   Aliasing: S_out may equal S_in and dS_in may equal dS_out (the carry
 *   loop's natural form).  Any other overlap between an output and any
 *   argument is undefined.
 *   Threads: a context is used by one host thread at a time.
 */
#ifndef LINREC_H
#define LINREC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* The library is built with hidden visibility: the functions declared here
 * are its only exports. */
#pragma GCC visibility push(default)

typedef enum {
    LINREC_OK = 0,
    LINREC_E_NULL = 1,      /* a required pointer is NULL                     */
    LINREC_E_SHAPE = 2,     /* unsupported B, H, T, d_k, d_v, chunk or pieces  */
    LINREC_E_DTYPE = 3,     /* unknown dtype, or dtype/shape combination      */
    LINREC_E_LAYOUT = 4,    /* unsupported strides or decay kind              */
    LINREC_E_ALIGN = 5,     /* a pointer or stride breaks 16-byte row alignment */
    LINREC_E_WORKSPACE = 6, /* states/workspace pointer missing or misaligned */
    LINREC_E_DEVICE = 7,    /* HIP runtime error outside a launch             */
    LINREC_E_LAUNCH = 8,    /* a kernel launch failed                         */
    LINREC_E_SCRATCH = 9    /* the call needs more than the fixed scratch of
                               linrec_bwd_noalloc                             */
} linrec_status;

typedef enum { LINREC_BF16 = 0, LINREC_F32 = 1 } linrec_dtype;

typedef enum {
    LINREC_DECAY_NONE = 0,
    LINREC_DECAY_HEAD = 1,
    LINREC_DECAY_TOKEN = 2
} linrec_decay_kind;

/* A device tensor: base pointer and element strides over (b, h, t). */
typedef struct {
    void* ptr;
    int64_t sb, sh, st;
} linrec_tensor;

/* Largest T of a call (2^31 - 4096): token counts, rounded up to whole
 * chunks and segments, stay within int32_t. */
#define LINREC_MAX_T 2147479552

/* Problem description of one call (T = tokens of this piece or sequence). */
typedef struct {
    int32_t B, H, T, dk, dv;
    int32_t chunk;            /* must be 64 */
    int32_t dtype;            /* linrec_dtype of q, k, v, dO */
    int32_t decay;            /* linrec_decay_kind */
    int32_t out_dtype;        /* linrec_dtype of o, dq, dk, dv */
} linrec_desc;

typedef struct linrec_ctx linrec_ctx;

/* Create a context on HIP device `device` (owns an auxiliary stream, created
 * at default priority, and events).  *out is set only on success. */
linrec_status linrec_ctx_create(linrec_ctx** out, int device);
/* Destroy a context; waits for its auxiliary stream.  NULL is a no-op. */
linrec_status linrec_ctx_destroy(linrec_ctx* ctx);

/* Bytes of the state store of one piece described by `d` (0 if `d` is
 * invalid): B*H*ceil(T/256) records of d_k*d_v + 64 fp32 values, the state
 * entering every segment of 4 chunks (row-major [d_k][d_v], as S_in) and the
 * segment's log-decay, written by
 * linrec_fwd and read by linrec_bwd.  It depends on the piece length only
 * (constant in the number of pieces already processed). */
size_t linrec_states_bytes(const linrec_desc* d);

/* Bytes of backward workspace for `d` (0 if `d` is invalid): the gradient
 * leaving every segment, B*H*ceil(T/256) records as above. */
size_t linrec_bwd_workspace_bytes(const linrec_desc* d);

/* Bytes of the state store linrec_fwd_seq / linrec_bwd_seq need for these
 * pieces of the sequence `d` (the sum of the pieces' own stores; 0 if the
 * arguments are invalid). */
size_t linrec_seq_states_bytes(const linrec_desc* d, int32_t npieces, const int32_t* lengths);

/* Forward over one piece.
 *   q, k: [B,H,T,d_k];  v, o: [B,H,T,d_v];  decay per d->decay.
 *   S_in: fp32 [B,H,d_k,d_v] or NULL (zeros).  S_out: fp32, required.
 *   states: required (linrec_states_bytes(d) bytes); pass it unmodified to
 *   linrec_bwd for the same piece.  The forward itself runs through it (the
 *   state entering every 256-token segment is formed there, then read by
 *   the output kernel), so a forward-only caller passes it too and may
 *   reuse one buffer for every piece.
 * Reference: the recurrence above (Sequence Accumulation and Beyond,
 * "Approach"; StateFlow, Abstract). */
linrec_status linrec_fwd(linrec_ctx* ctx, const linrec_desc* d,
                         linrec_tensor q, linrec_tensor k, linrec_tensor v,
                         linrec_tensor decay, const float* S_in,
                         linrec_tensor o, float* S_out, void* states,
                         void* stream);

/* Backward over one piece, for the loss L = <dO, o> + <dS_out, S_out>.
 *   states: as written by linrec_fwd for this piece (it holds S_in).
 *   dO: [B,H,T,d_v].  dS_out: fp32 [B,H,d_k,d_v] or NULL (zeros).
 *   dq, dk: [B,H,T,d_k], dv: [B,H,T,d_v], dS_in: fp32; all required.
 *   workspace: linrec_bwd_workspace_bytes(d) bytes.
 * The decay is not differentiated (it is an input, not a parameter).
 * Reference: boundary gradients propagated across chunks (StateFlow,
 * Abstract); backward pass over stored states (Sequence Accumulation and
 * Beyond, "Approach"). */
linrec_status linrec_bwd(linrec_ctx* ctx, const linrec_desc* d,
                         linrec_tensor q, linrec_tensor k, linrec_tensor v,
                         linrec_tensor decay, const void* states,
                         linrec_tensor dO, const float* dS_out,
                         linrec_tensor dq, linrec_tensor dk, linrec_tensor dv,
                         float* dS_in, void* workspace, void* stream);

/* Size of the fixed device scratch linrec_bwd_noalloc works in. */
#define LINREC_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)

/* linrec_bwd without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  The gradient records linrec_bwd keeps
 * in its workspace live instead in a static device array of
 * LINREC_NOALLOC_SCRATCH_BYTES (32 MiB) that the library holds on every GPU
 * it runs on until the process ends; nothing is allocated or freed by the
 * call.  Arguments, results and rules are those of linrec_bwd (results equal
 * linrec_bwd's bit for bit).  A piece whose workspace
 * (linrec_bwd_workspace_bytes(d)) exceeds the scratch is rejected with
 * LINREC_E_SCRATCH before anything is enqueued; e.g. B*H = 16 heads of
 * d_k = d_v = 128 fit pieces of up to 7936 tokens.  Every call on one GPU
 * shares that GPU's scratch: calls that may run concurrently on one GPU
 * (different streams, different threads) race and must be serialised by the
 * caller.  The scratch is written before it is read within each call, so it
 * needs no clearing between calls. */
linrec_status linrec_bwd_noalloc(linrec_ctx* ctx, const linrec_desc* d,
                                 linrec_tensor q, linrec_tensor k, linrec_tensor v,
                                 linrec_tensor decay, const void* states,
                                 linrec_tensor dO, const float* dS_out,
                                 linrec_tensor dq, linrec_tensor dk, linrec_tensor dv,
                                 float* dS_in, void* stream);

/* Bytes of workspace linrec_bwd_recompute needs (0 if `d` is invalid): the
 * piece's rebuilt state records, its gradient records and one fp32 state
 * of scratch, 2 * linrec_states_bytes(d) + B*H*d_k*d_v*4.  It depends on
 * the piece length only. */
size_t linrec_bwd_recompute_workspace_bytes(const linrec_desc* d);

/* Backward over one piece without states kept from the forward: the states
 * entering every segment are rebuilt from S_in, the boundary state the
 * piece's forward started from, by the forward state transition (one more
 * read of k and v), then the backward runs as linrec_bwd.  A caller of the
 * sequence accumulation then keeps one boundary state per piece instead of
 * the pieces' state records, so its memory does not grow with the sequence
 * (activation recomputation: the gptget summary of StateFlow, "Key
 * results"; constant memory in sequence length: Sequence Accumulation and
 * Beyond, "Key results").
 *   S_in: fp32 [B,H,d_k,d_v] or NULL (zeros).  Other arguments as
 *   linrec_bwd; workspace: linrec_bwd_recompute_workspace_bytes(d) bytes.
 * Results equal linrec_bwd's bit for bit. */
linrec_status linrec_bwd_recompute(linrec_ctx* ctx, const linrec_desc* d,
                                   linrec_tensor q, linrec_tensor k, linrec_tensor v,
                                   linrec_tensor decay, const float* S_in,
                                   linrec_tensor dO, const float* dS_out,
                                   linrec_tensor dq, linrec_tensor dk, linrec_tensor dv,
                                   float* dS_in, void* workspace, void* stream);

/* Bytes of workspace linrec_bwd_da needs (0 if `d` is invalid): the
 * gradient records of linrec_bwd plus one fp32 total per segment. */
size_t linrec_bwd_da_workspace_bytes(const linrec_desc* d);

/* linrec_bwd plus the gradient of the loss with respect to the decay, for
 * trained gates.  With g_t = q_t . dq_t - k_t . dk_t (the gradient with
 * respect to the cumulative log-decay at token t), the log-decay of token r
 * has gradient sum_{t >= r} g_t over the rest of the sequence, and
 *   da[r] = (sum_{t >= r in this piece} g_t + da_carry_in) / a_r.
 * da_carry_in is that sum over everything after the piece, which equals
 * <dS_out, S_out>: in a reverse loop over pieces it is the next piece's
 * da_carry_out, and after the last piece it is <dS_out, S_out> of the whole
 * sequence (0 when dS_out = 0).  NULL means 0.
 *   da: fp32 [B,H,T] (strides in elements, like a per-token decay), one
 *       value per token for per-token and per-head decay alike (the
 *       gradient of a per-head decay is the sum over tokens);
 *   da_carry_out: fp32 [B,H], required; may alias da_carry_in.
 *   d->decay must not be LINREC_DECAY_NONE (LINREC_E_LAYOUT).
 *   workspace: linrec_bwd_da_workspace_bytes(d) bytes.
 * dq, dk, dv and dS_in equal linrec_bwd's bit for bit.  g_t is formed from
 * the fp32 dq and dk before they are rounded to the output dtype.
 * Reference: gated (per-token) decay in the recurrences StateFlow trains
 * (the gptget summary, "Experimental design"). */
linrec_status linrec_bwd_da(linrec_ctx* ctx, const linrec_desc* d,
                            linrec_tensor q, linrec_tensor k, linrec_tensor v,
                            linrec_tensor decay, const void* states,
                            linrec_tensor dO, const float* dS_out,
                            linrec_tensor dq, linrec_tensor dk, linrec_tensor dv,
                            float* dS_in, linrec_tensor da, const float* da_carry_in,
                            float* da_carry_out, void* workspace, void* stream);

/* Sequence accumulation over `npieces` consecutive pieces of the sequence
 * described by `d` (d->T = total tokens; lengths[i] >= 1, sum = T;
 * lengths is host memory).  Piece i is processed as its own sub-sequence,
 * in order, with S carried from piece to piece; the state-transition
 * kernels run on the context's auxiliary stream so that piece i+1's state
 * transition overlaps piece i's intra-chunk work (state transitions with
 * limited parallelism overlapped with surrounding computation: StateFlow,
 * Abstract).  `states` covers the whole sequence
 * (linrec_seq_states_bytes() bytes).  Same arguments and rules as
 * linrec_fwd otherwise. */
linrec_status linrec_fwd_seq(linrec_ctx* ctx, const linrec_desc* d,
                             int32_t npieces, const int32_t* lengths,
                             linrec_tensor q, linrec_tensor k, linrec_tensor v,
                             linrec_tensor decay, const float* S_in,
                             linrec_tensor o, float* S_out, void* states,
                             void* stream);

/* Bytes of workspace linrec_bwd_seq needs for these pieces (0 if invalid):
 * three slots, each holding the gradient records of the longest piece. */
size_t linrec_bwd_seq_workspace_bytes(const linrec_desc* d, int32_t npieces,
                                      const int32_t* lengths);

/* Backward of linrec_fwd_seq: pieces in reverse order with dS carried back
 * from dS_out to dS_in, each piece's backward running over the states its
 * forward stored (the backward pass over stored states of Sequence
 * Accumulation and Beyond, "Approach"; boundary gradients carried from piece
 * to piece: StateFlow, Abstract; state transitions overlapped with the
 * surrounding computation: StateFlow, Abstract).  Every launch goes to
 * `stream`, one per piece: piece i's segment-kernel launch also carries
 * piece i - 1's reverse fold (which needs piece i's dS_in) and piece
 * i - 2's segment sums, as extra work of the same grid (a transition kernel
 * on a second stream could not share a CU with the segment kernel, whose
 * LDS fills it).  The gradient records of piece j live in workspace slot
 * j % 3.  Same arguments and rules as linrec_bwd otherwise; `states` as
 * written by linrec_fwd_seq. */
linrec_status linrec_bwd_seq(linrec_ctx* ctx, const linrec_desc* d,
                             int32_t npieces, const int32_t* lengths,
                             linrec_tensor q, linrec_tensor k, linrec_tensor v,
                             linrec_tensor decay, const void* states,
                             linrec_tensor dO, const float* dS_out,
                             linrec_tensor dq, linrec_tensor dk,
                             linrec_tensor dv, float* dS_in, void* workspace,
                             void* stream);

/* ------------------------------------------------------------ delta rule
 * The gated delta rule, per batch b and head h (one sub-sequence):
 *
 *   S_0 = S_in,  S_t = a_t (I - beta_t k_t^T k_t) S_{t-1} + beta_t k_t^T v_t,
 *   o_t = q_t S_t,  S_out = S_T
 *
 * the recurrence of the Gated DeltaNet models StateFlow trains (the gptget
 * summary, "Experimental design"), with the layer's d_k x d_v state.  The
 * erase term acts on the key dimension: with |k_t| = 1 and beta_t = 1 the
 * state read at k_t after the update is exactly v_t.  Pieces chain through
 * S_out -> S_in as for the linear recurrence.
 *
 * Chunkwise (64 tokens): per chunk, the new values U solve the unit
 * lower-triangular system (I + A) U = diag(beta) (V - diag(gamma) K S_0)
 * with A_ij = beta_i (gamma_i / gamma_j) k_i . k_j for j < i; a first kernel
 * forms T = (I + A)^{-1}, W_v = T diag(beta) V and W_k = T diag(beta gamma) K
 * for every chunk in parallel, a second carries S across the chunks (the
 * transition is S <- gamma_C S + K~^T (W_v - W_k S)), 16 state columns per
 * workgroup, and writes O = diag(gamma) Q S_0 + [(Q K^T) .* D] U.  Products
 * of two computed operands use bf16 hi + lo pairs on both sides; the state
 * is carried in fp32.
 */

/* Bytes of workspace linrec_delta_fwd needs (0 if `d` is invalid or
 * d_k != d_v): W_k and W_v of every token, then P = (Q K^T) .* D of every
 * chunk, then the chunk's decay tables (256 values), fp32,
 * B*H*T*(d_k + d_v + 64 + 4)*4. */
size_t linrec_delta_workspace_bytes(const linrec_desc* d);

/* Bytes linrec_delta_fwd writes to `saved` for the backward (0 if `d` is
 * invalid or d_k != d_v): the state entering every chunk, fp32
 * [B,H,T/64,d_k,d_v], then U of every token, fp32 [B,H,T,d_v]. */
size_t linrec_delta_saved_bytes(const linrec_desc* d);

/* Delta-rule forward over one piece.
 *   q, k: [B,H,T,d_k]; v, o: [B,H,T,d_v]; d_k == d_v (64 or 128; fp32 inputs
 *   only at 64).  beta: fp32 [B,H,T] with strides (sb, sh, st), values in
 *   [0, 1].  decay per d->decay (as linrec_fwd; the gate a_t).  S_in: fp32
 *   [B,H,d_k,d_v] or NULL (zeros).  S_out: fp32, required, may alias S_in.
 *   saved: NULL, or linrec_delta_saved_bytes(d) bytes (16-byte aligned) that
 *   the backward of this piece reads.
 *   workspace: linrec_delta_workspace_bytes(d) bytes, 16-byte aligned.
 * Errors and ownership as linrec_fwd. */
linrec_status linrec_delta_fwd(linrec_ctx* ctx, const linrec_desc* d,
                               linrec_tensor q, linrec_tensor k, linrec_tensor v,
                               linrec_tensor beta, linrec_tensor decay, const float* S_in,
                               linrec_tensor o, float* S_out, void* saved, void* workspace,
                               void* stream);

/* Bytes of workspace linrec_delta_bwd needs (0 if `d` is invalid or
 * d_k != d_v): W_k, W_v, per-chunk T (then the masked gradient of A),
 * dU (then T^T dU), the gradient leaving every chunk, per-chunk P and the
 * per-chunk decay tables (256 values), all fp32. */
size_t linrec_delta_bwd_workspace_bytes(const linrec_desc* d);

/* Delta-rule backward over one piece, for L = <dO, o> + <dS_out, S_out>:
 *   dU   = P^T dO + (K .* gamma_C/gamma) dS_C  and
 *   dS_0 = (Q .* gamma)^T dO + gamma_C dS_C - W_k^T dU  (carried across chunks,
 *   serially, 16 gradient columns per workgroup), then per chunk in parallel
 *   dV = beta .* (T^T dU), dbeta, dQ and dK through W = T R, T = (I + A)^-1,
 *   P = (Q K^T) .* D and the state update.  The gate is not differentiated.
 *   saved: as written by linrec_delta_fwd for this piece.  dO: [B,H,T,d_v];
 *   dS_out: fp32 [B,H,d_k,d_v] or NULL (zeros).  dq, dk, dv as linrec_bwd;
 *   dbeta: fp32 [B,H,T] (strides like beta); dS_in: fp32, required, may
 *   alias dS_out.  workspace: linrec_delta_bwd_workspace_bytes(d) bytes.
 * Errors and ownership as linrec_bwd. */
linrec_status linrec_delta_bwd(linrec_ctx* ctx, const linrec_desc* d,
                               linrec_tensor q, linrec_tensor k, linrec_tensor v,
                               linrec_tensor beta, linrec_tensor decay, const void* saved,
                               linrec_tensor dO, const float* dS_out, linrec_tensor dq,
                               linrec_tensor dk, linrec_tensor dv, linrec_tensor dbeta,
                               float* dS_in, void* workspace, void* stream);

/* Delta rule over a sequence of pieces (lengths[0..npieces), each >= 1,
 * summing to d->T), the state carried from piece to piece as through
 * linrec_delta_fwd / linrec_delta_bwd called once per piece in order (the
 * StateFlow pages train Gated DeltaNet with the state passed between the
 * sub-sequences of a long context: gptget summary, "Experimental design";
 * overlapping the state transitions with other work: Abstract).  The
 * results equal those of the per-piece calls bit for bit.  In the backward
 * the per-chunk gradient kernels of a piece, which need its serial walk but
 * nothing carried, run on the context's aux stream beside the next piece's
 * prep kernel and walk on the caller's stream.  Inputs and outputs span the
 * whole sequence, laid out as for the per-piece calls.
 *
 * saved: the per-piece saved buffers one after another, piece i's at the
 * sum of linrec_delta_saved_bytes over the pieces before it (a desc with
 * T = that piece's length); linrec_delta_seq_saved_bytes bytes in all,
 * 16-byte aligned.  Forward workspace: the per-piece workspace of the
 * longest piece; backward workspace: two such slots (one for a single
 * piece).  The size queries return 0 if `d`, `npieces` or `lengths` is
 * invalid or d_k != d_v. */
size_t linrec_delta_seq_saved_bytes(const linrec_desc* d, int32_t npieces, const int32_t* lengths);
size_t linrec_delta_fwd_seq_workspace_bytes(const linrec_desc* d, int32_t npieces,
                                            const int32_t* lengths);
size_t linrec_delta_bwd_seq_workspace_bytes(const linrec_desc* d, int32_t npieces,
                                            const int32_t* lengths);

/* Forward over the pieces: arguments as linrec_delta_fwd for the whole
 * sequence; S_in enters the first piece, S_out leaves the last.  saved may
 * be NULL (nothing kept for a backward). */
linrec_status linrec_delta_fwd_seq(linrec_ctx* ctx, const linrec_desc* d, int32_t npieces,
                                   const int32_t* lengths, linrec_tensor q, linrec_tensor k,
                                   linrec_tensor v, linrec_tensor beta, linrec_tensor decay,
                                   const float* S_in, linrec_tensor o, float* S_out, void* saved,
                                   void* workspace, void* stream);

/* Backward over the pieces in reverse: arguments as linrec_delta_bwd for the
 * whole sequence; saved as written by linrec_delta_fwd_seq with the same
 * lengths; dS_out enters the last piece, dS_in leaves the first. */
linrec_status linrec_delta_bwd_seq(linrec_ctx* ctx, const linrec_desc* d, int32_t npieces,
                                   const int32_t* lengths, linrec_tensor q, linrec_tensor k,
                                   linrec_tensor v, linrec_tensor beta, linrec_tensor decay,
                                   const void* saved, linrec_tensor dO, const float* dS_out,
                                   linrec_tensor dq, linrec_tensor dk, linrec_tensor dv,
                                   linrec_tensor dbeta, float* dS_in, void* workspace,
                                   void* stream);

/* Kernel kinds for linrec_ctx_kernel_times(). */
enum {
    LINREC_KERNEL_FWD_SUM = 0,    /* forward segment sums (parallel)           */
    LINREC_KERNEL_FWD_FOLD = 1,   /* forward fold across segments (S carried)  */
    LINREC_KERNEL_FWD_SEG = 2,    /* forward segment kernel: O                 */
    LINREC_KERNEL_BWD_SUM = 3,    /* reverse segment sums (parallel)           */
    LINREC_KERNEL_BWD_FOLD = 4,   /* reverse fold across segments (dS carried) */
    LINREC_KERNEL_BWD_SEG = 5,    /* backward segment kernel: dQ, dK, dV       */
    LINREC_KERNEL_DA_FINISH = 6,  /* decay gradient, last step                 */
    LINREC_KERNEL_DELTA_FWD = 7,  /* delta rule forward (each launch of a piece's kernels) */
    LINREC_KERNEL_DELTA_BWD = 8,  /* delta rule backward (each launch of a piece's kernels) */
    LINREC_KERNEL_KINDS = 9
};

/* Per-kernel timing (instrumentation, off by default).  While enabled, every
 * kernel the context launches is bracketed by two HIP events recorded on
 * the stream that kernel runs on.  Enabling or disabling resets the totals.
 * linrec_ctx_kernel_times() waits for the recorded launches, adds them to
 * the totals and returns the number of launches of `kind` and their summed
 * duration in milliseconds. */
linrec_status linrec_ctx_set_timing(linrec_ctx* ctx, int enable);
linrec_status linrec_ctx_kernel_times(linrec_ctx* ctx, int kind, int64_t* count, double* ms);

/* Human-readable name of a status code (static string, never NULL). */
const char* linrec_status_str(linrec_status s);

/* HIP error code of the most recent LINREC_E_DEVICE / LINREC_E_LAUNCH on
 * the calling thread (0 if none). */
int linrec_last_hip_error(void);

/* Library version, as major*10000 + minor*100 + patch. */
int linrec_version(void);

#pragma GCC visibility pop

#ifdef __cplusplus
}
#endif

#endif /* LINREC_H */
