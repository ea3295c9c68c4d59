/*
 * kda.h: C-ABI of the KDA (Kimi Delta Attention) mixer library for one
 * AMD Instinct MI355X (gfx950).
 *
 * The mixer, per sequence and head, keeps a recurrent state S (dk x dv,
 * rows = key channels) and, for every token:
 *   1. runs a depthwise causal short convolution (width 4, tap 3 on the
 *      current token, zero history before the first token, no bias, no
 *      activation) over the raw q, k and v channels;
 *   2. L2-normalises q and k: x / sqrt(|x|^2 + l2_eps) (q also times q_scale);
 *   3. decays the rows of S by alpha (one factor per key channel);
 *      alpha and beta arrive as values, or as logits a and b
 *      (kda_shape.gate_inputs), from which alpha = exp(-softplus(a)) and
 *      beta = sigmoid(b) are formed in the kernels;
 *   4. applies the gated delta-rule correction and write,
 *      S <- (I - beta k k^T) Diag(alpha) S + beta k v^T;
 *   5. reads out o = S^T q after the write;
 *   6. applies the gated RMSNorm over dv:
 *      y = norm_w * o / sqrt(mean(o^2) + norm_eps) * gate(g).
 * The recurrence always runs in FP32; the state may be stored as FP32 or
 * BF16 (round to nearest even, once per store).
 *
 * Sources: "Extend NVIDIA/TensorRT-LLM#19991 with isolated NVFP4 Kimi K3
 * targets" (fork pull request), Description: KDA fuses the convolution, the
 * FP32 recurrence and the gated output normalisation; recurrent-state storage
 * is FP32 or BF16; verify keeps FP32 per-token draft records under either
 * storage dtype and uses explicit FP32 loads and typed state stores.
 * "Kimi K3 on modeling_v2: stateful catalog entries, ..." section 1 (state
 * is a typed object the caller owns and passes in, made before any graph
 * capture; every written buffer is named), section 2 (lengths read on the
 * device so a captured call replays with inputs rewritten in place), section
 * 5 (per-token KDA verify states) and section 6 (KDA returns its output
 * before o_proj on every path).  The pages name the operation and its
 * properties; they print no formula, and the one above is the gated delta
 * rule in its usual statement.
 *
 * Conventions for every call:
 *   - All buffers are device pointers unless a comment says "host".
 *   - The library never allocates memory, never synchronises the host and
 *     reads no environment variable.  Every call is asynchronous on `stream`.
 *   - Host-detected errors (negative return codes) are found before any
 *     launch: nothing is written and the next call is unaffected.
 *   - Device-detected problems (a slot or accepted length out of range,
 *     non-monotone cu_seqlens, a negative position) skip the affected row or
 *     sequence and OR a KDA_STATUS_* bit into *status (nullable, device
 *     int32).  The caller clears *status when it wants a fresh report.
 *   - Inputs must not alias outputs.  The slot ids of the rows that a call
 *     writes must be distinct; two calls touching the same slot must be
 *     ordered on one stream.
 *   - Lengths, slots, positions and accepted counts are read on the device,
 *     so every call can be captured in a HIP graph and replayed with those
 *     buffers rewritten in place.
 *
 * Dtypes: the state is FP32 or BF16; q, k, v, the ring and the raw draft
 * tokens are in the activation dtype (FP32, BF16, or FP8 E4M3 with
 * per-tensor scales); alpha, beta and g are in the activation dtype, BF16
 * when it is FP8; y, the draft records and the conv and norm weights are
 * FP32.
 *
 * Layouts (row-major; q, k, v and g may have a token-row stride, see
 * kda_shape; everything else is contiguous):
 *   C = 2*dk + dv, the raw channels of one head in the order q | k | v.
 *   state pool   [num_slots, H, dk, dv]   state dtype, S[i][j] with i the key
 *                                          channel (dv contiguous)
 *   conv ring    [num_slots, 4, H, C]     act dtype; entry (p mod 4) holds the
 *                                          raw token at position p
 *   conv weights conv_w_q [H*dk, 4], conv_w_k [H*dk, 4], conv_w_v [H*dv, 4]
 *                                          FP32, tap 3 = current token
 *   norm_w       [dv] FP32, shared by all heads (NULL = all ones)
 */
#ifndef KDA_H
#define KDA_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Return codes.  Negative values are host-detected and leave every buffer
 * untouched. */
enum {
    KDA_OK = 0,
    KDA_ERR_NULL = -1,        /* a required pointer is NULL */
    KDA_ERR_SHAPE = -2,       /* a size or count is out of range */
    KDA_ERR_DTYPE = -3,       /* an unknown dtype or gate code */
    KDA_ERR_WORKSPACE = -4,   /* workspace missing or too small */
    KDA_ERR_UNSUPPORTED = -5, /* valid, but no kernel for these sizes */
    KDA_ERR_HIP = -6,         /* a HIP launch error */
    KDA_ERR_TOO_LARGE = -7    /* kda_prefill_noalloc: the call needs more
                               * scratch than KDA_PREFILL_SCRATCH_BYTES */
};

/* Bits OR-ed into *status by the device.  kda_status_str() also names each
 * single bit (a positive argument). */
enum {
    KDA_STATUS_BAD_SLOT = 1,      /* slot id >= num_slots */
    KDA_STATUS_BAD_POSITION = 2,  /* negative position */
    KDA_STATUS_BAD_ACCEPTED = 4,  /* accepted length outside [0, n_draft] */
    KDA_STATUS_BAD_SEQLENS = 8,   /* cu_seqlens not monotone, or past end */
    KDA_STATUS_STALLED = 16       /* kda_prefill: a hand-off between the waves
                                   * of a state workgroup did not arrive within
                                   * its bounded wait; the outputs and final
                                   * states of that call are not valid */
};

/* KDA_FP8_E4M3 is an activation dtype only: q, k, v, the conv ring and the
 * raw draft tokens are OCP FP8 E4M3 bytes (bias 7, no infinities, max 448)
 * times per-tensor scales (kda_params.qkv_scale), and alpha, beta and g are
 * BF16.  It follows the FP8 activations the model keeps ("Extend
 * NVIDIA/TensorRT-LLM#19991 ...", Description). */
typedef enum { KDA_F32 = 0, KDA_BF16 = 1, KDA_FP8_E4M3 = 2 } kda_dtype;
typedef enum { KDA_GATE_SIGMOID = 0, KDA_GATE_SILU = 1 } kda_gate;
/* What the alpha and beta buffers hold.  LOGITS: the decay logit a per key
 * channel and the write logit b per head, as the f_b projection the mixer
 * fuses produces them ("Extend NVIDIA/TensorRT-LLM#19991 ...", Description);
 * the kernels form alpha = exp(-softplus(a)) = 1 / (1 + e^a) and
 * beta = sigmoid(b) = 1 / (1 + e^-b) in FP32.  The stored tensors keep the
 * act dtype either way. */
typedef enum { KDA_GATES_VALUES = 0, KDA_GATES_LOGITS = 1 } kda_gate_inputs;

/* Host struct, passed by pointer.  Supported: head_k == head_v in {64, 128},
 * conv_width == 4. */
typedef struct {
    int32_t num_heads;   /* H */
    int32_t head_k;      /* dk */
    int32_t head_v;      /* dv */
    int32_t conv_width;  /* 4 */
    int32_t act_dtype;   /* kda_dtype of q, k, v, alpha, beta, g and the ring
                          * (FP8: q, k, v and the ring; alpha, beta, g BF16) */
    int32_t state_dtype; /* kda_dtype of the state pool */
    int32_t gate;        /* kda_gate of the output gate */
    float q_scale;       /* multiplies the normalised q (1 in the usual form);
                          * any finite value, else KDA_ERR_SHAPE */
    float l2_eps;        /* epsilon of the q/k L2 norms */
    float norm_eps;      /* epsilon of the gated RMSNorm */
    int32_t gate_inputs; /* kda_gate_inputs of the alpha and beta buffers */
    int32_t qkv_row_stride; /* elements from one token row of q (k, v) to the
                             * next; 0 = contiguous (H*dk).  Lets q, k and v be
                             * column ranges of one packed projection output,
                             * e.g. [tokens, H*(2dk+dv)].  Else >= H*dk and a
                             * multiple of 8 (KDA_ERR_SHAPE). */
    int32_t g_row_stride;   /* the same for g (0 = contiguous, H*dv) */
} kda_shape;

/* Host struct of the layer's parameters: device pointers to the weights,
 * and host values of the FP8 dequantisation scales. */
typedef struct {
    const float *conv_w_q; /* [H*dk, 4] */
    const float *conv_w_k; /* [H*dk, 4] */
    const float *conv_w_v; /* [H*dv, 4] */
    const float *norm_w;   /* [dv] or NULL for ones */
    float qkv_scale[3];    /* FP8 activations: q, k, v = E4M3 value * scale
                            * (each finite and > 0, else KDA_ERR_SHAPE);
                            * ignored for other activation dtypes */
} kda_params;

/* Text of a return code (zero or negative), or of one KDA_STATUS_* bit
 * (positive; a value with several bits set gets a generic text).  Host,
 * static storage. */
const char *kda_status_str(int code);

/* ----- sizes (host functions; 0 when the shape is invalid) ------------- */

/* Bytes of a state pool of `num_slots` slots: num_slots*H*dk*dv*sizeof. */
size_t kda_state_bytes(const kda_shape *shape, int64_t num_slots);
/* Bytes of a conv ring of `num_slots` slots: num_slots*4*H*C*sizeof(act). */
size_t kda_conv_bytes(const kda_shape *shape, int64_t num_slots);
/* Bytes of the FP32 verify records [batch, n_draft, H, dk, dv]. */
size_t kda_draft_state_bytes(const kda_shape *shape, int32_t batch,
                             int32_t n_draft);
/* Bytes of the raw draft tokens kept by verify [batch, n_draft, H, C] act. */
size_t kda_draft_conv_bytes(const kda_shape *shape, int32_t batch,
                            int32_t n_draft);
/* Bytes of workspace kda_prefill needs for `total_tokens` tokens in
 * `num_seqs` sequences: 147,456 bytes per (64-token chunk slot, head), with
 * ceil(total_tokens / 64) + num_seqs chunk slots (2,304 bytes per token and
 * head for long sequences; 1.14 GB for 15,360 tokens over 4 sequences at
 * H = 32).  0 for head sizes the prefill does not support. */
size_t kda_prefill_workspace_bytes(const kda_shape *shape, int32_t num_seqs,
                                   int64_t total_tokens);

/* ----- typed state store: the checkpoint format ------------------------ */
/* Logical FP32 import/export of the states of slots slot_ids[0..n).  The
 * typed store rounds to nearest even for BF16 pools; the load widens exactly.
 * Source: "Extend ... isolated NVFP4 Kimi K3 targets", Description (explicit
 * FP32 loads and typed state stores; FP32 or BF16 recurrent-state storage).
 *   src/dst  [n, H, dk, dv] FP32, S[i][j] with i the key channel.
 * Rows whose slot id is negative are skipped (dst left unwritten); slot ids
 * >= num_slots set KDA_STATUS_BAD_SLOT and are skipped. */
int kda_state_write(const kda_shape *shape, void *pool, int64_t num_slots,
                    const int32_t *slot_ids, int32_t n, const float *src,
                    int32_t *status, hipStream_t stream);
int kda_state_read(const kda_shape *shape, const void *pool,
                   int64_t num_slots, const int32_t *slot_ids, int32_t n,
                   float *dst, int32_t *status, hipStream_t stream);

/* Logical import/export of the conv history of slots slot_ids[0..n) at
 * positions[0..n) (tokens consumed so far).
 *   window [n, 3, H, C] act, oldest first: the raw tokens at positions
 *   p-3, p-2, p-1.  Read returns zeros for positions below 0; write skips
 *   them.  Source: the convolution KDA fuses ("Extend ... isolated NVFP4
 *   Kimi K3 targets", Description). */
int kda_conv_write(const kda_shape *shape, void *ring, int64_t num_slots,
                   const int32_t *slot_ids, const int32_t *positions,
                   int32_t n, const void *window, int32_t *status,
                   hipStream_t stream);
int kda_conv_read(const kda_shape *shape, const void *ring, int64_t num_slots,
                  const int32_t *slot_ids, const int32_t *positions,
                  int32_t n, void *window, int32_t *status,
                  hipStream_t stream);

/* ----- decode: one token for each of `batch` rows ---------------------- */
/* Source: the KDA one-token decode kernel every KDA layer takes ("Kimi K3 on
 * modeling_v2 ...", manual 16-rank runs) with the fused convolution, FP32
 * recurrence and gated norm of "Extend ... isolated NVFP4 Kimi K3 targets",
 * Description; output before o_proj (section 6).
 *   slot_ids [batch] int32: row b uses pool/ring slot slot_ids[b]; a negative
 *            id makes the row inactive (nothing read or written, y untouched).
 *   positions [batch] int32: tokens row b has consumed.  0 means a fresh
 *            sequence: zero state and empty history, pool and ring not read.
 *            The library never writes positions; the caller advances them.
 *   q, k, alpha [batch, H, dk]; v, g [batch, H, dv]; beta [batch, H]: act
 *            (with FP8 activations alpha, beta and g are BF16).
 *   pool, ring: read and written for active rows (state after the token;
 *            ring entry positions[b] mod 4 <- the raw q | k | v).
 *   y [batch, H, dv] FP32: the gated-norm output of active rows. */
int kda_decode(const kda_shape *shape, const kda_params *params,
               int32_t batch, int64_t num_slots, const int32_t *slot_ids,
               const int32_t *positions, const void *q, const void *k,
               const void *v, const void *alpha, const void *beta,
               const void *g, void *pool, void *ring, float *y,
               int32_t *status, hipStream_t stream);

/* ----- verify: n_draft tokens per row, pool and ring read-only ---------- */
/* Source: per-token KDA verify states and verify kernels ("Kimi K3 on
 * modeling_v2 ...", section 5); FP32 recurrence and FP32 per-token draft
 * records with either storage dtype ("Extend ... isolated NVFP4 Kimi K3
 * targets", Description).
 *   q, k, alpha [batch, n_draft, H, dk]; v, g [batch, n_draft, H, dv];
 *   beta [batch, n_draft, H]: act (alpha, beta, g BF16 with FP8
 *            activations).  1 <= n_draft <= 16.
 *   draft_states [batch, n_draft, H, dk, dv] FP32: the state after each
 *            draft token (never rounded, whatever the storage dtype).  May
 *            be NULL: no records are written, and the accepted prefix is
 *            then committed with kda_commit_recompute.
 *   draft_conv [batch, n_draft, H, C] act: the raw draft tokens, kept for
 *            kda_commit_accepted.  May be NULL (not kept).
 *   y [batch, n_draft, H, dv] FP32.
 * Inactive rows (negative slot) write nothing. */
int kda_verify(const kda_shape *shape, const kda_params *params,
               int32_t batch, int32_t n_draft, int64_t num_slots,
               const int32_t *slot_ids, const int32_t *positions,
               const void *q, const void *k, const void *v,
               const void *alpha, const void *beta, const void *g,
               const void *pool, const void *ring, float *draft_states,
               void *draft_conv, float *y, int32_t *status,
               hipStream_t stream);

/* ----- commit the accepted prefix of a verify --------------------------- */
/* Source: the per-token verify states ("Kimi K3 on modeling_v2 ...",
 * section 5), which let the accepted prefix be kept.
 *   accepted [batch] int32 (device): m in [0, n_draft].  m >= 1: the pool
 *            slot <- record m-1 (typed store, BF16 rounds once here) and the
 *            ring gets raw draft tokens 1..m at positions p..p+m-1.  m = 0
 *            writes nothing.  Out-of-range m sets KDA_STATUS_BAD_ACCEPTED.
 *   positions: the same values passed to kda_verify.  The caller advances
 *            them by m afterwards. */
int kda_commit_accepted(const kda_shape *shape, int32_t batch,
                        int32_t n_draft, int64_t num_slots,
                        const int32_t *slot_ids, const int32_t *positions,
                        const int32_t *accepted, const float *draft_states,
                        const void *draft_conv, void *pool, void *ring,
                        int32_t *status, hipStream_t stream);

/* ----- commit the accepted prefix by recomputing it --------------------- */
/* The alternative to per-token records: verify writes none (draft_states
 * NULL), and the commit runs the accepted tokens again from the stored state
 * and history.  Same result as kda_commit_accepted up to FP32 rounding order
 * (the same per-token arithmetic, FP32 across the m tokens, rounded once on
 * store for BF16 storage).  It trades the records' HBM traffic (n_draft
 * FP32 states per head) for reading the state once more.  Source: the
 * accepted-prefix commit of the speculative path ("Kimi K3 on modeling_v2
 * ...", section 5); the pages keep records ("Extend ... isolated NVFP4 Kimi
 * K3 targets", Description), which kda_commit_accepted follows.
 *   accepted [batch] int32 (device): m in [0, n_draft]; m >= 1 runs draft
 *            tokens 1..m of row b (the rows kda_verify was given, same
 *            layout) from the stored state, stores the state once and writes
 *            ring entries for positions p..p+m-1.  m = 0 writes nothing.
 *            Out-of-range m sets KDA_STATUS_BAD_ACCEPTED.
 *   q, k, alpha, v, g, beta: the verify's inputs, [batch, n_draft, H, .].
 *   positions: the same values passed to kda_verify; the caller advances
 *            them by m afterwards.  No output is written (verify gave y). */
int kda_commit_recompute(const kda_shape *shape, const kda_params *params,
                         int32_t batch, int32_t n_draft, int64_t num_slots,
                         const int32_t *slot_ids, const int32_t *positions,
                         const int32_t *accepted, const void *q, const void *k,
                         const void *v, const void *alpha, const void *beta,
                         const void *g, void *pool, void *ring,
                         int32_t *status, hipStream_t stream);

/* ----- chunked prefill over variable-length sequences ------------------- */
/* Source: the KDA prefill kernel and its varlen index glue ("Kimi K3 NVFP4
 * on Rubin (SM107): Modeling V2 target ...", section 3); FP32 recurrence
 * ("Extend ... isolated NVFP4 Kimi K3 targets", Description).  Chunkwise
 * WY/UT form with chunks of 64 tokens; the result equals the token-by-token
 * recurrence up to FP32-level rounding.  The chunk products run on the
 * matrix cores with operands split into fp16 pairs (2^-22 of each value).
 * Key-side operands are bounded; value-side operands (v, the writes U and
 * the state) carry an exact power-of-two scale per value column and chunk,
 * so any magnitude of v and of the stored state works, and any ratio between
 * them, with one limit: within a chunk and value column, a write or state
 * entry more than about 2^9 below the column's largest |U| or |S| keeps
 * about 2^-25 of that largest value in absolute terms rather than 2^-22 of
 * its own.  That matters only when a start state far larger than the
 * chunk's values decays away inside the chunk; the error is then about
 * 2^-25 x (start magnitude / result magnitude) relative to the result.
 * q_scale multiplies the read-outs, never an operand.
 *   cu_seqlens [num_seqs + 1] int32 (device): sequence s owns tokens
 *            cu_seqlens[s] .. cu_seqlens[s+1]-1 of the packed inputs.
 *   total_tokens: rows of the packed inputs (host).
 *   max_seqlen: host upper bound of any sequence length, sizes the grid.
 *   slot_ids, positions [num_seqs]: as in kda_decode; positions > 0
 *            continue a sequence from its stored state and history.
 *   q, k, alpha [total_tokens, H, dk]; v, g [total_tokens, H, dv];
 *   beta [total_tokens, H]: act (alpha, beta, g BF16 with FP8 activations).
 *   pool, ring: the final state (stored once) and the last 3 raw tokens.
 *   y [total_tokens, H, dv] FP32.
 *   workspace: device scratch of kda_prefill_workspace_bytes() bytes. */
int kda_prefill(const kda_shape *shape, const kda_params *params,
                int32_t num_seqs, const int32_t *cu_seqlens,
                int64_t total_tokens, int32_t max_seqlen, int64_t num_slots,
                const int32_t *slot_ids, const int32_t *positions,
                const void *q, const void *k, const void *v,
                const void *alpha, const void *beta, const void *g,
                void *pool, void *ring, float *y, void *workspace,
                size_t workspace_bytes, int32_t *status, hipStream_t stream);

/* ----- chunked prefill without any allocation --------------------------- */
/* For callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  The same
 * computation as kda_prefill with the same arguments, except that the
 * workspace is a fixed array of KDA_PREFILL_SCRATCH_BYTES inside the library
 * (one per GPU the library runs on, held until the process ends).
 *   - Calls whose kda_prefill_workspace_bytes(shape, num_seqs, total_tokens)
 *     exceeds KDA_PREFILL_SCRATCH_BYTES return KDA_ERR_TOO_LARGE before any
 *     launch (128 MiB holds 910 (64-token chunk slot, head) pairs: for
 *     example 1,728 tokens of one sequence at H = 32, or 29,056 at H = 2).
 *   - The call allocates nothing and calls no allocating routine.  Its first
 *     call on a device resolves that device's array address
 *     (hipGetSymbolAddress), which may load the library's code object; make
 *     that first call outside any graph capture.
 *   - Every call on a GPU shares that GPU's array, and nothing in it needs
 *     to start at zero.  Calls that overlap on one GPU (on different
 *     streams, or from different threads without ordering) race on it and
 *     give undefined results: order them on one stream. */
#define KDA_PREFILL_SCRATCH_BYTES ((size_t)128 << 20)
int kda_prefill_noalloc(const kda_shape *shape, const kda_params *params,
                        int32_t num_seqs, const int32_t *cu_seqlens,
                        int64_t total_tokens, int32_t max_seqlen,
                        int64_t num_slots, const int32_t *slot_ids,
                        const int32_t *positions, const void *q,
                        const void *k, const void *v, const void *alpha,
                        const void *beta, const void *g, void *pool,
                        void *ring, float *y, int32_t *status,
                        hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* KDA_H */
