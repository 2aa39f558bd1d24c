/*
 * gdr.h -- C ABI of libgdr.so: chunkwise gated delta-rule forward on AMD
 * MI355X (gfx950).
 *
 * The operation ("Systolic Linear Attention: Co-Designing Tile-Grouped Gated
 * Delta Attention for TPUs", section 2.1, Eq. (2)): for every batch b and value head h, with key head
 * h_k = h / (H_v / H_k) and S_0 = h0 (or 0), for t = 1..T
 *
 *     S_t = (I - beta_t k_t k_t^T) F_t S_{t-1} + beta_t k_t v_t^T,
 *     o_t = S_t^T q_t,
 *
 * with the diagonal decay F_t = diag(exp(log_alpha_t)) shared by the d_k/G
 * channels of each of G contiguous channel groups (G = 1: scalar Gated
 * DeltaNet gate; G = d_k: per-channel KDA gate; G = 4 with d_k = 256: the
 * four-tile gate of the same paper, section 2.3).  The value heads of one key
 * head are contiguous (grouped value heads, section 2.4.1).
 *
 * gdr_chunk_fwd evaluates it chunk by chunk in the WY form (same paper,
 * Table 2 and section 2.4.2): per chunk of C tokens it builds the strictly
 * lower-triangular Gram M_c and the score matrix L_c with division-free
 * relative decay, solves A_c = (I + M_c)^{-1} (exactly, or by the truncated
 * Neumann series with residual correction of "When Good Enough Is Optimal:
 * Multiplication-Only Matrix Inversion Approximation for Quantized Gated
 * DeltaNet"), and carries the d_k x d_v state
 * across chunks.  gdr_recurrent_step runs the token recurrence directly (the
 * stateful step-by-step decoding of section 2.4.3).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - All tensor pointers are DEVICE pointers (HBM), row-major, contiguous, and
 *   16-byte aligned.  The caller allocates and frees every buffer; the
 *   library never allocates device memory, never synchronises the stream and
 *   keeps no global state other than a thread-local error message and a
 *   record of the kernels whose LDS limit it has raised on each device.
 * - Layouts:   q, k       [B, T, H_k, d_k]          in_dtype
 *              v          [B, T, H_v, d_v]          in_dtype
 *              beta       [B, T, H_v]  ([B, T, H_k] if beta_per_key_head)  in_dtype
 *              log_alpha  [B, T, H_k, G]            in_dtype, natural log, <= 0
 *              o          [B, T, H_v, d_v]          out_dtype
 *              h0, hT, state [B, H_v, d_k, d_v]     fp32
 * - Work is enqueued on `stream` (a hipStream_t; NULL = the default stream)
 *   and runs asynchronously; kernel faults surface at the caller's next
 *   synchronisation, as usual for HIP.
 * - Every argument is validated before anything is enqueued; on a non-OK
 *   return nothing was enqueued and gdr_last_error() describes why.
 * - Non-finite inputs propagate; they are not checked.
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
  GDR_ERR_INVALID_ARG = 1, /* null/misaligned pointer, bad size, inconsistent heads */
  GDR_ERR_UNSUPPORTED = 2, /* valid problem outside the shapes the library is compiled for */
  GDR_ERR_WORKSPACE = 3,   /* workspace missing or smaller than the queried size  */
  GDR_ERR_HIP = 4          /* a HIP launch failed; gdr_last_error() has the text  */
} gdr_status;

typedef enum { GDR_F32 = 0, GDR_BF16 = 1 } gdr_dtype;

typedef enum {
  GDR_SOLVE_EXACT = 0,   /* A_c = (I + M_c)^{-1} exactly (recursive block doubling) */
  GDR_SOLVE_NEUMANN = 1, /* sum_{s=0}^{m} (-M_c)^s, then r corrections X <- X + X(I - (I + M_c)X) */
  GDR_SOLVE_BLOCK_NEUMANN = 2 /* sum_{s=0}^{m} (-N)^s D^{-1}: D the 16-row block diagonal of I + M_c,
                                 N = D^{-1}(I + M_c - D); m = 1 is SLA's 1-Step Neumann
                                 (section 2.4.3); r is not used */
} gdr_solve;

/* Problem description.  Enumerations are stored as int32_t for a stable ABI. */
typedef struct {
  int32_t B, T;                    /* batch, tokens (T >= 0; T need not divide by chunk) */
  int32_t H_k, H_v;                /* key heads, value heads; H_v % H_k == 0 */
  int32_t d_k, d_v;                /* key width, value width */
  int32_t chunk;                   /* C, tokens per chunk */
  int32_t gate_groups;             /* G: 1, d_k, or a divisor of d_k */
  int32_t beta_per_key_head;       /* 0: beta [B,T,H_v]; 1: beta [B,T,H_k] shared by R value heads */
  int32_t in_dtype;                /* gdr_dtype of q, k, v, beta, log_alpha */
  int32_t out_dtype;               /* gdr_dtype of o */
  int32_t solve;                   /* gdr_solve (chunk path only) */
  int32_t neumann_order;           /* m >= 0: powers 0..m are kept (both Neumann solves) */
  int32_t neumann_residual_steps;  /* r >= 0 residual corrections (GDR_SOLVE_NEUMANN) */
} gdr_problem;

/*
 * Bytes of device workspace gdr_chunk_fwd needs for problem p (0 for an
 * invalid problem).  The workspace holds every per-chunk quantity of the WY
 * form (Systolic Linear Attention, Table 2), prepared once per chunk and
 * head so that the sequential state scan only multiplies.  Six regions, in
 * this order, each a stack of tiles indexed [B][heads][N_c] (N_c =
 * ceil(T / C), H_beta = H_v, or H_k with beta_per_key_head):
 *   0  A    diag(beta_c) A_c           C x C     per beta head
 *   1  L    L_c (decayed q.k, t >= j)  C x C     per key head
 *   2  KB   Kbar_c = K (.) exp(Lambda) C x d_k   per key head
 *   3  QB   Qbar_c = Q (.) exp(Lambda) C x d_k   per key head
 *   4  KH   Khat_c^T, Khat = K (.) exp(Lambda_C - Lambda)
 *                                      d_k x C   per key head
 *   5  GM   exp(Lambda_C) per channel  d_k       per key head, fp32
 * Tile elements are fp16 for bf16 inputs (round to nearest even) and fp32
 * for fp32 inputs.  Tiles are fragment-major, the order in which 16x16x32
 * MFMA operands are read: an R x K tile is (R/16) x (K/32) blocks,
 * row-block-major; a block is 64 fragments of 8 consecutive columns,
 * fragment f = 16 q + r holding row r, columns 8 q .. 8 q + 7 of the block,
 * at byte 16 f (fp16, 1 KiB blocks) or 32 f (fp32, 2 KiB blocks).  A and L
 * are lower triangular: their blocks wholly above the diagonal (block
 * (i, j) with 32 j > 16 i + 15) are neither written nor read, and hold
 * whatever the buffer held.  Token rows
 * (columns of KH) of a short final chunk past T are zero and its gate values
 * are those of its last real token.  Region
 * offsets: gdr_chunk_workspace_layout.
 * When the (batch, value head, 32 value columns) units number fewer than
 * 256, d_v is a multiple of 32 and there are at least 18 chunks, the scan is
 * split into P >= 3 segments of the sequence (the affine chunk map of
 * section 3.3 composed across segments) and the workspace ends with one
 * more region, after GM at a 256-byte boundary, of
 * 4 B H_v d_k ((P - 2)(d_k + d_v) + (P - 1) d_v) bytes: the transitions
 * [J | B] of segments 1 .. P-2 and the entry states of segments 1 .. P-1.
 * The total size includes it.
 * Chunk 16 runs as chunk 32 on a padded sequence of T' = 32 ceil(T / 16)
 * tokens, each 16 tokens followed by 16 identity tokens (zero q, k, v, beta
 * and log alpha), which leaves the state and the per-16-token in-chunk
 * matrices as they are: the regions above are those of that padded problem
 * (chunk 32, T'), followed by padded copies of the inputs and of o.
 */
size_t gdr_chunk_fwd_workspace_size(const gdr_problem *p);

/*
 * Byte offsets of the six workspace regions above: offsets[0..5], and the
 * total size (== gdr_chunk_fwd_workspace_size) in offsets[6].  `offsets` is a
 * host array of 7 size_t.  For inspecting a prepared workspace.
 */
gdr_status gdr_chunk_workspace_layout(const gdr_problem *p, size_t *offsets);

/*
 * Chunkwise forward (Systolic Linear Attention Table 2 / section 2.4.2 WY
 * form; section 2.4.3 for the exact in-chunk inverse; the multiplication-only
 * inversion paper for the Neumann mode).
 *   q, k, v, beta, log_alpha : inputs, layouts above, read-only.
 *   h0        : initial state, fp32 [B,H_v,d_k,d_v]; NULL = zero state.
 *   o         : output, out_dtype [B,T,H_v,d_v].
 *   hT        : final state, fp32 [B,H_v,d_k,d_v]; NULL = not written; may alias h0.
 *   workspace : device scratch of at least gdr_chunk_fwd_workspace_size(p)
 *               bytes, 256-byte aligned; its contents on return are the
 *               per-chunk quantities documented there.
 * Supported here: in_dtype bf16 or f32, chunk 16, 32, 64 or 128, d_k in {64,128,256},
 * d_v a multiple of 16 (of 32 with chunk 16 or 32), G a divisor of d_k, B and H_v at most 65535, fewer
 * than 2^24 chunks per sequence, B H_v d_v / 16 below 2^23 and
 * chunk H_v d_v below 2^30 (one chunk of v or o within 4 GiB); beyond that
 * GDR_ERR_UNSUPPORTED.
 */
gdr_status gdr_chunk_fwd(const gdr_problem *p, const void *q, const void *k, const void *v,
                         const void *beta, const void *log_alpha, const float *h0, void *o,
                         float *hT, void *workspace, size_t workspace_bytes, void *stream);

/*
 * The parallel half of gdr_chunk_fwd: fills `workspace` with every per-chunk
 * quantity listed at gdr_chunk_fwd_workspace_size, exactly as gdr_chunk_fwd
 * leaves it, without touching any state or output.  All chunks of all heads
 * are independent here (one workgroup each).
 */
gdr_status gdr_chunk_prepare(const gdr_problem *p, const void *q, const void *k,
                             const void *beta, const void *log_alpha, void *workspace,
                             size_t workspace_bytes, void *stream);

/*
 * The sequential half of gdr_chunk_fwd: the state scan and output over a
 * workspace that gdr_chunk_prepare filled for the same problem, so
 * gdr_chunk_fwd(...) == gdr_chunk_prepare(...) then gdr_chunk_scan(...).
 * Only v, h0 and the workspace are read (everything derived from q, k, beta
 * and log_alpha is in the workspace).  Running it again with another h0 (or
 * v) reuses the prepared chunks; that is the second pass of a sequence split
 * across devices, where each piece re-reads its output from the state handed
 * over by the previous piece (Systolic Linear Attention, section 3.3, the
 * affine chunk map).  The scan's own regions of the workspace (the
 * segment-parallel scan's maps and entry states; with chunk 16 the padded
 * copies of v and o) are rewritten; the prepared chunks are not.  Other
 * arguments as for gdr_chunk_fwd.
 */
gdr_status gdr_chunk_scan(const gdr_problem *p, const void *v, const float *h0, void *o, float *hT,
                          const void *workspace, size_t workspace_bytes, void *stream);

/*
 * gdr_chunk_fwd without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, serving loops and
 * harnesses that forbid allocation.  The per-chunk quantities go to a static
 * device array of GDR_NOALLOC_SCRATCH_BYTES (128 MiB) that the library holds
 * on each device it runs on until the process ends; the array of the current
 * device (hipGetDevice) is used, so `stream` must belong to that device.
 * Problems whose gdr_chunk_fwd_workspace_size exceeds the array return
 * GDR_ERR_UNSUPPORTED with nothing enqueued.  No memory is allocated or
 * freed and nothing in the array needs clearing (the prep kernels write
 * every byte the scan reads).  Every call on one device shares its array:
 * calls that overlap in time on one device (two streams, two threads) race
 * and produce wrong results; the caller must serialise them.  Other
 * arguments, results and errors as for gdr_chunk_fwd.
 */
#define GDR_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)
gdr_status gdr_chunk_fwd_noalloc(const gdr_problem *p, const void *q, const void *k, const void *v,
                                 const void *beta, const void *log_alpha, const float *h0, void *o,
                                 float *hT, void *stream);

/*
 * Layer options of the chunk path: the sequence-level features of the
 * Systolic Linear Attention layer (Table 2, the symbols Z_c, mu and kappa_c;
 * section 2.3, "Why chunk-level momentum").
 *   reset    : NULL, or DEVICE bytes [B, T]; nonzero marks a token that starts
 *              a new document: the state carried into it is discarded
 *              (S_{t-1} <- 0 before its step).  Packed documents of any
 *              lengths therefore share one row of the batch.
 *   momentum : mu of the chunk-boundary momentum; 0 turns it off (z0 and zT
 *              are then ignored).  With mu != 0, over chunks of `chunk`
 *              tokens counted from each sequence's first token (the last may
 *              be shorter), with S~_c the state after chunk c's last token
 *              (evolved token by token from S_{c-1}; the chunk's outputs are
 *              read from that evolution), F_c the product of the chunk's
 *              decays and kappa_c = 0 when a reset falls in the chunk:
 *                carry = kappa_c F_c S_{c-1},
 *                Z_c = mu kappa_c Z_{c-1} + (S~_c - carry),  S_c = carry + Z_c.
 *              The result depends on where chunks start: a sequence split
 *              across calls must be split at a multiple of `chunk`.
 *   z0, zT   : momentum buffer in / out, fp32 [B, H_v, d_k, d_v] like h0 / hT;
 *              NULL z0 = zero, NULL zT = not written; zT may alias z0.
 */
typedef struct {
  const uint8_t *reset;
  float momentum;
  const float *z0;
  float *zT;
} gdr_layer_opts;

/*
 * gdr_chunk_fwd with layer options (opts NULL = gdr_chunk_fwd).  The
 * prepared chunks of a chunk holding a reset are formed entry by entry on
 * the block-pivot route: pairs of tokens from different documents get no
 * decay factor, the rows of Kbar and Qbar after the chunk's first reset and
 * the rows of Khat before its last one are zero, and region GM holds -0 in
 * every channel.  Other arguments, results and errors as for gdr_chunk_fwd;
 * a non-finite momentum is GDR_ERR_INVALID_ARG.
 */
gdr_status gdr_chunk_fwd_ex(const gdr_problem *p, const gdr_layer_opts *opts, const void *q, const void *k,
                            const void *v, const void *beta, const void *log_alpha, const float *h0,
                            void *o, float *hT, void *workspace, size_t workspace_bytes, void *stream);

/*
 * Training: forward with saved chunk-entry states, and the backward pass
 * (Systolic Linear Attention, section 2.5: a custom VJP that saves only the
 * state S_{c-1} entering each chunk and recomputes M_c, L_c and A_c;
 * D_c = A_c^T diag(beta) dE_c and dM_c = -tril_{-1}(D_c E~_c^T) with
 * E~_c = A_c (V_c - Kbar_c S_{c-1})).
 *
 * Supported: chunk 64, d_k in {64, 128}, d_v a multiple of 32, the exact
 * solve, in_dtype bf16 or f32; no layer options (resets, momentum).  Other
 * problems return GDR_ERR_UNSUPPORTED (size functions: 0).
 *
 * gdr_chunk_states_size: bytes of `states`, [B, H_v, N_c, d_k, d_v]
 * (N_c = ceil(T / chunk)): S_{c-1} of every chunk c, S_{-1} = h0 (or 0),
 * fp16 for bf16 inputs (round to nearest even: the value the forward's
 * state operand of that chunk holds, and the precision the gradient
 * kernel multiplies it in) and fp32 for fp32 inputs.
 *
 * gdr_chunk_fwd_train: gdr_chunk_fwd (same arguments, workspace size and
 * results) that also writes `states` (16-byte aligned; NULL allowed only
 * when B T = 0).
 */
size_t gdr_chunk_states_size(const gdr_problem *p);
gdr_status gdr_chunk_fwd_train(const gdr_problem *p, const void *q, const void *k, const void *v,
                               const void *beta, const void *log_alpha, const float *h0, void *o,
                               float *hT, void *states, void *workspace, size_t workspace_bytes,
                               void *stream);

/*
 * Bytes of device workspace gdr_chunk_bwd needs (0 for an unsupported
 * problem): the six operand regions of gdr_chunk_fwd_workspace_size (no
 * segment region) holding the reverse scan's operands, A_c and G_c in fp32
 * ([B][H_beta][N_c][C][C] and [B][H_k][N_c][C][C]), X_c = L_c^T dO_c +
 * Khat_c dS_c ([B, T, H_v, d_v]) and dS_c of every chunk ([B, H_v, N_c, d_k,
 * d_v]), the last two fp16 for bf16 inputs and fp32 for fp32 inputs, each
 * region at a 256-byte boundary.
 */
size_t gdr_chunk_bwd_workspace_size(const gdr_problem *p);

/*
 * Backward pass: gradients of sum(o (.) d_o) + sum(hT (.) dhT) with respect
 * to every input of gdr_chunk_fwd_train.
 *   q, k, v, beta, log_alpha : the forward's inputs (layouts and dtype as there).
 *   states : what gdr_chunk_fwd_train wrote for these inputs and h0.
 *   d_o    : upstream gradient of o, out_dtype [B, T, H_v, d_v].
 *   dhT    : upstream gradient of hT, fp32 [B, H_v, d_k, d_v]; NULL = zero.
 *   dq, dk : fp32 [B, T, H_k, d_k];  dv : fp32 [B, T, H_v, d_v];
 *   dbeta  : fp32, beta's layout;    dlog_alpha : fp32 [B, T, H_k, G];
 *   dh0    : fp32 [B, H_v, d_k, d_v], or NULL = not written.
 * Every output is written in full (no accumulation into existing values).
 * workspace: at least gdr_chunk_bwd_workspace_size(p) bytes, 256-byte aligned.
 * Three launches after the prep kernels (which write the reverse operands):
 * the reverse state scan (dv, X, dS_c, dh0; sequential over chunks) and the
 * per-chunk gradient kernel (dq, dk, dbeta, dlog_alpha; all chunks at once).
 */
gdr_status gdr_chunk_bwd(const gdr_problem *p, const void *q, const void *k, const void *v,
                         const void *beta, const void *log_alpha, const void *states, const void *d_o,
                         const float *dhT, float *dq, float *dk, float *dv, float *dbeta,
                         float *dlog_alpha, float *dh0, void *workspace, size_t workspace_bytes,
                         void *stream);

/*
 * Output epilogue of the same layer (section 2.3, token-level recurrence
 * box): per (batch, token, value head) row of d_v entries,
 *     y = sigmoid(z) (.) o / sqrt(mean(o^2) + eps) (.) weight,
 * o and y of p->out_dtype, z of p->in_dtype, all [B, T, H_v, d_v]; weight
 * fp32 [d_v] or NULL (= 1); eps >= 0.  y may alias o.  The pages fix
 * neither eps nor a scale vector: both are the caller's.
 */
gdr_status gdr_gated_rmsnorm(const gdr_problem *p, const void *o, const void *z, const float *weight,
                             float eps, void *y, void *stream);

/*
 * Token recurrence, p->T tokens in order (Systolic Linear Attention, section
 * 2.1, Eq. (2)), updating `state` in place (fp32 [B,H_v,d_k,d_v], read and
 * written) and writing o [B,T,H_v,d_v].  chunk / solve fields are ignored.
 * Supported here: d_k in {64,128,256}, d_v a multiple of 16, B and H_v at
 * most 65535.
 */
gdr_status gdr_recurrent_step(const gdr_problem *p, const void *q, const void *k, const void *v,
                              const void *beta, const void *log_alpha, float *state, void *o,
                              void *stream);

/*
 * Speculative verification (Systolic Linear Attention, section 3.2): the
 * outputs o [B, T, H_v, d_v] of T <= 16 drafted tokens per sequence, read
 * from `state` (fp32 [B, H_v, d_k, d_v], READ ONLY: the call does not advance
 * it) with the same block inversion as the chunk path -- the drafted tokens
 * form one chunk of the WY form (Table 2).  chunk / solve fields are
 * ignored; T > 16 is GDR_ERR_UNSUPPORTED.  Once n_b of sequence b's drafted
 * tokens are accepted, gdr_recurrent_step_ex with n_tokens advances each
 * state by exactly its accepted prefix.
 */
gdr_status gdr_verify(const gdr_problem *p, const void *q, const void *k, const void *v, const void *beta,
                      const void *log_alpha, const float *state, void *o, void *stream);

typedef enum {
  GDR_STATE_F32 = 0,   /* fp32 [B, H_v, d_k, d_v] */
  GDR_STATE_E4M3 = 1   /* row-scaled FP8: E4M3 codes (bytes) [B, H_v, d_k, d_v] and fp32 scales [B, H_v, d_k] */
} gdr_state_format;

/*
 * Options of the recurrent step (serving; all nullable / 0 = off).
 *   n_tokens     : DEVICE int32 [B]: sequence b steps only its first
 *                  min(n_tokens[b], T) tokens (speculative decoding commits
 *                  the accepted prefix); the outputs of the other tokens are
 *                  not written.
 *   reset        : DEVICE bytes [B, T]: nonzero = the token starts a new
 *                  document (the state carried into it is discarded).
 *   state_format : gdr_state_format of `state`.  GDR_STATE_E4M3 (the
 *                  row-scaled FP8 state of the same paper's serving study):
 *                  row i of a (batch, value head) state -- key channel i --
 *                  is stored as E4M3 codes c (OCP FP8, 4 exponent and 3
 *                  mantissa bits, largest finite 448) with one fp32 scale
 *                  s_i = max_j |S_ij| / 448, S_ij = value(c_ij) s_i.  The
 *                  call dequantises the state once, steps its tokens in fp32
 *                  and quantises once at the end: x (448 / max_j |S_ij|)
 *                  (fp32), clamped to +-448, rounded to E4M3 to nearest even;
 *                  a zero row gets scale 0.  Supported for d_v in {32, 64,
 *                  128}; one workgroup per (batch, value head).
 *   state_scale  : the fp32 scales [B, H_v, d_k] (E4M3 only), read and written.
 */
typedef struct {
  const int32_t *n_tokens;
  const uint8_t *reset;
  int32_t state_format;
  float *state_scale;
} gdr_step_opts;

/* gdr_recurrent_step with step options (opts NULL = gdr_recurrent_step);
 * `state` is fp32, or E4M3 codes when opts->state_format says so. */
gdr_status gdr_recurrent_step_ex(const gdr_problem *p, const gdr_step_opts *opts, const void *q, const void *k,
                                 const void *v, const void *beta, const void *log_alpha, void *state, void *o,
                                 void *stream);

/* Conversions between an fp32 state [B, H_v, d_k, d_v] and the row-scaled
 * E4M3 form above (codes [B, H_v, d_k, d_v] bytes, scales [B, H_v, d_k] fp32),
 * with the same rounding as gdr_recurrent_step_ex.  d_v <= 256. */
gdr_status gdr_state_quantize(const gdr_problem *p, const float *state, void *codes, float *scale, void *stream);
gdr_status gdr_state_dequantize(const gdr_problem *p, const void *codes, const float *scale, float *state,
                                void *stream);

/* Static text for a status code. */
const char *gdr_status_string(gdr_status s);

/* Thread-local detail for the last non-OK return on this thread ("" if none). */
const char *gdr_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* GDR_H_ */
