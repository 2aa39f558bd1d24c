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
 *   keeps no global state other than a thread-local error message.
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
  GDR_SOLVE_NEUMANN = 1  /* sum_{s=0}^{m} (-M_c)^s, then r corrections X <- X + X(I - (I + M_c)X) */
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
  int32_t neumann_order;           /* m >= 0: powers 0..m are kept */
  int32_t neumann_residual_steps;  /* r >= 0 residual corrections */
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
 * Supported here: in_dtype bf16 or f32, chunk 64 or 128, d_k in {64,128,256},
 * d_v a multiple of 16, G a divisor of d_k, B and H_v at most 65535, fewer
 * than 2^24 chunks per sequence and B H_v d_v / 16 below 2^23; beyond that
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
 * affine chunk map).  Other arguments as for gdr_chunk_fwd.
 */
gdr_status gdr_chunk_scan(const gdr_problem *p, const void *v, const float *h0, void *o, float *hT,
                          const void *workspace, size_t workspace_bytes, void *stream);

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

/* Static text for a status code. */
const char *gdr_status_string(gdr_status s);

/* Thread-local detail for the last non-OK return on this thread ("" if none). */
const char *gdr_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* GDR_H_ */
