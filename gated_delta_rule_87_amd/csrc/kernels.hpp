// Kernel arguments and launchers (host/device shared declarations).
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace gdr {

// Workspace written by the prep kernel and read by the scan kernel: one
// fragment-major tile (layout at TileIO in common.hpp) per (batch, head,
// chunk) in each region, regions in this order, each 256-byte aligned:
//   A   diag(beta) A_c     [C][C]    per beta head
//   L   L_c                [C][C]    per key head
//   KB  Kbar_c             [C][d_k]  per key head
//   QB  Qbar_c             [C][d_k]  per key head
//   KH  Khat_c^T           [d_k][C]  per key head
//   GM  exp(Lambda_C)      [d_k]     per key head, fp32 vector
// Tile elements are fp16 for bf16 inputs and fp32 for fp32 inputs.
struct WsLayout {
  size_t tile[6];   // bytes per tile, in region order
  size_t off[6];    // region offsets
  size_t seg_off, seg_bytes;   // the segment-parallel scan's region (0 bytes when not used)
  size_t total;
};
enum WsRegion { kWsA = 0, kWsL, kWsKB, kWsQB, kWsKH, kWsGM };

__host__ __device__ inline WsLayout ws_layout(int B, int H_k, int H_beta, int N_c, int C, int d_k, bool bf16) {
  const size_t pb = bf16 ? 2 : 4;
  WsLayout w;
  w.tile[kWsA] = pb * C * C;
  w.tile[kWsL] = pb * C * C;
  w.tile[kWsKB] = pb * C * d_k;
  w.tile[kWsQB] = pb * C * d_k;
  w.tile[kWsKH] = pb * d_k * C;
  w.tile[kWsGM] = 4 * (size_t)d_k;
  size_t at = 0;
  for (int r = 0; r < 6; ++r) {
    w.off[r] = at;
    const size_t heads = r == kWsA ? H_beta : H_k;
    at += (size_t)B * heads * N_c * w.tile[r];
    at = (at + 255) & ~(size_t)255;
  }
  w.seg_off = at;
  w.seg_bytes = 0;
  w.total = at;
  return w;
}

struct ChunkArgs {
  const void *q, *k, *v, *beta, *log_alpha;  // inputs (in_dtype)
  const float *h0;                            // nullable
  void *o;                                    // out_dtype
  float *hT;                                  // nullable
  unsigned char *ws;                          // workspace, laid out by wl
  WsLayout wl;
  int B, T, H_k, H_v, d_k, d_v, C, G, gshift;
  int H_beta;                                 // H_v, or H_k when beta is per key head
  int N_c;
  int beta_per_key_head;
  int solve, order, residual;
  // Layer options (nullable / 0 = off): document resets [B, T] (nonzero =
  // the token starts a new document) and chunk-boundary momentum.
  const unsigned char *reset;
  float momentum;
  const float *z0;
  float *zT;
  // Segment-parallel scan: chunks per segment (0 = one segment).  A launch
  // covers segments seg0 + y (y = blockIdx.y); the scan's h0 of segment
  // seg0 + y is h0 + y * h0_seg_stride, and the transfer pass writes [J | B]
  // of segment seg0 + y to slot y of xfer.
  int seg_len;
  size_t h0_seg_stride;
  float *xfer;
  int seg0;
  // Training forward: the scan stores the state entering every chunk,
  // S_{c-1}, to states [B][H_v][N_c][d_k][d_v] (nullable; fp16 for bf16
  // inputs, fp32 for fp32 inputs).
  void *states;
  // Backward preparation (bwd != 0): the prep kernels write the operands of
  // the reverse scan in place of the forward ones -- in reversed token order
  // within the chunk (J the reversal) region A holds J (diag(beta) A_c)^T J,
  // L holds J L_c^T J (both lower triangular again), KB holds J Khat_c
  // (token rows), QB holds (J Qbar_c)^T and KH holds (J Kbar_c)^T (channel
  // rows) -- and also the unscaled A_c to au [B][H_beta][N_c][C][C] and the
  // beta-free Gram G_c to gu [B][H_k][N_c][C][C] (fp32, row-major, zero above
  // the diagonal).
  int bwd;
  float *au, *gu;
};

// Tile of region r for (batch b, head, chunk c).
__device__ inline unsigned char *ws_tile(const ChunkArgs &a, int r, int heads, int head, int b, int c) {
  return a.ws + a.wl.off[r] + (((size_t)b * heads + head) * a.N_c + c) * a.wl.tile[r];
}

struct StepArgs {
  const void *q, *k, *v, *beta, *log_alpha;
  float *state;                 // fp32 state, or (E4M3 format) the row codes as bytes
  void *o;
  int B, T, H_k, H_v, d_k, d_v, G, gshift;
  int beta_per_key_head;
  const int *n_tokens;          // nullable [B]: tokens stepped per sequence (prefix of the T given)
  const unsigned char *reset;   // nullable [B, T]: the token starts a new document
  float *scale;                 // E4M3 format: one fp32 scale per state row [B, H_v, d_k]
};

// Backward pass (chunk size 64): the upstream gradients and the outputs of
// the reverse scan and the gradient kernel.
struct BwdArgs {
  const void *d_o;            // [B, T, H_v, d_v] out_dtype
  const float *dhT;           // nullable [B, H_v, d_k, d_v]
  const void *states;         // S_{c-1} of every chunk, [B][H_v][N_c][d_k][d_v] (fp16 / fp32 as above)
  float *dq, *dk;             // [B, T, H_k, d_k]
  float *dv;                  // [B, T, H_v, d_v]
  float *dbeta;               // [B, T, H_beta]
  float *dla;                 // [B, T, H_k, G]
  float *dh0;                 // nullable [B, H_v, d_k, d_v]
  // workspace, fp16 for bf16 inputs and fp32 for fp32 inputs:
  void *x;                    // X_c = L_c^T dO_c + Khat_c dS_c, [B, T, H_v, d_v]
  void *dstates;              // dS_c of every chunk, [B][H_v][N_c][d_k][d_v]
};

// Drafted tokens one verification call takes.
constexpr int kVerifyMaxTokens = 16;
// Largest finite value of the E4M3 format (OCP FP8, 4 exponent bits, bias 7).
constexpr float kE4M3Max = 448.f;

// Each launcher validates nothing (the API layer did) and returns the launch
// status.  `in_bf16`/`out_bf16` select the element types.
hipError_t launch_prep(const ChunkArgs &a, bool in_bf16, hipStream_t stream);
hipError_t launch_scan(const ChunkArgs &a, bool in_bf16, bool out_bf16, hipStream_t stream);
hipError_t launch_gated_rmsnorm(const void *o, const void *z, const float *weight, float eps, void *y,
                                long long rows, int d_v, bool o_bf16, bool z_bf16, hipStream_t stream);
hipError_t launch_step(const StepArgs &a, bool in_bf16, bool out_bf16, hipStream_t stream);
hipError_t launch_step_e4m3(const StepArgs &a, bool in_bf16, bool out_bf16, hipStream_t stream);
hipError_t launch_verify(const StepArgs &a, bool in_bf16, bool out_bf16, hipStream_t stream);
// Backward: the reverse state scan (dv, X, dS_c, dh0) and the per-chunk
// gradient kernel (dq, dk, dbeta, dlog_alpha).  `g_bf16`: d_o is bf16.
hipError_t launch_bwd_scan(const ChunkArgs &a, const BwdArgs &g, bool in_bf16, bool g_bf16, hipStream_t stream);
hipError_t launch_bwd_grad(const ChunkArgs &a, const BwdArgs &g, bool in_bf16, bool g_bf16, hipStream_t stream);
bool bwd_supported(int C, int d_k, int d_v);
// Row-scaled E4M3 <-> fp32 for `rows` state rows of d_v values.
hipError_t launch_state_quantize(const float *x, unsigned char *codes, float *scale, long long rows, int d_v,
                                 hipStream_t stream);
hipError_t launch_state_dequantize(const unsigned char *codes, const float *scale, float *x, long long rows, int d_v,
                                   hipStream_t stream);

}  // namespace gdr

#include "gdr.h"

namespace gdr {

// The chunk forward behind gdr_chunk_fwd and gdr_chunk_fwd_ex (prepare =
// true) and gdr_chunk_scan (prepare = false): validation, then the launches.
// opts may be NULL.  api.cpp.
// `states` (nullable): the training forward's chunk-entry states.
gdr_status chunk_forward(const gdr_problem *p, const void *q, const void *k, const void *v, const void *beta,
                         const void *log_alpha, const float *h0, void *o, float *hT, const void *workspace,
                         size_t workspace_bytes, void *stream, bool prepare, const gdr_layer_opts *opts,
                         void *states = nullptr);
// Workspace bytes of a valid problem (else the validation status).
gdr_status workspace_bytes_of(const gdr_problem *p, size_t *bytes);
// Rows of [B][T] tokens to the padded sequence of chunk size 16 (real token
// t at 32 (t / 16) + t % 16 of Tp, zeros elsewhere), or back (unpad).
hipError_t launch_pad_rows(void *dst, const void *src, size_t row_bytes, int B, int T, int Tp, bool unpad,
                           hipStream_t s);
// Record `text` as this thread's gdr_last_error() and return s.
gdr_status set_error(gdr_status s, const char *text);

// Raise a kernel's dynamic LDS limit to the CU's 160 KiB, once per kernel and
// device (each launch then passes its own size); later calls return at once.
hipError_t allow_full_lds(const void *kernel);

// Whether a shape is compiled in (the API layer reports GDR_ERR_UNSUPPORTED otherwise).
bool prep_supported(int C, int d_k, int G);
int scan_choose_bv(int B, int H_v, int C, int d_k, int d_v, bool in_bf16);
// Segments of the segment-parallel scan (1 = one scan over the whole
// sequence) and the bytes of its workspace region.
int scan_segments(int B, int H_v, int N_c, int d_v, int C, int d_k, bool f32);
size_t scan_seg_bytes(int B, int H_v, int N_c, int d_k, int d_v, int C, bool f32);
size_t prep_lds_bytes(int C, int d_k, int G);

}  // namespace gdr
