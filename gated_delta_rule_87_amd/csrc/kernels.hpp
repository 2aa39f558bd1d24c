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
};

// Tile of region r for (batch b, head, chunk c).
__device__ inline unsigned char *ws_tile(const ChunkArgs &a, int r, int heads, int head, int b, int c) {
  return a.ws + a.wl.off[r] + (((size_t)b * heads + head) * a.N_c + c) * a.wl.tile[r];
}

struct StepArgs {
  const void *q, *k, *v, *beta, *log_alpha;
  float *state;
  void *o;
  int B, T, H_k, H_v, d_k, d_v, G, gshift;
  int beta_per_key_head;
};

// Each launcher validates nothing (the API layer did) and returns the launch
// status.  `in_bf16`/`out_bf16` select the element types.
hipError_t launch_prep(const ChunkArgs &a, bool in_bf16, hipStream_t stream);
hipError_t launch_scan(const ChunkArgs &a, bool in_bf16, bool out_bf16, hipStream_t stream);
hipError_t launch_step(const StepArgs &a, bool in_bf16, bool out_bf16, hipStream_t stream);

// Whether a shape is compiled in (the API layer reports GDR_ERR_UNSUPPORTED otherwise).
bool prep_supported(int C, int d_k, int G);
int scan_choose_bv(int B, int H_v, int C, int d_k, int d_v, bool in_bf16);
size_t prep_lds_bytes(int C, int d_k, int G);

}  // namespace gdr
