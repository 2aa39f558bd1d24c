// Kernel arguments and launchers (host/device shared declarations).
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace gdr {

struct ChunkArgs {
  const void *q, *k, *v, *beta, *log_alpha;  // inputs (in_dtype)
  const float *h0;                            // nullable
  void *o;                                    // out_dtype
  float *hT;                                  // nullable
  float *A_ws;                                // [B, H_beta, N_c, C, C]
  float *L_ws;                                // [B, H_k, N_c, C, C]
  int B, T, H_k, H_v, d_k, d_v, C, G, gshift;
  int H_beta;                                 // H_v, or H_k when beta is per key head
  int N_c;
  int beta_per_key_head;
  int solve, order, residual;
};

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
int scan_choose_bv(int B, int H_v, int C, int d_k, int d_v, int G, bool in_bf16);
size_t prep_lds_bytes(int C, int G);

}  // namespace gdr
