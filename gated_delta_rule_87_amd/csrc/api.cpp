// C ABI of libgdr.so (declared in include/gdr.h): argument validation,
// workspace sizing and launch sequencing.  Nothing here allocates device
// memory or synchronises; every check runs before the first launch.
#include <hip/hip_runtime_api.h>

#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <string>

#include "gdr.h"
#include "kernels.hpp"

namespace {

thread_local std::string g_err;

gdr_status fail(gdr_status s, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return s;
}

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int log2_exact(int x) {
  int s = 0;
  while ((1 << s) < x) ++s;
  return ((1 << s) == x) ? s : -1;
}

// Shape checks shared by both paths.  `chunked` adds the chunk-path fields.
gdr_status check_problem(const gdr_problem *p, bool chunked) {
  if (!p) return fail(GDR_ERR_INVALID_ARG, "problem is NULL");
  if (p->B < 0 || p->T < 0) return fail(GDR_ERR_INVALID_ARG, "B=%d T=%d must be >= 0", p->B, p->T);
  if (p->H_k <= 0 || p->H_v <= 0) return fail(GDR_ERR_INVALID_ARG, "H_k=%d H_v=%d must be > 0", p->H_k, p->H_v);
  if (p->H_v % p->H_k != 0)
    return fail(GDR_ERR_INVALID_ARG, "H_v=%d is not a multiple of H_k=%d", p->H_v, p->H_k);
  if (p->d_k <= 0 || p->d_v <= 0) return fail(GDR_ERR_INVALID_ARG, "d_k=%d d_v=%d must be > 0", p->d_k, p->d_v);
  if (p->gate_groups <= 0 || p->d_k % p->gate_groups != 0)
    return fail(GDR_ERR_INVALID_ARG, "gate_groups=%d must divide d_k=%d", p->gate_groups, p->d_k);
  if (p->in_dtype != GDR_F32 && p->in_dtype != GDR_BF16)
    return fail(GDR_ERR_INVALID_ARG, "in_dtype=%d is not a gdr_dtype", p->in_dtype);
  if (p->out_dtype != GDR_F32 && p->out_dtype != GDR_BF16)
    return fail(GDR_ERR_INVALID_ARG, "out_dtype=%d is not a gdr_dtype", p->out_dtype);
  if (p->beta_per_key_head != 0 && p->beta_per_key_head != 1)
    return fail(GDR_ERR_INVALID_ARG, "beta_per_key_head=%d must be 0 or 1", p->beta_per_key_head);
  // every flat element index must fit in int64 and each kernel's per-tensor
  // token count in int32
  const double elems = (double)p->B * p->T * (double)(p->H_v > p->H_k ? p->H_v : p->H_k) *
                       (double)(p->d_k > p->d_v ? p->d_k : p->d_v);
  if (elems > 9.0e15 || (double)p->B * p->T > 2147483647.0)
    return fail(GDR_ERR_INVALID_ARG, "problem too large (B*T=%lld)", (long long)p->B * p->T);
  // Launch geometry: the batch and head indices are grid dimensions z and y
  // (at most 65535 each), and no grid dimension may count 2^32 work items.
  if (p->B > 65535 || p->H_v > 65535)
    return fail(GDR_ERR_UNSUPPORTED, "B=%d H_v=%d: at most 65535 each", p->B, p->H_v);
  if (!(p->d_k == 64 || p->d_k == 128 || p->d_k == 256))
    return fail(GDR_ERR_UNSUPPORTED, "d_k=%d: libgdr supports d_k in {64, 128, 256}", p->d_k);
  if (p->d_v % 16 != 0) return fail(GDR_ERR_UNSUPPORTED, "d_v=%d: must be a multiple of 16", p->d_v);
  if (chunked) {
    if (p->chunk <= 0) return fail(GDR_ERR_INVALID_ARG, "chunk=%d must be > 0", p->chunk);
    if (p->solve != GDR_SOLVE_EXACT && p->solve != GDR_SOLVE_NEUMANN)
      return fail(GDR_ERR_INVALID_ARG, "solve=%d is not a gdr_solve", p->solve);
    if (p->solve == GDR_SOLVE_NEUMANN) {
      if (p->neumann_order < 0 || p->neumann_residual_steps < 0)
        return fail(GDR_ERR_INVALID_ARG, "neumann_order=%d residual_steps=%d must be >= 0", p->neumann_order,
                    p->neumann_residual_steps);
      if (p->neumann_order > 1024 || p->neumann_residual_steps > 16)
        return fail(GDR_ERR_INVALID_ARG, "neumann_order=%d residual_steps=%d too large", p->neumann_order,
                    p->neumann_residual_steps);
    }
    if (!(p->chunk == 64 || p->chunk == 128))
      return fail(GDR_ERR_UNSUPPORTED, "chunk=%d: libgdr supports chunk in {64, 128}", p->chunk);
    // prep: one 256-thread workgroup per chunk along x; scan: one 512-thread
    // workgroup per (batch, value head, tile of at least 16 value columns)
    const long long n_c = ((long long)p->T + p->chunk - 1) / p->chunk;
    const long long scan_units = (long long)p->B * p->H_v * (p->d_v / 16);
    if (n_c * 256 >= (1LL << 32) || scan_units * 512 >= (1LL << 32))
      return fail(GDR_ERR_UNSUPPORTED, "T=%d chunks or B*H_v*d_v/16=%lld tiles exceed a launch", p->T, scan_units);
    const int beta_heads_per_key = p->beta_per_key_head ? 1 : p->H_v / p->H_k;
    if (p->chunk * beta_heads_per_key > 1024)
      return fail(GDR_ERR_UNSUPPORTED, "chunk * (H_v / H_k) = %d: at most 1024 beta values per chunk",
                  p->chunk * beta_heads_per_key);
    if (!gdr::prep_supported(p->chunk, p->d_k, p->gate_groups) ||
        gdr::scan_choose_bv(p->B, p->H_v, p->chunk, p->d_k, p->d_v, p->in_dtype == GDR_BF16) == 0)
      return fail(GDR_ERR_UNSUPPORTED, "chunk=%d d_k=%d G=%d exceeds the 160 KiB LDS budget", p->chunk, p->d_k,
                  p->gate_groups);
  }
  return GDR_OK;
}

gdr_status check_ptr(const void *ptr, const char *name, bool required, uintptr_t align = 16) {
  if (!ptr) {
    if (required) return fail(GDR_ERR_INVALID_ARG, "%s is NULL", name);
    return GDR_OK;
  }
  if (!aligned(ptr, align)) return fail(GDR_ERR_INVALID_ARG, "%s is not %d-byte aligned", name, (int)align);
  return GDR_OK;
}

gdr::WsLayout layout_of(const gdr_problem *p) {
  const int nc = (int)(((size_t)p->T + p->chunk - 1) / p->chunk);
  const int hb = p->beta_per_key_head ? p->H_k : p->H_v;
  return gdr::ws_layout(p->B, p->H_k, hb, nc, p->chunk, p->d_k, p->in_dtype == GDR_BF16);
}

size_t ws_bytes(const gdr_problem *p) { return layout_of(p).total; }

gdr::ChunkArgs make_chunk_args(const gdr_problem *p, void *workspace) {
  gdr::ChunkArgs a{};
  a.B = p->B;
  a.T = p->T;
  a.H_k = p->H_k;
  a.H_v = p->H_v;
  a.d_k = p->d_k;
  a.d_v = p->d_v;
  a.C = p->chunk;
  a.G = p->gate_groups;
  a.gshift = log2_exact(p->d_k / p->gate_groups);
  a.H_beta = p->beta_per_key_head ? p->H_k : p->H_v;
  a.N_c = (p->T + p->chunk - 1) / p->chunk;
  a.beta_per_key_head = p->beta_per_key_head;
  a.solve = p->solve;
  a.order = p->neumann_order;
  a.residual = p->neumann_residual_steps;
  a.ws = static_cast<unsigned char *>(workspace);
  a.wl = layout_of(p);
  return a;
}

gdr_status launched(hipError_t e, const char *what) {
  if (e != hipSuccess) return fail(GDR_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return GDR_OK;
}

}  // namespace

extern "C" {

size_t gdr_chunk_fwd_workspace_size(const gdr_problem *p) {
  if (check_problem(p, true) != GDR_OK) return 0;
  return ws_bytes(p);
}

gdr_status gdr_chunk_workspace_layout(const gdr_problem *p, size_t *offsets) {
  gdr_status s = check_problem(p, true);
  if (s != GDR_OK) return s;
  if (!offsets) return fail(GDR_ERR_INVALID_ARG, "offsets is NULL");
  const gdr::WsLayout w = layout_of(p);
  for (int r = 0; r < 6; ++r) offsets[r] = w.off[r];
  offsets[6] = w.total;
  return GDR_OK;
}

gdr_status gdr_chunk_prepare(const gdr_problem *p, const void *q, const void *k, const void *beta,
                             const void *log_alpha, void *workspace, size_t workspace_bytes, void *stream) {
  gdr_status s = check_problem(p, true);
  if (s != GDR_OK) return s;
  if (p->B == 0 || p->T == 0) return GDR_OK;
  if ((s = check_ptr(q, "q", true)) || (s = check_ptr(k, "k", true)) || (s = check_ptr(beta, "beta", true)) ||
      (s = check_ptr(log_alpha, "log_alpha", true)) || (s = check_ptr(workspace, "workspace", true, 256)))
    return s;
  if (workspace_bytes < ws_bytes(p))
    return fail(GDR_ERR_WORKSPACE, "workspace_bytes=%zu < required %zu", workspace_bytes, ws_bytes(p));
  gdr::ChunkArgs a = make_chunk_args(p, workspace);
  a.q = q;
  a.k = k;
  a.beta = beta;
  a.log_alpha = log_alpha;
  return launched(gdr::launch_prep(a, p->in_dtype == GDR_BF16, static_cast<hipStream_t>(stream)), "prep kernel");
}

namespace {

// Shared by gdr_chunk_fwd (prepare + scan) and gdr_chunk_scan (scan only).
gdr_status chunk_forward(const gdr_problem *p, const void *q, const void *k, const void *v, const void *beta,
                         const void *log_alpha, const float *h0, void *o, float *hT, const void *workspace,
                         size_t workspace_bytes, void *stream, bool prepare) {
  gdr_status s = check_problem(p, true);
  if (s != GDR_OK) return s;
  if ((s = check_ptr(h0, "h0", false)) || (s = check_ptr(hT, "hT", false))) return s;
  if (p->B == 0) return GDR_OK;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const bool in_bf16 = p->in_dtype == GDR_BF16, out_bf16 = p->out_dtype == GDR_BF16;
  if (p->T == 0) {
    // No tokens: the final state is the initial one.  The scan kernel over
    // zero chunks writes hT from h0 (or zeros) and touches nothing else.
    if (!hT) return GDR_OK;
    gdr::ChunkArgs a = make_chunk_args(p, nullptr);
    a.h0 = h0;
    a.hT = hT;
    return launched(gdr::launch_scan(a, in_bf16, out_bf16, st), "scan kernel");
  }
  if ((s = check_ptr(q, "q", prepare)) || (s = check_ptr(k, "k", prepare)) || (s = check_ptr(v, "v", true)) ||
      (s = check_ptr(beta, "beta", prepare)) || (s = check_ptr(log_alpha, "log_alpha", prepare)) ||
      (s = check_ptr(o, "o", true)) || (s = check_ptr(workspace, "workspace", true, 256)))
    return s;
  if (workspace_bytes < ws_bytes(p))
    return fail(GDR_ERR_WORKSPACE, "workspace_bytes=%zu < required %zu", workspace_bytes, ws_bytes(p));
  gdr::ChunkArgs a = make_chunk_args(p, const_cast<void *>(workspace));
  a.q = q;
  a.k = k;
  a.v = v;
  a.beta = beta;
  a.log_alpha = log_alpha;
  a.h0 = h0;
  a.o = o;
  a.hT = hT;
  if (prepare && (s = launched(gdr::launch_prep(a, in_bf16, st), "prep kernel")) != GDR_OK) return s;
  return launched(gdr::launch_scan(a, in_bf16, out_bf16, st), "scan kernel");
}

}  // namespace

gdr_status gdr_chunk_fwd(const gdr_problem *p, const void *q, const void *k, const void *v, const void *beta,
                         const void *log_alpha, const float *h0, void *o, float *hT, void *workspace,
                         size_t workspace_bytes, void *stream) {
  return chunk_forward(p, q, k, v, beta, log_alpha, h0, o, hT, workspace, workspace_bytes, stream, true);
}

gdr_status gdr_chunk_scan(const gdr_problem *p, const void *v, const float *h0, void *o, float *hT,
                          const void *workspace, size_t workspace_bytes, void *stream) {
  return chunk_forward(p, nullptr, nullptr, v, nullptr, nullptr, h0, o, hT, workspace, workspace_bytes, stream,
                       false);
}

gdr_status gdr_recurrent_step(const gdr_problem *p, const void *q, const void *k, const void *v, const void *beta,
                              const void *log_alpha, float *state, void *o, void *stream) {
  gdr_status s = check_problem(p, false);
  if (s != GDR_OK) return s;
  if (p->B == 0 || p->T == 0) return GDR_OK;
  if ((s = check_ptr(q, "q", true)) || (s = check_ptr(k, "k", true)) || (s = check_ptr(v, "v", true)) ||
      (s = check_ptr(beta, "beta", true)) || (s = check_ptr(log_alpha, "log_alpha", true)) ||
      (s = check_ptr(state, "state", true)) || (s = check_ptr(o, "o", true)))
    return s;
  gdr::StepArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.beta = beta;
  a.log_alpha = log_alpha;
  a.state = state;
  a.o = o;
  a.B = p->B;
  a.T = p->T;
  a.H_k = p->H_k;
  a.H_v = p->H_v;
  a.d_k = p->d_k;
  a.d_v = p->d_v;
  a.G = p->gate_groups;
  a.gshift = log2_exact(p->d_k / p->gate_groups);
  a.beta_per_key_head = p->beta_per_key_head;
  return launched(gdr::launch_step(a, p->in_dtype == GDR_BF16, p->out_dtype == GDR_BF16, static_cast<hipStream_t>(stream)),
                  "recurrent kernel");
}

const char *gdr_status_string(gdr_status s) {
  switch (s) {
    case GDR_OK: return "GDR_OK";
    case GDR_ERR_INVALID_ARG: return "GDR_ERR_INVALID_ARG";
    case GDR_ERR_UNSUPPORTED: return "GDR_ERR_UNSUPPORTED";
    case GDR_ERR_WORKSPACE: return "GDR_ERR_WORKSPACE";
    case GDR_ERR_HIP: return "GDR_ERR_HIP";
  }
  return "GDR_ERR_UNKNOWN";
}

const char *gdr_last_error(void) { return g_err.c_str(); }

}  // extern "C"
