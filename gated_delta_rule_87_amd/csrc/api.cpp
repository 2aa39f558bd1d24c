// C ABI of libgdr.so (declared in include/gdr.h): argument validation,
// workspace sizing and launch sequencing.  Nothing here allocates device
// memory or synchronises; every check runs before the first launch.
#include <hip/hip_runtime_api.h>

#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <mutex>
#include <set>
#include <string>
#include <utility>

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

// Chunk size 16 runs the C = 32 path on a padded sequence: every 16 tokens
// followed by 16 identity tokens (csrc/pad.hip).
gdr_problem padded16(const gdr_problem *p) {
  gdr_problem q = *p;
  q.chunk = 32;
  q.T = 32 * ((p->T + 15) / 16);
  return q;
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
    if (p->solve != GDR_SOLVE_EXACT && p->solve != GDR_SOLVE_NEUMANN && p->solve != GDR_SOLVE_BLOCK_NEUMANN)
      return fail(GDR_ERR_INVALID_ARG, "solve=%d is not a gdr_solve", p->solve);
    if (p->solve != GDR_SOLVE_EXACT) {
      if (p->neumann_order < 0 || p->neumann_residual_steps < 0)
        return fail(GDR_ERR_INVALID_ARG, "neumann_order=%d residual_steps=%d must be >= 0", p->neumann_order,
                    p->neumann_residual_steps);
      if (p->neumann_order > 1024 || p->neumann_residual_steps > 16)
        return fail(GDR_ERR_INVALID_ARG, "neumann_order=%d residual_steps=%d too large", p->neumann_order,
                    p->neumann_residual_steps);
    }
    if (p->chunk == 16) {
      // runs as 32-token chunks whose second halves are identity tokens
      const long long tp = 32LL * ((p->T + 15) / 16);
      if (tp > 2147483647LL || (double)p->B * (double)tp > 2147483647.0)
        return fail(GDR_ERR_UNSUPPORTED, "chunk=16: the padded sequence (2 T tokens) is too long");
      const gdr_problem pp = padded16(p);
      return check_problem(&pp, true);
    }
    if (!(p->chunk == 32 || p->chunk == 64 || p->chunk == 128))
      return fail(GDR_ERR_UNSUPPORTED, "chunk=%d: libgdr supports chunk in {16, 32, 64, 128}", p->chunk);
    if (p->chunk == 32 && p->d_v % 32 != 0)
      return fail(GDR_ERR_UNSUPPORTED, "chunk=32 needs d_v a multiple of 32 (d_v=%d)", p->d_v);
    // prep: one 256-thread workgroup per chunk along x; scan: one 512-thread
    // workgroup per (batch, value head, tile of at least 16 value columns)
    const long long n_c = ((long long)p->T + p->chunk - 1) / p->chunk;
    const long long scan_units = (long long)p->B * p->H_v * (p->d_v / 16);
    if (n_c * 256 >= (1LL << 32) || scan_units * 512 >= (1LL << 32))
      return fail(GDR_ERR_UNSUPPORTED, "T=%d chunks or B*H_v*d_v/16=%lld tiles exceed a launch", p->T, scan_units);
    // The scan addresses the rows of v and o within one chunk with 32-bit
    // byte offsets from the chunk's first row: C rows of H_v * d_v elements
    // of at most 4 bytes must stay below 4 GiB.
    if ((long long)p->chunk * p->H_v * p->d_v * 4 >= (1LL << 32))
      return fail(GDR_ERR_UNSUPPORTED, "chunk * H_v * d_v = %lld: one chunk of v or o must stay below 2^30 elements",
                  (long long)p->chunk * p->H_v * p->d_v);
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

// Chunk size 16: the padded copies of the inputs and of o, after the padded
// problem's own workspace (offsets from the workspace start, 256-aligned).
struct Pad16Layout {
  size_t q, k, v, beta, la, reset, o, end;
};
gdr::WsLayout layout_of(const gdr_problem *p);
Pad16Layout pad16_layout(const gdr_problem *p) {
  const gdr_problem pp = padded16(p);
  const size_t rows = (size_t)p->B * pp.T;
  const size_t es = p->in_dtype == GDR_BF16 ? 2 : 4, os = p->out_dtype == GDR_BF16 ? 2 : 4;
  const size_t hb = p->beta_per_key_head ? p->H_k : p->H_v;
  Pad16Layout L;
  size_t at = layout_of(&pp).total;
  auto take = [&](size_t bytes) {
    const size_t o = at;
    at = (at + bytes + 255) & ~(size_t)255;
    return o;
  };
  L.q = take(rows * p->H_k * p->d_k * es);
  L.k = take(rows * p->H_k * p->d_k * es);
  L.v = take(rows * p->H_v * p->d_v * es);
  L.beta = take(rows * hb * es);
  L.la = take(rows * p->H_k * p->gate_groups * es);
  L.reset = take(rows);
  L.o = take(rows * p->H_v * p->d_v * os);
  L.end = at;
  return L;
}

gdr::WsLayout layout_of(const gdr_problem *p) {
  if (p->chunk == 16) {
    const gdr_problem pp = padded16(p);
    gdr::WsLayout w = layout_of(&pp);
    w.total = pad16_layout(p).end;
    return w;
  }
  const int nc = (int)(((size_t)p->T + p->chunk - 1) / p->chunk);
  const int hb = p->beta_per_key_head ? p->H_k : p->H_v;
  gdr::WsLayout w = gdr::ws_layout(p->B, p->H_k, hb, nc, p->chunk, p->d_k, p->in_dtype == GDR_BF16);
  w.seg_bytes = gdr::scan_seg_bytes(p->B, p->H_v, nc, p->d_k, p->d_v, p->chunk, p->in_dtype != GDR_BF16);
  w.total = w.seg_off + ((w.seg_bytes + 255) & ~(size_t)255);
  return w;
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

// Chunk size 16: the key-side inputs (each nullable) to their padded copies.
gdr_status pad_inputs16(const gdr_problem *p, const gdr_problem &pp, const Pad16Layout &L, unsigned char *ws,
                        const void *q, const void *k, const void *beta, const void *log_alpha, hipStream_t st) {
  const size_t es = p->in_dtype == GDR_BF16 ? 2 : 4;
  const size_t hb = p->beta_per_key_head ? p->H_k : p->H_v;
  const struct {
    const void *src;
    size_t off, row;
  } t[4] = {{q, L.q, (size_t)p->H_k * p->d_k * es},
            {k, L.k, (size_t)p->H_k * p->d_k * es},
            {beta, L.beta, hb * es},
            {log_alpha, L.la, (size_t)p->H_k * p->gate_groups * es}};
  for (const auto &x : t) {
    if (!x.src) continue;
    gdr_status s = launched(gdr::launch_pad_rows(ws + x.off, x.src, x.row, p->B, p->T, pp.T, false, st), "pad kernel");
    if (s != GDR_OK) return s;
  }
  return GDR_OK;
}

}  // namespace

namespace gdr {

hipError_t allow_full_lds(const void *kernel) {
  static std::mutex mu;
  static std::set<std::pair<const void *, int>> done;   // (kernel, device) pairs already raised
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lock(mu);
  if (done.count({kernel, dev})) return hipSuccess;
  e = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
  if (e == hipSuccess) done.insert({kernel, dev});
  return e;
}

}  // namespace gdr

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
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (p->chunk == 16) {
    const gdr_problem pp = padded16(p);
    const Pad16Layout L = pad16_layout(p);
    unsigned char *ws = static_cast<unsigned char *>(workspace);
    if ((s = pad_inputs16(p, pp, L, ws, q, k, beta, log_alpha, st)) != GDR_OK) return s;
    gdr::ChunkArgs a = make_chunk_args(&pp, workspace);
    a.q = ws + L.q;
    a.k = ws + L.k;
    a.beta = ws + L.beta;
    a.log_alpha = ws + L.la;
    return launched(gdr::launch_prep(a, p->in_dtype == GDR_BF16, st), "prep kernel");
  }
  gdr::ChunkArgs a = make_chunk_args(p, workspace);
  a.q = q;
  a.k = k;
  a.beta = beta;
  a.log_alpha = log_alpha;
  return launched(gdr::launch_prep(a, p->in_dtype == GDR_BF16, st), "prep kernel");
}

}  // extern "C"

namespace gdr {

// Chunk size 16: pad the inputs into the workspace, run the C = 32 path on
// the padded sequence (its own workspace at the front), gather o back.  The
// final state is unaffected by the identity tokens.
gdr_status chunk_forward16(const gdr_problem *p, const void *q, const void *k, const void *v, const void *beta,
                           const void *log_alpha, const float *h0, void *o, float *hT, const void *workspace,
                           size_t workspace_bytes, void *stream, bool prepare, const gdr_layer_opts *opts,
                           void *states) {
  const gdr_problem pp = padded16(p);
  if (states) return set_error(GDR_ERR_UNSUPPORTED, "chunk=16: the training forward runs at chunk 64");
  if (p->B == 0 || p->T == 0)
    return chunk_forward(&pp, q, k, v, beta, log_alpha, h0, o, hT, workspace, workspace_bytes, stream, prepare, opts,
                         nullptr);
  gdr_status s;
  if ((s = check_ptr(q, "q", prepare)) || (s = check_ptr(k, "k", prepare)) || (s = check_ptr(v, "v", true)) ||
      (s = check_ptr(beta, "beta", prepare)) || (s = check_ptr(log_alpha, "log_alpha", prepare)) ||
      (s = check_ptr(o, "o", true)) || (s = check_ptr(workspace, "workspace", true, 256)))
    return s;
  size_t need = 0;
  if ((s = workspace_bytes_of(p, &need)) != GDR_OK) return s;
  if (workspace_bytes < need) return set_error(GDR_ERR_WORKSPACE, "workspace_bytes is below gdr_chunk_fwd_workspace_size");
  hipStream_t st = static_cast<hipStream_t>(stream);
  const Pad16Layout L = pad16_layout(p);
  unsigned char *ws = static_cast<unsigned char *>(const_cast<void *>(workspace));
  const size_t es = p->in_dtype == GDR_BF16 ? 2 : 4, os = p->out_dtype == GDR_BF16 ? 2 : 4;
  if (prepare && (s = pad_inputs16(p, pp, L, ws, q, k, beta, log_alpha, st)) != GDR_OK) return s;
  if ((s = launched(launch_pad_rows(ws + L.v, v, (size_t)p->H_v * p->d_v * es, p->B, p->T, pp.T, false, st),
                    "pad kernel")) != GDR_OK)
    return s;
  gdr_layer_opts o2{};
  if (opts) {
    o2 = *opts;
    if (opts->reset) {
      if ((s = launched(launch_pad_rows(ws + L.reset, opts->reset, 1, p->B, p->T, pp.T, false, st), "pad kernel")) !=
          GDR_OK)
        return s;
      o2.reset = ws + L.reset;
    }
  }
  s = chunk_forward(&pp, ws + L.q, ws + L.k, ws + L.v, ws + L.beta, ws + L.la, h0, ws + L.o, hT, workspace,
                    ws_bytes(&pp), stream, prepare, opts ? &o2 : nullptr, nullptr);
  if (s != GDR_OK) return s;
  return launched(launch_pad_rows(o, ws + L.o, (size_t)p->H_v * p->d_v * os, p->B, p->T, pp.T, true, st),
                  "unpad kernel");
}

// Shared by gdr_chunk_fwd (prepare + scan), gdr_chunk_scan (scan only) and
// the entry point that brings its own scratch (noalloc.hip).
gdr_status chunk_forward(const gdr_problem *p, const void *q, const void *k, const void *v, const void *beta,
                         const void *log_alpha, const float *h0, void *o, float *hT, const void *workspace,
                         size_t workspace_bytes, void *stream, bool prepare, const gdr_layer_opts *opts,
                         void *states) {
  gdr_status s = check_problem(p, true);
  if (s != GDR_OK) return s;
  if (p->chunk == 16) return chunk_forward16(p, q, k, v, beta, log_alpha, h0, o, hT, workspace, workspace_bytes,
                                             stream, prepare, opts, states);
  if ((s = check_ptr(h0, "h0", false)) || (s = check_ptr(hT, "hT", false)) || (s = check_ptr(states, "states", false)))
    return s;
  const bool mom = opts && opts->momentum != 0.f;
  if (opts && !std::isfinite(opts->momentum))
    return fail(GDR_ERR_INVALID_ARG, "momentum=%g is not finite", (double)opts->momentum);
  if (mom && ((s = check_ptr(opts->z0, "z0", false)) || (s = check_ptr(opts->zT, "zT", false)))) return s;
  if (p->B == 0) return GDR_OK;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const bool in_bf16 = p->in_dtype == GDR_BF16, out_bf16 = p->out_dtype == GDR_BF16;
  if (p->T == 0) {
    // No tokens: the final state is the initial one.  The scan kernel over
    // zero chunks writes hT from h0 (and zT from z0, or zeros) and touches
    // nothing else.
    if (!hT && !(mom && opts->zT)) return GDR_OK;
    gdr::ChunkArgs a = make_chunk_args(p, nullptr);
    a.h0 = h0;
    a.hT = hT;
    if (mom) {
      a.momentum = opts->momentum;
      a.z0 = opts->z0;
      a.zT = opts->zT;
    }
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
  a.states = states;
  if (opts) {
    a.reset = opts->reset;
    if (mom) {
      a.momentum = opts->momentum;
      a.z0 = opts->z0;
      a.zT = opts->zT;
    }
  }
  if (prepare && (s = launched(gdr::launch_prep(a, in_bf16, st), "prep kernel")) != GDR_OK) return s;
  return launched(gdr::launch_scan(a, in_bf16, out_bf16, st), "scan kernel");
}

gdr_status workspace_bytes_of(const gdr_problem *p, size_t *bytes) {
  gdr_status s = check_problem(p, true);
  if (s != GDR_OK) return s;
  *bytes = ws_bytes(p);
  return GDR_OK;
}

gdr_status set_error(gdr_status s, const char *text) { return fail(s, "%s", text); }

}  // namespace gdr

extern "C" {

gdr_status gdr_chunk_fwd(const gdr_problem *p, const void *q, const void *k, const void *v, const void *beta,
                         const void *log_alpha, const float *h0, void *o, float *hT, void *workspace,
                         size_t workspace_bytes, void *stream) {
  return gdr::chunk_forward(p, q, k, v, beta, log_alpha, h0, o, hT, workspace, workspace_bytes, stream, true,
                            nullptr);
}

gdr_status gdr_chunk_fwd_ex(const gdr_problem *p, const gdr_layer_opts *opts, const void *q, const void *k,
                            const void *v, const void *beta, const void *log_alpha, const float *h0, void *o,
                            float *hT, void *workspace, size_t workspace_bytes, void *stream) {
  return gdr::chunk_forward(p, q, k, v, beta, log_alpha, h0, o, hT, workspace, workspace_bytes, stream, true,
                            opts);
}

}  // extern "C"

namespace {

// Training forward and backward: the shapes and solve the backward supports.
gdr_status check_train(const gdr_problem *p) {
  gdr_status s = check_problem(p, true);
  if (s != GDR_OK) return s;
  if (!gdr::bwd_supported(p->chunk, p->d_k, p->d_v))
    return fail(GDR_ERR_UNSUPPORTED, "chunk=%d d_k=%d d_v=%d: the backward pass supports chunk 64, d_k in {64, 128} "
                "and d_v a multiple of 32", p->chunk, p->d_k, p->d_v);
  if (p->solve != GDR_SOLVE_EXACT)
    return fail(GDR_ERR_UNSUPPORTED, "solve=%d: the backward pass differentiates the exact in-chunk solve", p->solve);
  return GDR_OK;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Backward workspace: the forward's six operand regions (holding the reverse
// scan's operands), then A_c and G_c in fp32, X, and dS_c of every chunk.
struct BwdLayout {
  gdr::WsLayout ops;
  size_t au_off, gu_off, x_off, ds_off, total;
};

BwdLayout bwd_layout_of(const gdr_problem *p) {
  const size_t nc = ((size_t)p->T + p->chunk - 1) / p->chunk;
  const int hb = p->beta_per_key_head ? p->H_k : p->H_v;
  BwdLayout L;
  L.ops = gdr::ws_layout(p->B, p->H_k, hb, (int)nc, p->chunk, p->d_k, p->in_dtype == GDR_BF16);
  const size_t cc = (size_t)p->chunk * p->chunk * 4;
  size_t at = L.ops.total;
  L.au_off = at;
  at = align256(at + (size_t)p->B * hb * nc * cc);
  L.gu_off = at;
  at = align256(at + (size_t)p->B * p->H_k * nc * cc);
  L.x_off = at;
  const size_t wb = p->in_dtype == GDR_BF16 ? 2 : 4;   // X and dS_c: fp16 for bf16 inputs
  at = align256(at + (size_t)p->B * p->T * p->H_v * p->d_v * wb);
  L.ds_off = at;
  at = align256(at + (size_t)p->B * p->H_v * nc * p->d_k * p->d_v * wb);
  L.total = at;
  return L;
}

size_t states_bytes(const gdr_problem *p) {
  const size_t nc = ((size_t)p->T + p->chunk - 1) / p->chunk;
  return (size_t)p->B * p->H_v * nc * p->d_k * p->d_v * (p->in_dtype == GDR_BF16 ? 2 : 4);
}

}  // namespace

extern "C" {

size_t gdr_chunk_states_size(const gdr_problem *p) {
  if (check_train(p) != GDR_OK) return 0;
  return states_bytes(p);
}

gdr_status gdr_chunk_fwd_train(const gdr_problem *p, const void *q, const void *k, const void *v, const void *beta,
                               const void *log_alpha, const float *h0, void *o, float *hT, void *states,
                               void *workspace, size_t workspace_bytes, void *stream) {
  gdr_status s = check_train(p);
  if (s != GDR_OK) return s;
  if ((s = check_ptr(states, "states", p->B > 0 && p->T > 0))) return s;
  return gdr::chunk_forward(p, q, k, v, beta, log_alpha, h0, o, hT, workspace, workspace_bytes, stream, true,
                            nullptr, p->T > 0 ? states : nullptr);
}

size_t gdr_chunk_bwd_workspace_size(const gdr_problem *p) {
  if (check_train(p) != GDR_OK) return 0;
  return bwd_layout_of(p).total;
}

gdr_status gdr_chunk_bwd(const gdr_problem *p, const void *q, const void *k, const void *v, const void *beta,
                         const void *log_alpha, const void *states, const void *d_o, const float *dhT, float *dq,
                         float *dk, float *dv, float *dbeta, float *dlog_alpha, float *dh0, void *workspace,
                         size_t workspace_bytes, void *stream) {
  gdr_status s = check_train(p);
  if (s != GDR_OK) return s;
  if ((s = check_ptr(dhT, "dhT", false)) || (s = check_ptr(dh0, "dh0", false))) return s;
  if (p->B == 0) return GDR_OK;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const bool in_bf16 = p->in_dtype == GDR_BF16, g_bf16 = p->out_dtype == GDR_BF16;
  gdr::ChunkArgs a = make_chunk_args(p, nullptr);
  gdr::BwdArgs g{};
  g.dhT = dhT;
  g.dh0 = dh0;
  if (p->T == 0) {
    // No tokens: dh0 = dhT.  The reverse scan over zero chunks writes only dh0.
    if (!dh0) return GDR_OK;
    return launched(gdr::launch_bwd_scan(a, g, in_bf16, g_bf16, st), "reverse scan kernel");
  }
  if ((s = check_ptr(q, "q", true)) || (s = check_ptr(k, "k", true)) || (s = check_ptr(v, "v", true)) ||
      (s = check_ptr(beta, "beta", true)) || (s = check_ptr(log_alpha, "log_alpha", true)) ||
      (s = check_ptr(states, "states", true)) || (s = check_ptr(d_o, "d_o", true)) ||
      (s = check_ptr(dq, "dq", true)) || (s = check_ptr(dk, "dk", true)) || (s = check_ptr(dv, "dv", true)) ||
      (s = check_ptr(dbeta, "dbeta", true, 4)) || (s = check_ptr(dlog_alpha, "dlog_alpha", true, 4)) ||
      (s = check_ptr(workspace, "workspace", true, 256)))
    return s;
  const BwdLayout L = bwd_layout_of(p);
  if (workspace_bytes < L.total)
    return fail(GDR_ERR_WORKSPACE, "workspace_bytes=%zu < required %zu", workspace_bytes, L.total);
  unsigned char *ws = static_cast<unsigned char *>(workspace);
  a.q = q;
  a.k = k;
  a.v = v;
  a.beta = beta;
  a.log_alpha = log_alpha;
  a.ws = ws;
  a.wl = L.ops;
  a.solve = GDR_SOLVE_EXACT;
  a.bwd = 1;
  a.au = reinterpret_cast<float *>(ws + L.au_off);
  a.gu = reinterpret_cast<float *>(ws + L.gu_off);
  g.d_o = d_o;
  g.states = states;
  g.dq = dq;
  g.dk = dk;
  g.dv = dv;
  g.dbeta = dbeta;
  g.dla = dlog_alpha;
  g.x = ws + L.x_off;
  g.dstates = ws + L.ds_off;
  if ((s = launched(gdr::launch_prep(a, in_bf16, st), "prep kernel (backward operands)")) != GDR_OK) return s;
  if ((s = launched(gdr::launch_bwd_scan(a, g, in_bf16, g_bf16, st), "reverse scan kernel")) != GDR_OK) return s;
  return launched(gdr::launch_bwd_grad(a, g, in_bf16, g_bf16, st), "gradient kernel");
}

gdr_status gdr_gated_rmsnorm(const gdr_problem *p, const void *o, const void *z, const float *weight, float eps,
                             void *y, void *stream) {
  gdr_status s = check_problem(p, false);
  if (s != GDR_OK) return s;
  if (!(eps >= 0.f) || !std::isfinite(eps)) return fail(GDR_ERR_INVALID_ARG, "eps=%g must be finite and >= 0", (double)eps);
  if (p->B == 0 || p->T == 0) return GDR_OK;
  if ((s = check_ptr(o, "o", true)) || (s = check_ptr(z, "z", true)) || (s = check_ptr(y, "y", true)) ||
      (s = check_ptr(weight, "weight", false, 4)))
    return s;
  const long long rows = (long long)p->B * p->T * p->H_v;
  if ((rows + 3) / 4 >= (1LL << 31)) return fail(GDR_ERR_UNSUPPORTED, "B*T*H_v=%lld rows exceed a launch", rows);
  return launched(gdr::launch_gated_rmsnorm(o, z, weight, eps, y, rows, p->d_v, p->out_dtype == GDR_BF16,
                                            p->in_dtype == GDR_BF16, static_cast<hipStream_t>(stream)),
                  "gated rmsnorm kernel");
}

gdr_status gdr_chunk_scan(const gdr_problem *p, const void *v, const float *h0, void *o, float *hT,
                          const void *workspace, size_t workspace_bytes, void *stream) {
  return gdr::chunk_forward(p, nullptr, nullptr, v, nullptr, nullptr, h0, o, hT, workspace, workspace_bytes, stream,
                            false, nullptr);
}

gdr_status gdr_recurrent_step(const gdr_problem *p, const void *q, const void *k, const void *v, const void *beta,
                              const void *log_alpha, float *state, void *o, void *stream) {
  return gdr_recurrent_step_ex(p, nullptr, q, k, v, beta, log_alpha, state, o, stream);
}

namespace {

gdr::StepArgs make_step_args(const gdr_problem *p, const void *q, const void *k, const void *v, const void *beta,
                             const void *log_alpha, void *state, void *o) {
  gdr::StepArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.beta = beta;
  a.log_alpha = log_alpha;
  a.state = static_cast<float *>(state);
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
  return a;
}

}  // namespace

gdr_status gdr_recurrent_step_ex(const gdr_problem *p, const gdr_step_opts *opts, const void *q, const void *k,
                                 const void *v, const void *beta, const void *log_alpha, void *state, void *o,
                                 void *stream) {
  gdr_status s = check_problem(p, false);
  if (s != GDR_OK) return s;
  const int fmt = opts ? opts->state_format : GDR_STATE_F32;
  if (fmt != GDR_STATE_F32 && fmt != GDR_STATE_E4M3)
    return fail(GDR_ERR_INVALID_ARG, "state_format=%d is not a gdr_state_format", fmt);
  if (fmt == GDR_STATE_E4M3) {
    if (!(p->d_v == 32 || p->d_v == 64 || p->d_v == 128))
      return fail(GDR_ERR_UNSUPPORTED, "d_v=%d: the E4M3 state supports d_v in {32, 64, 128}", p->d_v);
    if ((s = check_ptr(opts->state_scale, "state_scale", true, 4))) return s;
  }
  if (p->B == 0 || p->T == 0) return GDR_OK;
  if ((s = check_ptr(q, "q", true)) || (s = check_ptr(k, "k", true)) || (s = check_ptr(v, "v", true)) ||
      (s = check_ptr(beta, "beta", true)) || (s = check_ptr(log_alpha, "log_alpha", true)) ||
      (s = check_ptr(state, "state", true)) || (s = check_ptr(o, "o", true)) ||
      (opts && (s = check_ptr(opts->n_tokens, "n_tokens", false, 4))))
    return s;
  if (fmt == GDR_STATE_E4M3 && (s = check_ptr(state, "state", true, 256))) return s;
  gdr::StepArgs a = make_step_args(p, q, k, v, beta, log_alpha, state, o);
  if (opts) {
    a.n_tokens = opts->n_tokens;
    a.reset = opts->reset;
    a.scale = opts->state_scale;
  }
  const bool in_bf16 = p->in_dtype == GDR_BF16, out_bf16 = p->out_dtype == GDR_BF16;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (fmt == GDR_STATE_E4M3) return launched(gdr::launch_step_e4m3(a, in_bf16, out_bf16, st), "recurrent kernel");
  return launched(gdr::launch_step(a, in_bf16, out_bf16, st), "recurrent kernel");
}

gdr_status gdr_verify(const gdr_problem *p, const void *q, const void *k, const void *v, const void *beta,
                      const void *log_alpha, const float *state, void *o, void *stream) {
  gdr_status s = check_problem(p, false);
  if (s != GDR_OK) return s;
  if (p->T > gdr::kVerifyMaxTokens)
    return fail(GDR_ERR_UNSUPPORTED, "T=%d drafted tokens: gdr_verify takes at most %d", p->T, gdr::kVerifyMaxTokens);
  if (p->B == 0 || p->T == 0) return GDR_OK;
  if ((s = check_ptr(q, "q", true)) || (s = check_ptr(k, "k", true)) || (s = check_ptr(v, "v", true)) ||
      (s = check_ptr(beta, "beta", true)) || (s = check_ptr(log_alpha, "log_alpha", true)) ||
      (s = check_ptr(state, "state", true)) || (s = check_ptr(o, "o", true)))
    return s;
  gdr::StepArgs a = make_step_args(p, q, k, v, beta, log_alpha, const_cast<float *>(state), o);
  return launched(gdr::launch_verify(a, p->in_dtype == GDR_BF16, p->out_dtype == GDR_BF16,
                                     static_cast<hipStream_t>(stream)),
                  "verify kernel");
}

gdr_status gdr_state_quantize(const gdr_problem *p, const float *state, void *codes, float *scale, void *stream) {
  gdr_status s = check_problem(p, false);
  if (s != GDR_OK) return s;
  if (p->d_v > 256) return fail(GDR_ERR_UNSUPPORTED, "d_v=%d: state conversion supports d_v <= 256", p->d_v);
  if (p->B == 0) return GDR_OK;
  if ((s = check_ptr(state, "state", true)) || (s = check_ptr(codes, "codes", true, 4)) ||
      (s = check_ptr(scale, "scale", true, 4)))
    return s;
  const long long rows = (long long)p->B * p->H_v * p->d_k;
  return launched(gdr::launch_state_quantize(state, static_cast<unsigned char *>(codes), scale, rows, p->d_v,
                                             static_cast<hipStream_t>(stream)),
                  "state quantize kernel");
}

gdr_status gdr_state_dequantize(const gdr_problem *p, const void *codes, const float *scale, float *state,
                                void *stream) {
  gdr_status s = check_problem(p, false);
  if (s != GDR_OK) return s;
  if (p->d_v > 256) return fail(GDR_ERR_UNSUPPORTED, "d_v=%d: state conversion supports d_v <= 256", p->d_v);
  if (p->B == 0) return GDR_OK;
  if ((s = check_ptr(state, "state", true)) || (s = check_ptr(codes, "codes", true, 4)) ||
      (s = check_ptr(scale, "scale", true, 4)))
    return s;
  const long long rows = (long long)p->B * p->H_v * p->d_k;
  return launched(gdr::launch_state_dequantize(static_cast<const unsigned char *>(codes), scale, state, rows, p->d_v,
                                               static_cast<hipStream_t>(stream)),
                  "state dequantize kernel");
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
