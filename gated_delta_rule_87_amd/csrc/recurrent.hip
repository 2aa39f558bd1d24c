// Token recurrence (stateful step-by-step decoding): for each of T tokens in
// order (Systolic Linear Attention, section 2.1, Eq. (2))
//   S <- F_t S;  u = v_t - S^T k_t;  S <- S + beta_t k_t u^T;  o_t = S^T q_t.
// One workgroup (four waves) per (batch, value head, 4 NQ value columns):
// thread t owns the four columns 4 (t % NQ) .. + 3 and RP consecutive state
// rows of row group t / NQ, in fp32 registers, so the state moves as 16-byte
// pieces of whole rows.  The two d_k reductions per token run over the row
// groups: shuffles within a wave, then one LDS exchange across the waves.
// The state is read once and written once per call.
#include "common.hpp"
#include "kernels.hpp"

namespace gdr {

constexpr int kStepThreads = 256;

template <typename TIn, typename TOut, int DK, int NQ>
__global__ __launch_bounds__(kStepThreads) void step_kernel(StepArgs a) {
  constexpr int NG = kStepThreads / NQ;       // row groups
  constexpr int RP = DK / NG;                 // rows per thread
  constexpr int NW = kStepThreads / 64;
  static_assert(RP >= 1 && DK % NG == 0, "rows per thread");
  __shared__ f32x4 red[2][NW][NQ];            // per-wave partial sums: u (buffer 0), o (buffer 1)

  const int tid = threadIdx.x, l = lane_id(), w = wave_id();
  const int cq = tid % NQ, rg = tid / NQ;
  const int col = blockIdx.x * 4 * NQ + 4 * cq, r0 = rg * RP;
  const int hv = blockIdx.y, b = blockIdx.z;
  const int R = a.H_v / a.H_k, hk = hv / R;
  const int hb = a.beta_per_key_head ? hk : hv;
  const int G = a.G, gs = a.gshift, T = a.T;
  const TIn *qp = reinterpret_cast<const TIn *>(a.q);
  const TIn *kp = reinterpret_cast<const TIn *>(a.k);
  const TIn *vp = reinterpret_cast<const TIn *>(a.v);
  const TIn *bp = reinterpret_cast<const TIn *>(a.beta);
  const TIn *lap = reinterpret_cast<const TIn *>(a.log_alpha);
  TOut *op = reinterpret_cast<TOut *>(a.o);

  f32x4 S[RP];
  float *srow = a.state + ((size_t)b * a.H_v + hv) * DK * a.d_v + (size_t)r0 * a.d_v + col;
#pragma unroll
  for (int i = 0; i < RP; ++i) S[i] = *reinterpret_cast<const f32x4 *>(srow + (size_t)i * a.d_v);

  // sum of x over all row groups, for this thread's four columns
  auto reduce = [&](f32x4 x, int buf) {
#pragma unroll
    for (int m = NQ; m < 64; m *= 2) {
#pragma unroll
      for (int e = 0; e < 4; ++e) x[e] += __shfl_xor(x[e], m);
    }
    if (l < NQ) red[buf][w][l] = x;
    __syncthreads();
    f32x4 s = red[buf][0][cq];
#pragma unroll
    for (int v = 1; v < NW; ++v) s += red[buf][v][cq];
    return s;
  };

  const int Tb = a.n_tokens ? min(max(a.n_tokens[b], 0), T) : T;   // this sequence's tokens
  for (int t = 0; t < Tb; ++t) {
    const size_t bt = (size_t)b * T + t;
    if (a.reset && a.reset[bt]) {              // a new document: the carried state is discarded
#pragma unroll
      for (int i = 0; i < RP; ++i) S[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    const TIn *krow = kp + (bt * a.H_k + hk) * DK + r0;
    const TIn *qrow = qp + (bt * a.H_k + hk) * DK + r0;
    const TIn *larow = lap + (bt * a.H_k + hk) * G;
    const float beta = ldf(bp + bt * (a.beta_per_key_head ? a.H_k : a.H_v) + hb);
    const TIn *vrow = vp + (bt * a.H_v + hv) * a.d_v + col;
    float kv[RP], qv[RP];
#pragma unroll
    for (int i = 0; i < RP; ++i) {
      kv[i] = ldf(krow + i);
      qv[i] = ldf(qrow + i);
    }
    f32x4 pk = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < RP; ++i) {
      const float f = __expf(ldf(larow + ((r0 + i) >> gs)));
      S[i] *= f;
      pk += S[i] * kv[i];
    }
    pk = reduce(pk, 0);
    f32x4 bu;
#pragma unroll
    for (int e = 0; e < 4; ++e) bu[e] = beta * (ldf(vrow + e) - pk[e]);
    f32x4 po = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < RP; ++i) {
      S[i] += kv[i] * bu;
      po += S[i] * qv[i];
    }
    po = reduce(po, 1);
    if (rg == 0) {
      TOut *orow = op + (bt * a.H_v + hv) * a.d_v + col;
#pragma unroll
      for (int e = 0; e < 4; ++e) st(orow + e, po[e]);
    }
  }
#pragma unroll
  for (int i = 0; i < RP; ++i) *reinterpret_cast<f32x4 *>(srow + (size_t)i * a.d_v) = S[i];
}

// 32 value columns per workgroup when d_v allows, else 16.
template <typename TIn, typename TOut, int NQ>
static hipError_t launch_step_q(const StepArgs &a, hipStream_t s) {
  dim3 grid(a.d_v / (4 * NQ), a.H_v, a.B);
  switch (a.d_k) {
    case 64: hipLaunchKernelGGL((step_kernel<TIn, TOut, 64, NQ>), grid, dim3(kStepThreads), 0, s, a); break;
    case 128: hipLaunchKernelGGL((step_kernel<TIn, TOut, 128, NQ>), grid, dim3(kStepThreads), 0, s, a); break;
    case 256: hipLaunchKernelGGL((step_kernel<TIn, TOut, 256, NQ>), grid, dim3(kStepThreads), 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <typename TIn, typename TOut>
static hipError_t launch_step_t(const StepArgs &a, hipStream_t s) {
  if (a.d_v % 32 == 0) return launch_step_q<TIn, TOut, 8>(a, s);
  return launch_step_q<TIn, TOut, 4>(a, s);
}

// ------------------------------------------------------ row-scaled E4M3 state
// A state stored in FP8 (Systolic Linear Attention, section 3.2, and its
// serving study: row-scaled E4M3): row i of S (the d_v values of key channel
// i) is kept as E4M3 codes c with one fp32 scale s_i = max_j |S_ij| / 448, so
// S_ij = value(c_ij) s_i.  Quantising takes x * (448 / max_j |S_ij|) in fp32
// (a correctly rounded division, then a correctly rounded product), clamps
// it to [-448, 448] and rounds it to E4M3 with round-to-nearest-even (the
// gfx950 conversion instruction); a row of zeros gets scale 0 and codes 0.

// fp32 -> E4M3 code of a value already scaled into [-448, 448]
__device__ __forceinline__ unsigned e4m3_pack4(float x0, float x1, float x2, float x3) {
  const auto clampv = [](float x) { return __builtin_amdgcn_fmed3f(x, kE4M3Max, -kE4M3Max); };
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(clampv(x0), clampv(x1), 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(clampv(x2), clampv(x3), w, true);
  return (unsigned)w;
}
__device__ __forceinline__ f32x4 e4m3_unpack4(unsigned w, float scale) {
  return f32x4{__builtin_amdgcn_cvt_f32_fp8((int)w, 0) * scale, __builtin_amdgcn_cvt_f32_fp8((int)w, 1) * scale,
               __builtin_amdgcn_cvt_f32_fp8((int)w, 2) * scale, __builtin_amdgcn_cvt_f32_fp8((int)w, 3) * scale};
}
// quantisation factor of a row from its largest magnitude
__device__ __forceinline__ float e4m3_row_inv(float amax) { return amax > 0.f ? kE4M3Max / amax : 0.f; }

// The recurrent step over an E4M3 state: one workgroup per (batch, value
// head) holds the whole d_k x d_v state in fp32 registers (row scaling needs
// all of a row, the step's reductions all of a column); with few heads in
// the batch it takes up to 1024 threads so that each carries few rows.  Thread t owns columns
// 4 (t % NQ) .. + 3 and RP rows; the state is dequantised once, stepped
// over the call's tokens in fp32 and quantised once at the end.
template <int DK, int NQ, bool kWide>
constexpr int e4m3_threads() { return kWide ? (DK * NQ < 1024 ? DK * NQ : 1024) : (DK * NQ < 256 ? DK * NQ : 256); }
template <typename TIn, typename TOut, int DK, int NQ, bool kWide>
__global__ __launch_bounds__((e4m3_threads<DK, NQ, kWide>())) void step_e4m3_kernel(StepArgs a) {
  constexpr int NTH = e4m3_threads<DK, NQ, kWide>();
  constexpr int NG = NTH / NQ;                // row groups
  constexpr int RP = DK / NG;                 // rows per thread
  constexpr int NW = NTH / 64;
  static_assert(RP >= 1 && DK % NG == 0 && NQ <= 64, "rows per thread");
  __shared__ f32x4 red[2][NW][NQ];

  const int tid = threadIdx.x, l = lane_id(), w = wave_id();
  const int cq = tid % NQ, rg = tid / NQ;
  const int col = 4 * cq, r0 = rg * RP;
  const int hv = blockIdx.x, b = blockIdx.y;
  const int R = a.H_v / a.H_k, hk = hv / R;
  const int hb = a.beta_per_key_head ? hk : hv;
  const int G = a.G, gs = a.gshift, T = a.T;
  const TIn *qp = reinterpret_cast<const TIn *>(a.q);
  const TIn *kp = reinterpret_cast<const TIn *>(a.k);
  const TIn *vp = reinterpret_cast<const TIn *>(a.v);
  const TIn *bp = reinterpret_cast<const TIn *>(a.beta);
  const TIn *lap = reinterpret_cast<const TIn *>(a.log_alpha);
  TOut *op = reinterpret_cast<TOut *>(a.o);

  const size_t unit = (size_t)b * a.H_v + hv;
  unsigned char *codes = reinterpret_cast<unsigned char *>(a.state) + unit * DK * a.d_v + (size_t)r0 * a.d_v + col;
  float *scale = a.scale + unit * DK + r0;
  f32x4 S[RP];
#pragma unroll
  for (int i = 0; i < RP; ++i) S[i] = e4m3_unpack4(*reinterpret_cast<const unsigned *>(codes + (size_t)i * a.d_v), scale[i]);

  auto reduce = [&](f32x4 x, int buf) {
#pragma unroll
    for (int m = NQ; m < 64; m *= 2) {
#pragma unroll
      for (int e = 0; e < 4; ++e) x[e] += __shfl_xor(x[e], m);
    }
    if (l < NQ) red[buf][w][l] = x;
    __syncthreads();
    f32x4 s = red[buf][0][cq];
#pragma unroll
    for (int v = 1; v < NW; ++v) s += red[buf][v][cq];
    __syncthreads();
    return s;
  };

  const int Tb = a.n_tokens ? min(max(a.n_tokens[b], 0), T) : T;
  for (int t = 0; t < Tb; ++t) {
    const size_t bt = (size_t)b * T + t;
    if (a.reset && a.reset[bt]) {
#pragma unroll
      for (int i = 0; i < RP; ++i) S[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    const TIn *krow = kp + (bt * a.H_k + hk) * DK + r0;
    const TIn *qrow = qp + (bt * a.H_k + hk) * DK + r0;
    const TIn *larow = lap + (bt * a.H_k + hk) * G;
    const float beta = ldf(bp + bt * (a.beta_per_key_head ? a.H_k : a.H_v) + hb);
    const TIn *vrow = vp + (bt * a.H_v + hv) * a.d_v + col;
    f32x4 pk = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < RP; ++i) {
      S[i] *= __expf(ldf(larow + ((r0 + i) >> gs)));
      pk += S[i] * ldf(krow + i);
    }
    pk = reduce(pk, 0);
    f32x4 bu;
#pragma unroll
    for (int e = 0; e < 4; ++e) bu[e] = beta * (ldf(vrow + e) - pk[e]);
    f32x4 po = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < RP; ++i) {
      S[i] += ldf(krow + i) * bu;
      po += S[i] * ldf(qrow + i);
    }
    po = reduce(po, 1);
    if (rg == 0) {
      TOut *orow = op + (bt * a.H_v + hv) * a.d_v + col;
#pragma unroll
      for (int e = 0; e < 4; ++e) st(orow + e, po[e]);
    }
  }
  // requantise: the NQ threads of a row group hold the row's d_v values
#pragma unroll
  for (int i = 0; i < RP; ++i) {
    float m = fmaxf(fmaxf(fabsf(S[i][0]), fabsf(S[i][1])), fmaxf(fabsf(S[i][2]), fabsf(S[i][3])));
#pragma unroll
    for (int s = 1; s < NQ; s *= 2) m = fmaxf(m, __shfl_xor(m, s));
    const float inv = e4m3_row_inv(m);
    *reinterpret_cast<unsigned *>(codes + (size_t)i * a.d_v) =
        e4m3_pack4(S[i][0] * inv, S[i][1] * inv, S[i][2] * inv, S[i][3] * inv);
    if (cq == 0) scale[i] = m / kE4M3Max;
  }
}

template <typename TIn, typename TOut, int NQ>
static hipError_t launch_step_e4m3_q(const StepArgs &a, hipStream_t s) {
  dim3 grid(a.H_v, a.B);
  // few (batch, head) workgroups: up to 1024 threads each, so each carries
  // few rows (latency); many: 256 threads, fewer waves in each reduction
  // (measured at B = 2 / 64 / 256, H = 32: 6.4 / 48 / 190 us per step with
  // 1024 threads, 9.8 / 43.6 / 173 us with 256)
  const bool wide = (long)a.B * a.H_v < 512;
#define GDR_E4M3(dk_)                                                                                         \
  if (wide)                                                                                                   \
    hipLaunchKernelGGL((step_e4m3_kernel<TIn, TOut, dk_, NQ, true>), grid, dim3(e4m3_threads<dk_, NQ, true>()), \
                       0, s, a);                                                                              \
  else                                                                                                        \
    hipLaunchKernelGGL((step_e4m3_kernel<TIn, TOut, dk_, NQ, false>), grid,                                   \
                       dim3(e4m3_threads<dk_, NQ, false>()), 0, s, a)
  switch (a.d_k) {
    case 64: GDR_E4M3(64); break;
    case 128: GDR_E4M3(128); break;
    case 256: GDR_E4M3(256); break;
    default: return hipErrorInvalidValue;
  }
#undef GDR_E4M3
  return hipGetLastError();
}

template <typename TIn, typename TOut>
static hipError_t launch_step_e4m3_t(const StepArgs &a, hipStream_t s) {
  switch (a.d_v) {
    case 32: return launch_step_e4m3_q<TIn, TOut, 8>(a, s);
    case 64: return launch_step_e4m3_q<TIn, TOut, 16>(a, s);
    case 128: return launch_step_e4m3_q<TIn, TOut, 32>(a, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_step_e4m3(const StepArgs &a, bool in_bf16, bool out_bf16, hipStream_t stream) {
  if (in_bf16) {
    if (out_bf16) return launch_step_e4m3_t<bf16, bf16>(a, stream);
    return launch_step_e4m3_t<bf16, float>(a, stream);
  }
  if (out_bf16) return launch_step_e4m3_t<float, bf16>(a, stream);
  return launch_step_e4m3_t<float, float>(a, stream);
}

// Stand-alone conversions of a state: one wave per row of d_v <= 256 values,
// lane l owning values 4 l .. 4 l + 3.
__global__ __launch_bounds__(256) void state_quantize_kernel(const float *x, unsigned char *codes, float *scale,
                                                             long long rows, int d_v) {
  const long long row = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const int l = lane_id();
  const bool mine = 4 * l < d_v;
  const float *xr = x + row * d_v;
  const float4 v = mine ? *reinterpret_cast<const float4 *>(xr + 4 * l) : make_float4(0.f, 0.f, 0.f, 0.f);
  float m = fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
#pragma unroll
  for (int s = 1; s < 64; s *= 2) m = fmaxf(m, __shfl_xor(m, s));
  const float inv = e4m3_row_inv(m);
  if (mine) *reinterpret_cast<unsigned *>(codes + row * d_v + 4 * l) = e4m3_pack4(v.x * inv, v.y * inv, v.z * inv, v.w * inv);
  if (l == 0) scale[row] = m / kE4M3Max;
}

__global__ __launch_bounds__(256) void state_dequantize_kernel(const unsigned char *codes, const float *scale, float *x,
                                                               long long rows, int d_v) {
  const long long row = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const int l = lane_id();
  if (4 * l >= d_v) return;
  const f32x4 v = e4m3_unpack4(*reinterpret_cast<const unsigned *>(codes + row * d_v + 4 * l), scale[row]);
  *reinterpret_cast<float4 *>(x + row * d_v + 4 * l) = make_float4(v[0], v[1], v[2], v[3]);
}

hipError_t launch_state_quantize(const float *x, unsigned char *codes, float *scale, long long rows, int d_v,
                                 hipStream_t stream) {
  hipLaunchKernelGGL(state_quantize_kernel, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, stream, x, codes, scale,
                     rows, d_v);
  return hipGetLastError();
}

hipError_t launch_state_dequantize(const unsigned char *codes, const float *scale, float *x, long long rows, int d_v,
                                   hipStream_t stream) {
  hipLaunchKernelGGL(state_dequantize_kernel, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, stream, codes, scale,
                     x, rows, d_v);
  return hipGetLastError();
}

hipError_t launch_step(const StepArgs &a, bool in_bf16, bool out_bf16, hipStream_t stream) {
  if (in_bf16) {
    if (out_bf16) return launch_step_t<bf16, bf16>(a, stream);
    return launch_step_t<bf16, float>(a, stream);
  }
  if (out_bf16) return launch_step_t<float, bf16>(a, stream);
  return launch_step_t<float, float>(a, stream);
}

}  // namespace gdr
