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

  for (int t = 0; t < T; ++t) {
    const size_t bt = (size_t)b * T + t;
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

hipError_t launch_step(const StepArgs &a, bool in_bf16, bool out_bf16, hipStream_t stream) {
  if (in_bf16) {
    if (out_bf16) return launch_step_t<bf16, bf16>(a, stream);
    return launch_step_t<bf16, float>(a, stream);
  }
  if (out_bf16) return launch_step_t<float, bf16>(a, stream);
  return launch_step_t<float, float>(a, stream);
}

}  // namespace gdr
