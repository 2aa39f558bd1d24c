// Token recurrence (stateful step-by-step decoding): for each of T tokens in
// order (Systolic Linear Attention, section 2.1, Eq. (2))
//   S <- F_t S;  u = v_t - S^T k_t;  S <- S + beta_t k_t u^T;  o_t = S^T q_t.
// One wave per (batch, value head, 16 value columns): lane l owns column
// l%16 and the quarter l/16 of the d_k rows of that column, in fp32 registers;
// the two d_k reductions per token are finished with cross-lane shuffles.
// The state is read once and written once per call.
#include "common.hpp"
#include "kernels.hpp"

namespace gdr {

template <typename TIn, typename TOut, int DK>
__global__ __launch_bounds__(64) void step_kernel(StepArgs a) {
  constexpr int RP = DK / 4;   // rows per lane
  const int l = lane_id();
  const int col = blockIdx.x * 16 + (l & 15), part = l >> 4;
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

  float S[RP];
  const size_t sbase = ((size_t)b * a.H_v + hv) * DK * a.d_v;
  const int r0 = part * RP;
#pragma unroll
  for (int i = 0; i < RP; ++i) S[i] = a.state[sbase + (size_t)(r0 + i) * a.d_v + col];

  for (int t = 0; t < T; ++t) {
    const size_t bt = (size_t)b * T + t;
    const TIn *krow = kp + (bt * a.H_k + hk) * DK + r0;
    const TIn *qrow = qp + (bt * a.H_k + hk) * DK + r0;
    const TIn *larow = lap + (bt * a.H_k + hk) * G;
    const float beta = ldf(bp + bt * (a.beta_per_key_head ? a.H_k : a.H_v) + hb);
    float kv[RP], qv[RP];
#pragma unroll
    for (int i = 0; i < RP; i += 8) {
      float x[8];
      ld8(krow + i, x);
#pragma unroll
      for (int e = 0; e < 8; ++e) kv[i + e] = x[e];
      ld8(qrow + i, x);
#pragma unroll
      for (int e = 0; e < 8; ++e) qv[i + e] = x[e];
    }
    float pk = 0.f;
#pragma unroll
    for (int i = 0; i < RP; ++i) {
      S[i] *= __expf(ldf(larow + ((r0 + i) >> gs)));
      pk += S[i] * kv[i];
    }
    pk += __shfl_xor(pk, 16);
    pk += __shfl_xor(pk, 32);
    const float u = ldf(vp + (bt * a.H_v + hv) * a.d_v + col) - pk;
    const float bu = beta * u;
    float po = 0.f;
#pragma unroll
    for (int i = 0; i < RP; ++i) {
      S[i] += kv[i] * bu;
      po += S[i] * qv[i];
    }
    po += __shfl_xor(po, 16);
    po += __shfl_xor(po, 32);
    if (part == 0) st(op + (bt * a.H_v + hv) * a.d_v + col, po);
  }
#pragma unroll
  for (int i = 0; i < RP; ++i) a.state[sbase + (size_t)(r0 + i) * a.d_v + col] = S[i];
}

template <typename TIn, typename TOut>
static hipError_t launch_step_t(const StepArgs &a, hipStream_t s) {
  dim3 grid(a.d_v / 16, a.H_v, a.B);
  switch (a.d_k) {
    case 64: hipLaunchKernelGGL((step_kernel<TIn, TOut, 64>), grid, dim3(64), 0, s, a); break;
    case 128: hipLaunchKernelGGL((step_kernel<TIn, TOut, 128>), grid, dim3(64), 0, s, a); break;
    case 256: hipLaunchKernelGGL((step_kernel<TIn, TOut, 256>), grid, dim3(64), 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
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
