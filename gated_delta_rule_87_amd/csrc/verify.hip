// Speculative verification (Systolic Linear Attention, section 3.2): the
// outputs of T <= 16 drafted tokens, read from a state that the call does
// not change, with the same block inversion as the chunk path -- the drafted
// tokens form one chunk of the WY form (Table 2):
//   Lambda = prefix sum of log alpha over the drafted tokens;
//   G_tj = sum_i k_ti k_ji e^{Lambda_ti - Lambda_ji} (t > j),
//   L_tj = sum_i q_ti k_ji e^{Lambda_ti - Lambda_ji} (t >= j)
//     (only pairs t >= j: every exponent is <= 0, no division by decay);
//   A = (I + G diag(beta))^{-1} by forward substitution (16 x 16);
//   Y = V - Kbar S, E = diag(beta) A Y, O = Qbar S + L E.
// One workgroup per (batch, value head, BV value columns); fp32 throughout
// (vector ALU: a 16-token chunk is too small for matrix cores to matter).
// Accepting the first n tokens of each sequence then advances its state
// with gdr_recurrent_step_ex (per-sequence token counts).
#include "common.hpp"
#include "kernels.hpp"

namespace gdr {

template <typename TIn, typename TOut, int DK, int BV>
__global__ __launch_bounds__(256) void verify_kernel(StepArgs a) {
  constexpr int TV = kVerifyMaxTokens;
  __shared__ float sS[DK][BV + 1];             // state tile S[:, c0 .. c0 + BV)
  __shared__ float sQ[TV][DK], sK[TV][DK], sLam[TV][DK];
  __shared__ float sV[TV][BV], sY[TV][BV], sE[TV][BV];
  __shared__ float sG[TV][TV + 1], sL[TV][TV + 1], sA[TV][TV + 1], sBeta[TV];
  const int tid = threadIdx.x, T = a.T;
  const int c0 = blockIdx.x * BV, hv = blockIdx.y, b = blockIdx.z;
  const int R = a.H_v / a.H_k, hk = hv / R;
  const int hb = a.beta_per_key_head ? hk : hv, Hb = a.beta_per_key_head ? a.H_k : a.H_v;
  const TIn *qp = reinterpret_cast<const TIn *>(a.q);
  const TIn *kp = reinterpret_cast<const TIn *>(a.k);
  const TIn *vp = reinterpret_cast<const TIn *>(a.v);
  const TIn *bp = reinterpret_cast<const TIn *>(a.beta);
  const TIn *lap = reinterpret_cast<const TIn *>(a.log_alpha);
  const float *state = a.state + ((size_t)b * a.H_v + hv) * DK * a.d_v;

  for (int i = tid; i < DK * BV; i += 256) {
    const int r = i / BV, c = i % BV;
    sS[r][c] = state[(size_t)r * a.d_v + c0 + c];
  }
  // drafted tokens; rows past T are zero (and take no part below)
  for (int i = tid; i < TV * DK; i += 256) {
    const int t = i / DK, ch = i % DK;
    const bool ok = t < T;
    const size_t bt = (size_t)b * T + (ok ? t : 0);
    sQ[t][ch] = ok ? ldf(qp + (bt * a.H_k + hk) * DK + ch) : 0.f;
    sK[t][ch] = ok ? ldf(kp + (bt * a.H_k + hk) * DK + ch) : 0.f;
    sLam[t][ch] = ok ? ldf(lap + (bt * a.H_k + hk) * a.G + (ch >> a.gshift)) : 0.f;
  }
  for (int i = tid; i < TV * BV; i += 256) {
    const int t = i / BV, c = i % BV;
    sV[t][c] = t < T ? ldf(vp + ((size_t)b * T + t) * a.H_v * a.d_v + (size_t)hv * a.d_v + c0 + c) : 0.f;
  }
  if (tid < TV) sBeta[tid] = tid < T ? ldf(bp + ((size_t)b * T + tid) * Hb + hb) : 0.f;
  __syncthreads();
  if (tid < DK) {                              // Lambda: prefix over the drafted tokens, per channel
    float acc = 0.f;
    for (int t = 0; t < TV; ++t) {
      acc += sLam[t][tid];
      sLam[t][tid] = acc;
    }
  }
  __syncthreads();
  {                                            // G and L, one pair (t, j) per thread
    const int t = tid / TV, j = tid % TV;
    float g = 0.f, l = 0.f;
    if (j <= t && t < T) {
      for (int ch = 0; ch < DK; ++ch) {
        const float d = __expf(sLam[t][ch] - sLam[j][ch]);   // t >= j: exponent <= 0
        const float kj = sK[j][ch] * d;
        g += sK[t][ch] * kj;
        l += sQ[t][ch] * kj;
      }
    }
    sG[t][j] = j < t ? g : 0.f;
    sL[t][j] = l;
  }
  __syncthreads();
  if (tid < TV) {                              // column tid of A = (I + G diag(beta))^{-1}
    const int c = tid;
    float x[TV];
#pragma unroll
    for (int i = 0; i < TV; ++i) {
      float s = (i == c) ? 1.f : 0.f;
#pragma unroll
      for (int m = 0; m < i; ++m) s -= sG[i][m] * sBeta[m] * x[m];
      x[i] = (i < c) ? 0.f : s;
      sA[i][c] = x[i];
    }
  }
  // decayed operands in place: Qbar = Q e^Lambda, Kbar = K e^Lambda
  __syncthreads();
  for (int i = tid; i < TV * DK; i += 256) {
    const int t = i / DK, ch = i % DK;
    const float d = __expf(sLam[t][ch]);
    sQ[t][ch] *= d;
    sK[t][ch] *= d;
  }
  __syncthreads();
  for (int i = tid; i < TV * BV; i += 256) {   // Y = V - Kbar S
    const int t = i / BV, c = i % BV;
    float y = sV[t][c];
    for (int ch = 0; ch < DK; ++ch) y -= sK[t][ch] * sS[ch][c];
    sY[t][c] = y;
  }
  __syncthreads();
  for (int i = tid; i < TV * BV; i += 256) {   // E = diag(beta) A Y
    const int t = i / BV, c = i % BV;
    float e = 0.f;
    for (int j = 0; j <= t; ++j) e += sA[t][j] * sY[j][c];
    sE[t][c] = sBeta[t] * e;
  }
  __syncthreads();
  TOut *op = reinterpret_cast<TOut *>(a.o);
  for (int i = tid; i < TV * BV; i += 256) {   // O = Qbar S + L E
    const int t = i / BV, c = i % BV;
    if (t >= T) continue;
    float o = 0.f;
    for (int ch = 0; ch < DK; ++ch) o += sQ[t][ch] * sS[ch][c];
    for (int j = 0; j <= t; ++j) o += sL[t][j] * sE[j][c];
    st(op + ((size_t)b * T + t) * a.H_v * a.d_v + (size_t)hv * a.d_v + c0 + c, o);
  }
}

template <typename TIn, typename TOut, int BV>
static hipError_t launch_verify_bv(const StepArgs &a, hipStream_t s) {
  const dim3 grid(a.d_v / BV, a.H_v, a.B);
  switch (a.d_k) {
    case 64: hipLaunchKernelGGL((verify_kernel<TIn, TOut, 64, BV>), grid, dim3(256), 0, s, a); break;
    case 128: hipLaunchKernelGGL((verify_kernel<TIn, TOut, 128, BV>), grid, dim3(256), 0, s, a); break;
    case 256: hipLaunchKernelGGL((verify_kernel<TIn, TOut, 256, BV>), grid, dim3(256), 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <typename TIn, typename TOut>
static hipError_t launch_verify_t(const StepArgs &a, hipStream_t s) {
  return a.d_v % 32 == 0 ? launch_verify_bv<TIn, TOut, 32>(a, s) : launch_verify_bv<TIn, TOut, 16>(a, s);
}

hipError_t launch_verify(const StepArgs &a, bool in_bf16, bool out_bf16, hipStream_t stream) {
  if (in_bf16) {
    if (out_bf16) return launch_verify_t<bf16, bf16>(a, stream);
    return launch_verify_t<bf16, float>(a, stream);
  }
  if (out_bf16) return launch_verify_t<float, bf16>(a, stream);
  return launch_verify_t<float, float>(a, stream);
}

}  // namespace gdr
