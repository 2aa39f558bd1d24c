// Speculative verification (Systolic Linear Attention, section 3.2): the
// outputs of T <= 16 drafted tokens, read from a state that the call does
// not change, with the same block inversion as the chunk path -- the drafted
// tokens form one chunk of the WY form (Table 2):
//   Lambda = prefix sum of log alpha over the drafted tokens;
//   G_tj = sum_i k_ti k_ji e^{Lambda_ti - Lambda_ji} (t > j),
//   L_tj = sum_i q_ti k_ji e^{Lambda_ti - Lambda_ji} (t >= j),
//     formed as 16 x 16 products Kbar C^T, Qbar C^T with Kbar = K e^Lambda,
//     Qbar = Q e^Lambda, C = K e^{-Lambda} while every |Lambda| over the
//     drafted tokens is within a bound; otherwise pair by pair with exponent
//     Lambda_t - Lambda_j <= 0 (no division by decay);
//   A = (I + G diag(beta))^{-1} by forward substitution (16 x 16);
//   Y = V - Kbar S, E = diag(beta) A Y, O = Qbar S + L E.
// Loads are unconditional (rows past T read the last drafted row and are
// zeroed after): a load behind a branch waits for every load in flight.
// One workgroup of 8 waves per (batch, value head, up to 128 value
// columns), one wave per 16 columns; fp32 throughout.  Each wave loads its 16 columns of the
// state into registers first (in the MFMA operand layout), so the state read
// overlaps the 16 x 16 work; the products with the state, E and L E are fp32
// MFMA tiles, E and O taken straight from the accumulators.
// Accepting the first n tokens of each sequence then advances its state
// with gdr_recurrent_step_ex (per-sequence token counts).
#include "common.hpp"
#include "kernels.hpp"

namespace gdr {

// Bound on |Lambda| over the drafted tokens for the products with
// e^{+-Lambda} (e^64 ~ 6e27 keeps every factor and partial sum finite and
// normal); beyond it the pairs are formed one by one.
constexpr float kVerifyLambdaBound = 64.f;
constexpr int kVerifyWaves = 8;              // 16-column tiles per workgroup

// Waves per SIMD the register budget is set for: three workgroups per
// compute unit for 16-bit inputs with d_k <= 128 (a few bytes of spill),
// else what the code needs.
template <typename TIn, int DK>
constexpr int verify_waves_per_simd() { return sizeof(TIn) == 2 && DK <= 128 ? 6 : 1; }

template <typename TIn, typename TOut, int DK>
__global__ __launch_bounds__(64 * kVerifyWaves, (verify_waves_per_simd<TIn, DK>())) void verify_kernel(StepArgs a) {
  constexpr int TV = kVerifyMaxTokens;
  constexpr int QP = DK + 4;                   // row pitch: MFMA operand reads hit distinct banks
  __shared__ float sK[TV][QP], sQ[TV][QP];     // Kbar, Qbar
  __shared__ float sC[TV][QP], sLam[TV][QP];   // K e^{-Lambda}, log alpha
  __shared__ float sG[TV][TV + 1], sL[TV][TV + 1], sA[TV][TV + 1], sBeta[TV];
  __shared__ int sWide[kVerifyWaves];         // per wave: some channel beyond the bound
  const int tid = threadIdx.x, T = a.T, w = wave_id(), l = lane_id();
  const int i16 = l & 15, kk = l >> 4;
  const int hv = blockIdx.y, b = blockIdx.z;
  const int R = a.H_v / a.H_k, hk = hv / R;
  const int hb = a.beta_per_key_head ? hk : hv, Hb = a.beta_per_key_head ? a.H_k : a.H_v;
  const TIn *qp = reinterpret_cast<const TIn *>(a.q);
  const TIn *kp = reinterpret_cast<const TIn *>(a.k);
  const TIn *vp = reinterpret_cast<const TIn *>(a.v);
  const TIn *bp = reinterpret_cast<const TIn *>(a.beta);
  const TIn *lap = reinterpret_cast<const TIn *>(a.log_alpha);
  const int col = 16 * (blockIdx.x * kVerifyWaves + w) + i16;   // this lane's value column
  const bool tile = col - i16 < a.d_v;                          // uniform per wave (d_v % 16 == 0)
  const size_t qk_row = (size_t)a.H_k * DK;                     // q, k elements per token
  const int nth = 64 * kVerifyWaves;

  // ---- the drafted q, k, log alpha as (token, 8 channels) items, at most
  // one per thread, and beta into LDS.  Rows past T read the last drafted row
  // (a valid address; loads stay unconditional) and are zeroed.
  constexpr int NI = TV * DK / 8;
  static_assert(NI <= 64 * kVerifyWaves, "one (token, 8 channels) item per thread");
  const int item = min(tid, NI - 1);
  const int t_in = item / (DK / 8), ch_in = 8 * (item % (DK / 8));
  const size_t row = ((size_t)b * T + min(t_in, T - 1)) * a.H_k + hk;
  float xq[8], xk[8], xl[8];
  ld8(qp + row * DK + ch_in, xq);
  ld8(kp + row * DK + ch_in, xk);
#pragma unroll
  for (int e = 0; e < 8; ++e) xl[e] = ldf(lap + row * a.G + ((ch_in + e) >> a.gshift));
  const float xb = ldf(bp + ((size_t)b * T + min(tid & (TV - 1), T - 1)) * Hb + hb);
  if (tid < TV) sBeta[tid] = tid < T ? xb : 0.f;
  if (tid < NI) {
    const bool ok = t_in < T;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      sQ[t_in][ch_in + e] = ok ? xq[e] : 0.f;
      sK[t_in][ch_in + e] = ok ? xk[e] : 0.f;
      sLam[t_in][ch_in + e] = ok ? xl[e] : 0.f;
    }
  }
  __syncthreads();
  // ---- this wave's state columns and V tile in the MFMA operand layouts,
  // s[u] = S[4u + kk][col], vt[r] = V[4 kk + r][col]: issued here and first
  // waited for in the products with the state, so the state read overlaps
  // the 16 x 16 work below (columns past d_v read a valid clamped column and
  // are not stored)
  const int colc = min(col, a.d_v - 1);
  const float *sp = a.state + ((size_t)b * a.H_v + hv) * DK * a.d_v + colc;
  float s[DK / 4], vt[4];
#pragma unroll
  for (int u = 0; u < DK / 4; ++u) s[u] = sp[(size_t)(4 * u + kk) * a.d_v];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int t = 4 * kk + r;
    const float x = ldf(vp + (((size_t)b * T + min(t, T - 1)) * a.H_v + hv) * a.d_v + colc);
    vt[r] = t < T ? x : 0.f;
  }
  // ---- Lambda and the operands Kbar, Qbar, C in place: TPC threads per key
  // channel, each for TT consecutive tokens; the prefix before its first
  // token is summed again in token order (the same sums as one running
  // prefix), so no thread waits for another.  sLam keeps log alpha.
  constexpr int TPC = 64 * kVerifyWaves / DK;  // 8, 4 or 2
  constexpr int TT = TV / TPC;
  bool beyond;
  {
    const int ch = tid % DK, t0 = (tid / DK) * TT;
    float pre[TV], la[TT], kv[TT], qv[TT];
#pragma unroll
    for (int t = 0; t < TV; ++t) pre[t] = sLam[t][ch];
#pragma unroll
    for (int j = 0; j < TT; ++j) {
      la[j] = sLam[t0 + j][ch];
      kv[j] = sK[t0 + j][ch];
      qv[j] = sQ[t0 + j][ch];
    }
    float acc = 0.f, big = 0.f;
#pragma unroll
    for (int t = 0; t < TV; ++t) acc += t < t0 ? pre[t] : 0.f;
#pragma unroll
    for (int j = 0; j < TT; ++j) {
      acc += la[j];
      const float up = __expf(acc), dn = __expf(-acc);
      sK[t0 + j][ch] = kv[j] * up;
      sQ[t0 + j][ch] = qv[j] * up;
      sC[t0 + j][ch] = kv[j] * dn;
      big = fmaxf(big, fabsf(acc));
    }
    beyond = !(big <= kVerifyLambdaBound);     // NaN too
  }
  const bool wave_beyond = __ballot(beyond) != 0;
  if (l == 0) sWide[w] = wave_beyond;
  __syncthreads();
  bool wide = false;
  for (int i = 0; i < kVerifyWaves; ++i) wide |= sWide[i] != 0;
  // Y = V - Kbar S and Qbar S (rows 4 kk + r, column col in the accumulators);
  // they need neither G, L nor A, so waves 2..7 form them while waves 0, 1
  // form G and L, and waves 0, 1 while wave 2 solves for A
  f32x4 y = {0.f, 0.f, 0.f, 0.f}, o = {0.f, 0.f, 0.f, 0.f};
  auto state_products = [&]() {
#pragma unroll
    for (int u = 0; u < DK / 4; ++u) {
      y = mfma_f32(sK[i16][4 * u + kk], s[u], y);
      o = mfma_f32(sQ[i16][4 * u + kk], s[u], o);
    }
  };
  if (!wide) {                                 // G diag(beta) = Kbar C^T diag(beta) (wave 0), L = Qbar C^T (wave 1)
    if (w < 2) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int k0 = 0; k0 < DK; k0 += 64)
        tile_f32_n<4>(acc, [&](int i, int k) { return w == 0 ? sK[i][k] : sQ[i][k]; },
                      [&](int k, int j) { return sC[j][k]; }, k0);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = 4 * kk + r;
        if (w == 0) {
          sG[t][i16] = i16 < t ? acc[r] * sBeta[i16] : 0.f;
        } else {
          sL[t][i16] = i16 <= t ? acc[r] : 0.f;
        }
      }
    }
  } else {
    // Lambda per channel into sC (not used in this mode), then one pair
    // (t, j) per thread from the raw q, k (read again; they are in cache)
    for (int ch = tid; ch < DK; ch += nth) {
      float acc = 0.f;
      for (int t = 0; t < TV; ++t) {
        acc += sLam[t][ch];
        sC[t][ch] = acc;
      }
    }
    __syncthreads();
    for (int p = tid; p < TV * TV; p += nth) {
      const int t = p / TV, j = p % TV;
      float g = 0.f, lv = 0.f;
      if (j <= t && t < T) {
        const size_t rt = ((size_t)b * T + t) * qk_row + (size_t)hk * DK;
        const size_t rj = ((size_t)b * T + j) * qk_row + (size_t)hk * DK;
        for (int ch = 0; ch < DK; ++ch) {
          const float kj = ldf(kp + rj + ch) * __expf(sC[t][ch] - sC[j][ch]);   // exponent <= 0
          g += ldf(kp + rt + ch) * kj;
          lv += ldf(qp + rt + ch) * kj;
        }
      }
      sG[t][j] = j < t ? g * sBeta[j] : 0.f;
      sL[t][j] = lv;
    }
  }
  if (w >= 2 && tile) state_products();
  __syncthreads();
  if (w == 2) {
    if (l < TV) {                              // column l of diag(beta) A, A = (I + G diag(beta))^{-1}
      const int c = l;
      float x[TV];
#pragma unroll
      for (int i = 0; i < TV; ++i) {
        float v = (i == c) ? 1.f : 0.f;
#pragma unroll
        for (int m = 0; m < i; ++m) v -= sG[i][m] * x[m];
        x[i] = (i < c) ? 0.f : v;
        sA[i][c] = sBeta[i] * x[i];
      }
    }
  } else if (w < 2 && tile) {
    state_products();
  }
  __syncthreads();
  if (!tile) return;
#pragma unroll
  for (int r = 0; r < 4; ++r) y[r] = vt[r] - y[r];
  // E = diag(beta) A Y, O += L E: the contraction index runs as 4 kk + u, the
  // order in which each lane holds the rows of Y (and then E)
  f32x4 e = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int u = 0; u < 4; ++u) e = mfma_f32(sA[i16][4 * kk + u], y[u], e);
#pragma unroll
  for (int u = 0; u < 4; ++u) o = mfma_f32(sL[i16][4 * kk + u], e[u], o);
  TOut *op = reinterpret_cast<TOut *>(a.o);
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int t = 4 * kk + r;
    if (t < T) st(op + (((size_t)b * T + t) * a.H_v + hv) * a.d_v + col, o[r]);
  }
}

template <typename TIn, typename TOut>
static hipError_t launch_verify_t(const StepArgs &a, hipStream_t s) {
  const int tiles = a.d_v / 16;
  const dim3 grid((tiles + kVerifyWaves - 1) / kVerifyWaves, a.H_v, a.B);
  const dim3 block(64 * kVerifyWaves);
  switch (a.d_k) {
    case 64: hipLaunchKernelGGL((verify_kernel<TIn, TOut, 64>), grid, block, 0, s, a); break;
    case 128: hipLaunchKernelGGL((verify_kernel<TIn, TOut, 128>), grid, block, 0, s, a); break;
    case 256: hipLaunchKernelGGL((verify_kernel<TIn, TOut, 256>), grid, block, 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
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
