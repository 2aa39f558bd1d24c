// Chunk preparation: per (batch, key head, chunk) build the beta-free Gram
// G_c (strictly lower) and the score matrix L_c (lower, diagonal included)
// with division-free relative decay, then for every beta head solve
// A_c = (I + G_c diag(beta))^{-1} and store A_c and L_c as fp32 C x C.
//
// Systolic Linear Attention (paperpeel 2611.06828):
//  - cumulative log-decay Lambda and the chunk matrices: Table 2;
//  - the Gram entries M_{t,j} = 1[t>j] beta_j sum_i exp(Lambda_{t,i} -
//    Lambda_{j,i}) k_{t,i} k_{j,i}: section 2.2, "Bottleneck 2";
//  - exp(+-Lambda) leaves fp32 once |Lambda| > 88.7: section 2.4.2;
//  - the exact inverse by recursive block doubling: section 2.4.3.
// Muir (ai.info 2611.08376), "Key Contributions" item 4: relative decays are
// split at chunk-internal boundaries instead of dividing by cumulative decay.
// Multiplication-only inversion paper (pith.science JIMYX2Z6): truncated
// Neumann series with residual correction.
//
// Division-free decay with block pivots.  The chunk is cut into 16-token
// blocks.  For a block pair (I, J), I >= J, every t in I and j in J satisfy
// j <= p <= t for the pivot p = first token of I, so
//   exp(Lambda_t - Lambda_j) = exp(Lambda_t - Lambda_p) * exp(Lambda_p - Lambda_j)
// and for I > J both factors are <= 1: the pair is one MFMA product of the
// row-scaled keys (or queries) of I with the row-scaled keys of J.  On a
// diagonal block (I == J) the second factor is >= 1 and at most
// exp(range of Lambda over the block); if that range exceeds kPivotRange in
// any channel the block is evaluated element by element with the causal mask
// applied before the exponential.  No exponential of a positive Lambda
// difference on the causal side is ever formed.
#include "common.hpp"
#include "kernels.hpp"

namespace gdr {

constexpr float kPivotRange = 64.f;  // exp(64) ~ 6e27 keeps every partial sum finite

__host__ __device__ inline int prep_region0_floats(int C, int G) {
  return (C * G > C * C) ? C * G : C * C;
}
__host__ __device__ inline int prep_tmp_floats(int C) {
  return (C * C / 4 > C * 16) ? C * C / 4 : C * 16;
}

size_t prep_lds_bytes(int C, int G) {
  const int nb = C / 16;
  return sizeof(float) * (size_t)(prep_region0_floats(C, G) + C * C + prep_tmp_floats(C) + C) +
         sizeof(int) * (size_t)nb;
}

// --------------------------------------------------------------- fp32 tiles
// acc += X[r0 + i, k] * Y[k, c0 + j] over k in [k0, k1) (multiple of 4), with
// element accessors.  fp32 MFMA: lane l supplies X[i = l%16][k + l/16] and
// Y[k + l/16][j = l%16].
template <class FX, class FY>
__device__ __forceinline__ void tile_f32(f32x4 &acc, const FX &x, const FY &y, int k0, int k1) {
  const int l = lane_id();
  const int i = l & 15, kk = l >> 4;
  for (int k = k0; k < k1; k += 4) acc = mfma_f32(x(i, k + kk), y(k + kk, i), acc);
}

// ------------------------------------------------------------- exact solve
// amat <- (I + M)^{-1}, M = gmat diag(bet): 16x16 diagonal blocks by forward
// substitution (one lane per column), then block-doubling merges
// A[B,T] = -A[B,B] (M[B,T] A[T,T]) with fp32 MFMA.
template <int C>
__device__ void solve_exact(const float *gmat, const float *bet, float *amat, float *tmp) {
  constexpr int NB = C / 16;
  const int tid = threadIdx.x, w = wave_id(), l = lane_id();
  for (int i = tid; i < C * C; i += blockDim.x) amat[i] = 0.f;
  __syncthreads();
  if (tid < NB * 16) {
    const int base = 16 * (tid >> 4), cc = tid & 15;
    float x[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float s = (i == cc) ? 1.f : 0.f;
#pragma unroll
      for (int m = 0; m < i; ++m) s -= gmat[(base + i) * C + base + m] * bet[base + m] * x[m];
      x[i] = s;
      amat[(base + i) * C + base + cc] = s;
    }
  }
  __syncthreads();
  for (int bs = 16; bs < C; bs *= 2) {
    const int tpb = bs / 16;                  // tiles per block side
    const int jobs = (C / (2 * bs)) * tpb * tpb;
    // X_p = M[bot, top] * A[top, top] -> tmp (pair p at tmp + p * bs * bs)
    for (int job = w; job < jobs; job += blockDim.x / kWave) {
      const int p = job / (tpb * tpb), ti = (job / tpb) % tpb, tj = job % tpb;
      const int top = 2 * bs * p, bot = top + bs;
      const int r0 = bot + 16 * ti, c0 = top + 16 * tj;
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      tile_f32(acc,
               [&](int i, int k) { return gmat[(r0 + i) * C + k] * bet[k]; },
               [&](int k, int j) { return amat[k * C + c0 + j]; },
               c0, top + bs);                 // A[top,top] is lower: rows k >= column
      float *X = tmp + p * bs * bs;
#pragma unroll
      for (int r = 0; r < 4; ++r) X[(16 * ti + 4 * (l >> 4) + r) * bs + 16 * tj + (l & 15)] = acc[r];
    }
    __syncthreads();
    // A[bot, top] = -A[bot, bot] * X_p
    for (int job = w; job < jobs; job += blockDim.x / kWave) {
      const int p = job / (tpb * tpb), ti = (job / tpb) % tpb, tj = job % tpb;
      const int top = 2 * bs * p, bot = top + bs;
      const int r0 = bot + 16 * ti;
      const float *X = tmp + p * bs * bs;
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      tile_f32(acc,
               [&](int i, int k) { return amat[(r0 + i) * C + k]; },
               [&](int k, int j) { return X[(k - bot) * bs + 16 * tj + j]; },
               bot, r0 + 16);                 // A[bot,bot] is lower: columns k <= row
#pragma unroll
      for (int r = 0; r < 4; ++r)
        amat[(r0 + 4 * (l >> 4) + r) * C + top + 16 * tj + (l & 15)] = -acc[r];
    }
    __syncthreads();
  }
}

// ----------------------------------------------------------- Neumann solve
// X = sum_{s=0}^{m} (-M)^s by Horner (X <- I - M X, m times), then r residual
// corrections X <- X + X (I - (I + M) X).  Both products are evaluated one
// 16-column block of the result at a time, so X is updated in place: a column
// block of M X needs only the same column block of X, and X Rm[:, J] needs the
// columns of X at and right of J, which are still the old ones.
template <int C>
__device__ void solve_neumann(const float *gmat, const float *bet, float *amat, float *tmp, int order,
                              int residual) {
  constexpr int NB = C / 16;
  constexpr int kMaxTiles = (NB + 3) / 4;
  const int tid = threadIdx.x, w = wave_id(), l = lane_id();
  const int nw = blockDim.x / kWave;
  for (int i = tid; i < C * C; i += blockDim.x) amat[i] = ((i / C) == (i % C)) ? 1.f : 0.f;
  __syncthreads();
  auto Mx = [&](int i, int k, int r0) { return gmat[(r0 + i) * C + k] * bet[k]; };
  for (int it = 0; it < order; ++it) {
    for (int J = 0; J < NB; ++J) {
      f32x4 acc[kMaxTiles];
      int nt = 0;
      for (int I = J + w; I < NB; I += nw, ++nt) {
        acc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
        const int r0 = 16 * I;
        tile_f32(acc[nt], [&](int i, int k) { return Mx(i, k, r0); },
                 [&](int k, int j) { return amat[k * C + 16 * J + j]; }, 16 * J, r0 + 16);
      }
      __syncthreads();
      nt = 0;
      for (int I = J + w; I < NB; I += nw, ++nt) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = 16 * I + 4 * (l >> 4) + r, col = 16 * J + (l & 15);
          amat[row * C + col] = ((row == col) ? 1.f : 0.f) - acc[nt][r];
        }
      }
      __syncthreads();
    }
  }
  for (int it = 0; it < residual; ++it) {
    for (int J = 0; J < NB; ++J) {
      // Rm[:, J] = I - X[:, J] - (M X)[:, J] -> tmp[row * 16 + col - 16J]
      for (int I = J + w; I < NB; I += nw) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        const int r0 = 16 * I;
        tile_f32(acc, [&](int i, int k) { return Mx(i, k, r0); },
                 [&](int k, int j) { return amat[k * C + 16 * J + j]; }, 16 * J, r0 + 16);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = 16 * I + 4 * (l >> 4) + r, col = 16 * J + (l & 15);
          tmp[row * 16 + (l & 15)] = ((row == col) ? 1.f : 0.f) - amat[row * C + col] - acc[r];
        }
      }
      __syncthreads();
      f32x4 acc[kMaxTiles];
      int nt = 0;
      for (int I = J + w; I < NB; I += nw, ++nt) {
        acc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
        const int r0 = 16 * I;
        tile_f32(acc[nt], [&](int i, int k) { return amat[(r0 + i) * C + k]; },
                 [&](int k, int j) { return tmp[k * 16 + j]; }, 16 * J, r0 + 16);
      }
      __syncthreads();
      nt = 0;
      for (int I = J + w; I < NB; I += nw, ++nt) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = 16 * I + 4 * (l >> 4) + r, col = 16 * J + (l & 15);
          amat[row * C + col] += acc[nt][r];
        }
      }
      __syncthreads();
    }
  }
}

// ------------------------------------------------------------------ kernel
template <typename TIn, class P, int C, int DK>
__global__ __launch_bounds__(256) void prep_kernel(ChunkArgs a) {
  constexpr int NB = C / 16;
  using Split = typename P::Split;
  extern __shared__ __align__(16) unsigned char smem_raw[];
  float *smem = reinterpret_cast<float *>(smem_raw);
  const int c = blockIdx.x, hk = blockIdx.y, b = blockIdx.z;
  const int G = a.G, gs = a.gshift, T = a.T;
  const int t0 = c * C;
  const int tid = threadIdx.x, w = wave_id(), l = lane_id();

  float *lam = smem;                                   // [C][G] (Gram phase)
  float *amat = smem;                                  // [C][C] (solve phase, aliases lam)
  float *gmat = smem + prep_region0_floats(C, G);      // [C][C]
  float *tmp = gmat + C * C;
  float *bet = tmp + prep_tmp_floats(C);               // [C]
  int *flags = reinterpret_cast<int *>(bet + C);       // [NB]

  const TIn *la = reinterpret_cast<const TIn *>(a.log_alpha);
  const TIn *qp = reinterpret_cast<const TIn *>(a.q);
  const TIn *kp = reinterpret_cast<const TIn *>(a.k);

  // Lambda: in-chunk prefix sums of log alpha per decay group (padding: 0).
  for (int g = tid; g < G; g += blockDim.x)
    lambda_column<C>(la + ((size_t)(b * T + t0) * a.H_k + hk) * G + g, (size_t)a.H_k * G, T - t0, lam + g, G);
  if (tid < NB) flags[tid] = 0;
  for (int i = tid; i < C * C; i += blockDim.x) gmat[i] = 0.f;
  __syncthreads();
  for (int idx = tid; idx < NB * G; idx += blockDim.x) {
    const int I = idx / G, g = idx - I * G;
    float lo = lam[(16 * I) * G + g], hi = lo;
    for (int r = 1; r < 16; ++r) {
      const float x = lam[(16 * I + r) * G + g];
      lo = fminf(lo, x);
      hi = fmaxf(hi, x);
    }
    if (!(hi - lo <= kPivotRange)) atomicOr(&flags[I], 1);
  }
  __syncthreads();

  // Gram G_c (beta-free, strictly lower) and L_c (lower incl. diagonal).
  float *Lout = a.L_ws + (((size_t)b * a.H_k + hk) * a.N_c + c) * (size_t)(C * C);
  const size_t row_stride = (size_t)a.H_k * DK;
  const TIn *kbase = kp + ((size_t)(b * T + t0) * a.H_k + hk) * DK;
  const TIn *qbase = qp + ((size_t)(b * T + t0) * a.H_k + hk) * DK;
  for (int pi = w; pi < NB * (NB + 1) / 2; pi += blockDim.x / kWave) {
    int I = 0;
    while ((I + 1) * (I + 2) / 2 <= pi) ++I;
    const int J = pi - I * (I + 1) / 2;
    f32x4 accG = {0.f, 0.f, 0.f, 0.f}, accL = {0.f, 0.f, 0.f, 0.f};
    if (!(I == J && flags[I])) {
      const int tr = 16 * I + (l & 15), jr = 16 * J + (l & 15), piv = 16 * I;
      const bool vt = t0 + tr < T, vj = t0 + jr < T;
      for (int s = 0; s < DK / 32; ++s) {
        const int ch0 = 32 * s + 8 * (l >> 4);
        float kt[8], qt[8], kj[8];
        if (vt) {
          ld8(kbase + tr * row_stride + ch0, kt);
          ld8(qbase + tr * row_stride + ch0, qt);
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) kt[e] = qt[e] = 0.f;
        }
        if (vj) {
          ld8(kbase + jr * row_stride + ch0, kj);
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) kj[e] = 0.f;
        }
        float xk[8], xq[8], xj[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int g = (ch0 + e) >> gs;
          const float lp = lam[piv * G + g];
          const float ea = __expf(lam[tr * G + g] - lp);
          const float eb = __expf(lp - lam[jr * G + g]);
          xk[e] = kt[e] * ea;
          xq[e] = qt[e] * ea;
          xj[e] = kj[e] * eb;
        }
        const Split fk = make_frag<Split>(xk), fq = make_frag<Split>(xq), fj = make_frag<Split>(xj);
        mma(accG, fk, fj);
        mma(accL, fq, fj);
      }
    } else {
      // Diagonal block whose decay range is too wide for one pivot: each
      // entry by its definition, causal mask before the exponential.
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = 16 * I + 4 * (l >> 4) + r, col = 16 * J + (l & 15);
        float sg = 0.f, sl = 0.f;
        if (row >= col && t0 + row < T) {
          for (int ch = 0; ch < DK; ++ch) {
            const int g = ch >> gs;
            const float d = __expf(lam[row * G + g] - lam[col * G + g]);
            const float kc = ldf(kbase + col * row_stride + ch);
            sg += ldf(kbase + row * row_stride + ch) * kc * d;
            sl += ldf(qbase + row * row_stride + ch) * kc * d;
          }
        }
        accG[r] = sg;
        accL[r] = sl;
      }
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = 16 * I + 4 * (l >> 4) + r, col = 16 * J + (l & 15);
      gmat[row * C + col] = (I > J || row > col) ? accG[r] : 0.f;
      Lout[row * C + col] = (I > J || row >= col) ? accL[r] : 0.f;
    }
  }
  for (int i = tid; i < C * C; i += blockDim.x) {
    if ((i / C) / 16 < (i % C) / 16) Lout[i] = 0.f;   // blocks above the diagonal
  }

  // Solve per beta head.
  const int Rb = a.H_beta / a.H_k;
  for (int rb = 0; rb < Rb; ++rb) {
    const int hb = hk * Rb + rb;
    __syncthreads();
    for (int t = tid; t < C; t += blockDim.x) {
      bet[t] = (t0 + t < T) ? ldf(reinterpret_cast<const TIn *>(a.beta) + (size_t)(b * T + t0 + t) * a.H_beta + hb)
                            : 0.f;
    }
    __syncthreads();
    if (a.solve == 0) {
      solve_exact<C>(gmat, bet, amat, tmp);
    } else {
      solve_neumann<C>(gmat, bet, amat, tmp, a.order, a.residual);
    }
    __syncthreads();
    float *Aout = a.A_ws + (((size_t)b * a.H_beta + hb) * a.N_c + c) * (size_t)(C * C);
    for (int i = 4 * tid; i < C * C; i += 4 * blockDim.x) {
      *reinterpret_cast<float4 *>(Aout + i) = *reinterpret_cast<const float4 *>(amat + i);
    }
  }
}

bool prep_supported(int C, int d_k, int G) {
  if (!(C == 64 || C == 128)) return false;
  if (!(d_k == 64 || d_k == 128 || d_k == 256)) return false;
  return prep_lds_bytes(C, G) <= 160 * 1024;
}

template <typename TIn, class P, int C, int DK>
static hipError_t launch_prep_t(const ChunkArgs &a, hipStream_t stream) {
  const size_t lds = prep_lds_bytes(C, a.G);
  auto kern = prep_kernel<TIn, P, C, DK>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  dim3 grid(a.N_c, a.H_k, a.B);
  hipLaunchKernelGGL(kern, grid, dim3(256), lds, stream, a);
  return hipGetLastError();
}

template <typename TIn, class P>
static hipError_t launch_prep_dk(const ChunkArgs &a, hipStream_t s) {
  switch (a.C * 1000 + a.d_k) {
    case 64064: return launch_prep_t<TIn, P, 64, 64>(a, s);
    case 64128: return launch_prep_t<TIn, P, 64, 128>(a, s);
    case 64256: return launch_prep_t<TIn, P, 64, 256>(a, s);
    case 128064: return launch_prep_t<TIn, P, 128, 64>(a, s);
    case 128128: return launch_prep_t<TIn, P, 128, 128>(a, s);
    case 128256: return launch_prep_t<TIn, P, 128, 256>(a, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_prep(const ChunkArgs &a, bool in_bf16, hipStream_t stream) {
  if (in_bf16) return launch_prep_dk<bf16, PrecBF16>(a, stream);
  return launch_prep_dk<float, PrecF32>(a, stream);
}

}  // namespace gdr
