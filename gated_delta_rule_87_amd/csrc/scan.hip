// State scan + output: per (batch, value head, tile of BV value columns) walk
// the chunks in order, carrying the d_k x BV slice of the state S in the MFMA
// accumulators of the four waves.  Per chunk c (Systolic Linear Attention,
// Table 2, section 2.3 and the WY equivalence proof of section 2.4.2):
//
//   Y   = V_c - Kbar_c S_{c-1}                 (C x BV)
//   E_c = diag(beta) A_c Y  = U_c - W_c S_{c-1} (the chunk writes)
//   O_c = Qbar_c S_{c-1} + L_c E_c              (readout; L_c includes t = j)
//   S_c = F_c S_{c-1} + Khat_c^T E_c            (Delta S_c = Khat_c^T E_c)
//
// with Qbar = Q (.) exp(Lambda_t), Kbar = K (.) exp(Lambda_t),
// Khat = K (.) exp(Lambda_C - Lambda_t), F_c = diag(exp(Lambda_C)): every
// exponent is a non-positive Lambda difference, so nothing overflows however
// strong the decay (no division by a cumulative decay).
//
// Value columns never mix in the recurrence (each column of S evolves on its
// own), so tiling d_v across workgroups is exact.  A_c and L_c come from the
// prep kernel's workspace.
//
// Operand precision (bf16 policy): Kbar and A_c as plain bf16; S, Y, Qbar,
// L_c, E and Khat split into bf16 hi + lo.  Rounding any one of the latter to
// plain bf16 alone breaks a 1e-2 max-error bar on the per-channel-gate
// workload; Kbar or A_c alone costs about 1e-3.
#include "common.hpp"
#include "kernels.hpp"

namespace gdr {

template <int C, int DK, int BV, typename TIn>
struct ScanLds {
  static size_t bytes(int G) {
    return sizeof(float) * (size_t)C * G          // lam
           + sizeof(TIn) * (size_t)C * DK         // staged k chunk
           + 4 * (size_t)BV * DK                  // S^T operand
           + 2 * 4 * (size_t)BV * C               // Y^T, E^T operands
           + sizeof(float) * (size_t)C;           // beta
  }
};

template <typename TIn, typename TOut, class P, int C, int DK, int BV>
__global__ __launch_bounds__(256) void scan_kernel(ChunkArgs a) {
  constexpr int RB = C / 64;     // 16-row token blocks per wave
  constexpr int CB = DK / 64;    // 16-row channel blocks of S per wave
  constexpr int NT = BV / 16;    // 16-column tiles
  using Plain = typename P::Plain;
  using Split = typename P::Split;

  extern __shared__ __align__(16) unsigned char smem_raw[];
  const int G = a.G, gs = a.gshift, T = a.T;
  const int c0 = blockIdx.x * BV, hv = blockIdx.y, b = blockIdx.z;
  const int R = a.H_v / a.H_k;
  const int hk = hv / R;
  const int hb = a.beta_per_key_head ? hk : hv;
  const int tid = threadIdx.x, w = wave_id(), l = lane_id();
  const int lr = l & 15, lq = l >> 4;

  float *lam = reinterpret_cast<float *>(smem_raw);
  TIn *ks = reinterpret_cast<TIn *>(lam + C * G);
  unsigned char *ops = reinterpret_cast<unsigned char *>(ks + C * DK);
  OperandLds<P> sT, yT, eT;
  sT.init(ops, BV, DK);
  yT.init(ops + 4 * BV * DK, BV, C);
  eT.init(ops + 4 * BV * DK + 4 * BV * C, BV, C);
  float *bet = reinterpret_cast<float *>(ops + 4 * BV * DK + 8 * BV * C);

  const TIn *qp = reinterpret_cast<const TIn *>(a.q);
  const TIn *kp = reinterpret_cast<const TIn *>(a.k);
  const TIn *vp = reinterpret_cast<const TIn *>(a.v);
  const TIn *bp = reinterpret_cast<const TIn *>(a.beta);
  const TIn *lap = reinterpret_cast<const TIn *>(a.log_alpha);
  TOut *op = reinterpret_cast<TOut *>(a.o);
  const size_t qk_row = (size_t)a.H_k * DK;   // token stride of q, k
  const size_t v_row = (size_t)a.H_v * a.d_v; // token stride of v, o

  // State slice: wave w owns channel blocks w*CB .. w*CB+CB-1, all NT tiles.
  f32x4 S[CB][NT];
  const size_t sbase = ((size_t)b * a.H_v + hv) * DK * a.d_v;
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) {
    const int i0 = (w * CB + cb) * 16;
#pragma unroll
    for (int n = 0; n < NT; ++n) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = i0 + 4 * lq + r, col = c0 + 16 * n + lr;
        S[cb][n][r] = a.h0 ? a.h0[sbase + (size_t)i * a.d_v + col] : 0.f;
      }
      sT.put4(16 * n + lr, i0 + 4 * lq, S[cb][n]);
    }
  }

  for (int c = 0; c < a.N_c; ++c) {
    const int t0 = c * C;
    // ---- stage: Lambda, k chunk, beta
    for (int g = tid; g < G; g += blockDim.x) {
      float acc = 0.f;
      for (int t = 0; t < C; ++t) {
        if (t0 + t < T) acc += ldf(lap + ((size_t)(b * T + t0 + t) * a.H_k + hk) * G + g);
        lam[t * G + g] = acc;
      }
    }
    for (int idx = 8 * tid; idx < C * DK; idx += 8 * blockDim.x) {
      const int t = idx / DK, ch = idx - t * DK;
      if (t0 + t < T) {
        const TIn *src = kp + (size_t)(b * T + t0 + t) * qk_row + hk * DK + ch;
        if constexpr (sizeof(TIn) == 2) {
          *reinterpret_cast<uint4 *>(ks + idx) = *reinterpret_cast<const uint4 *>(src);
        } else {
          *reinterpret_cast<float4 *>(ks + idx) = *reinterpret_cast<const float4 *>(src);
          *reinterpret_cast<float4 *>(ks + idx + 4) = *reinterpret_cast<const float4 *>(src + 4);
        }
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) ks[idx + e] = TIn(0.f);
      }
    }
    for (int t = tid; t < C; t += blockDim.x)
      bet[t] = (t0 + t < T) ? ldf(bp + (size_t)(b * T + t0 + t) * a.H_beta + hb) : 0.f;
    __syncthreads();

    // ---- Y = V - Kbar S and Qbar S for this wave's token rows
    f32x4 accO[RB][NT];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const int I = w * RB + rb;
      const int t = 16 * I + lr;
      f32x4 accY[NT];
#pragma unroll
      for (int n = 0; n < NT; ++n) {
        accY[n] = f32x4{0.f, 0.f, 0.f, 0.f};
        accO[rb][n] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
      const bool tv = t0 + t < T;
#pragma unroll
      for (int s = 0; s < DK / 32; ++s) {
        const int ch0 = 32 * s + 8 * lq;
        float kv[8], qv[8];
        ld8(ks + t * DK + ch0, kv);
        if (tv) {
          ld8(qp + (size_t)(b * T + t0 + t) * qk_row + hk * DK + ch0, qv);
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) qv[e] = 0.f;
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float d = __expf(lam[t * G + ((ch0 + e) >> gs)]);
          kv[e] *= d;
          qv[e] *= d;
        }
        const Plain fk = make_frag<Plain>(kv);
        const Split fq = make_frag<Split>(qv);
#pragma unroll
        for (int n = 0; n < NT; ++n) {
          const Split fs = sT.get(16 * n + lr, ch0);
          mma(accY[n], fk, fs);
          mma(accO[rb][n], fq, fs);
        }
      }
#pragma unroll
      for (int n = 0; n < NT; ++n) {
        f32x4 y;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = 16 * I + 4 * lq + r;
          const float vv = (t0 + row < T) ? ldf(vp + (size_t)(b * T + t0 + row) * v_row + hv * a.d_v + c0 + 16 * n + lr) : 0.f;
          y[r] = vv - accY[n][r];
        }
        yT.put4(16 * n + lr, 16 * I + 4 * lq, y);
      }
    }
    __syncthreads();

    // ---- E = diag(beta) A Y
    const float *Ac = a.A_ws + (((size_t)b * a.H_beta + hb) * a.N_c + c) * (size_t)(C * C);
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const int I = w * RB + rb;
      f32x4 accE[NT];
#pragma unroll
      for (int n = 0; n < NT; ++n) accE[n] = f32x4{0.f, 0.f, 0.f, 0.f};
      const int row = 16 * I + lr;
      for (int s = 0; s * 32 < 16 * I + 16; ++s) {
        const int j0 = 32 * s + 8 * lq;
        float av[8];
        ld8(Ac + row * C + j0, av);
        const Plain fa = make_frag<Plain>(av);
#pragma unroll
        for (int n = 0; n < NT; ++n) mma(accE[n], fa, yT.get(16 * n + lr, j0));
      }
#pragma unroll
      for (int n = 0; n < NT; ++n) {
        f32x4 e;
#pragma unroll
        for (int r = 0; r < 4; ++r) e[r] = bet[16 * I + 4 * lq + r] * accE[n][r];
        eT.put4(16 * n + lr, 16 * I + 4 * lq, e);
      }
    }
    __syncthreads();

    // ---- O = Qbar S + L E
    const float *Lc = a.L_ws + (((size_t)b * a.H_k + hk) * a.N_c + c) * (size_t)(C * C);
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const int I = w * RB + rb;
      const int row = 16 * I + lr;
      for (int s = 0; s * 32 < 16 * I + 16; ++s) {
        const int j0 = 32 * s + 8 * lq;
        float lv[8];
        ld8(Lc + row * C + j0, lv);
        const Split fl = make_frag<Split>(lv);
#pragma unroll
        for (int n = 0; n < NT; ++n) mma(accO[rb][n], fl, eT.get(16 * n + lr, j0));
      }
#pragma unroll
      for (int n = 0; n < NT; ++n) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int tr = 16 * I + 4 * lq + r;
          if (t0 + tr < T) st(op + (size_t)(b * T + t0 + tr) * v_row + hv * a.d_v + c0 + 16 * n + lr, accO[rb][n][r]);
        }
      }
    }

    // ---- S = F_c S + Khat^T E
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      const int i0 = (w * CB + cb) * 16;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float gam = __expf(lam[(C - 1) * G + ((i0 + 4 * lq + r) >> gs)]);
#pragma unroll
        for (int n = 0; n < NT; ++n) S[cb][n][r] *= gam;
      }
      const int i = i0 + lr;
      const float lamC = lam[(C - 1) * G + (i >> gs)];
#pragma unroll
      for (int s = 0; s < C / 32; ++s) {
        const int tt0 = 32 * s + 8 * lq;
        float kh[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int tt = tt0 + e;
          kh[e] = static_cast<float>(ks[tt * DK + i]) * __expf(lamC - lam[tt * G + (i >> gs)]);
        }
        const Split fkh = make_frag<Split>(kh);
#pragma unroll
        for (int n = 0; n < NT; ++n) mma(S[cb][n], fkh, eT.get(16 * n + lr, tt0));
      }
#pragma unroll
      for (int n = 0; n < NT; ++n) sT.put4(16 * n + lr, i0 + 4 * lq, S[cb][n]);
    }
    __syncthreads();
  }

  if (a.hT) {
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      const int i0 = (w * CB + cb) * 16;
#pragma unroll
      for (int n = 0; n < NT; ++n) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int i = i0 + 4 * lq + r, col = c0 + 16 * n + lr;
          a.hT[sbase + (size_t)i * a.d_v + col] = S[cb][n][r];
        }
      }
    }
  }
}

static size_t scan_lds_bytes(int C, int d_k, int G, int BV, bool in_bf16) {
  return sizeof(float) * (size_t)C * G + (in_bf16 ? 2 : 4) * (size_t)C * d_k + 4 * (size_t)BV * d_k +
         8 * (size_t)BV * C + sizeof(float) * (size_t)C;
}

// Value-column tile width: 32 when that already gives a workgroup per CU
// (256 of them), else 16 for more parallelism; 0 if neither fits in LDS.
int scan_choose_bv(int B, int H_v, int C, int d_k, int d_v, int G, bool in_bf16) {
  if (!(C == 64 || C == 128) || !(d_k == 64 || d_k == 128 || d_k == 256) || d_v % 16 != 0) return 0;
  const size_t cap = 160 * 1024;
  const bool fit32 = d_v % 32 == 0 && scan_lds_bytes(C, d_k, G, 32, in_bf16) <= cap;
  const bool fit16 = scan_lds_bytes(C, d_k, G, 16, in_bf16) <= cap;
  const long n32 = (long)B * H_v * (d_v / 32);
  if (fit32 && (n32 >= 256 || !fit16)) return 32;
  return fit16 ? 16 : 0;
}

template <typename TIn, typename TOut, class P, int C, int DK, int BV>
static hipError_t launch_scan_t(const ChunkArgs &a, hipStream_t stream) {
  const size_t lds = ScanLds<C, DK, BV, TIn>::bytes(a.G);
  auto kern = scan_kernel<TIn, TOut, P, C, DK, BV>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  dim3 grid(a.d_v / BV, a.H_v, a.B);
  hipLaunchKernelGGL(kern, grid, dim3(256), lds, stream, a);
  return hipGetLastError();
}

template <typename TIn, typename TOut, class P, int C, int DK>
static hipError_t launch_scan_bv(const ChunkArgs &a, hipStream_t s) {
  const int bv = scan_choose_bv(a.B, a.H_v, C, DK, a.d_v, a.G, sizeof(TIn) == 2);
  if (bv == 32) return launch_scan_t<TIn, TOut, P, C, DK, 32>(a, s);
  if (bv == 16) return launch_scan_t<TIn, TOut, P, C, DK, 16>(a, s);
  return hipErrorInvalidValue;
}

template <typename TIn, typename TOut, class P>
static hipError_t launch_scan_shape(const ChunkArgs &a, hipStream_t s) {
  switch (a.C * 1000 + a.d_k) {
    case 64064: return launch_scan_bv<TIn, TOut, P, 64, 64>(a, s);
    case 64128: return launch_scan_bv<TIn, TOut, P, 64, 128>(a, s);
    case 64256: return launch_scan_bv<TIn, TOut, P, 64, 256>(a, s);
    case 128064: return launch_scan_bv<TIn, TOut, P, 128, 64>(a, s);
    case 128128: return launch_scan_bv<TIn, TOut, P, 128, 128>(a, s);
    case 128256: return launch_scan_bv<TIn, TOut, P, 128, 256>(a, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_scan(const ChunkArgs &a, bool in_bf16, bool out_bf16, hipStream_t stream) {
  if (in_bf16) {
    if (out_bf16) return launch_scan_shape<bf16, bf16, PrecBF16>(a, stream);
    return launch_scan_shape<bf16, float, PrecBF16>(a, stream);
  }
  if (out_bf16) return launch_scan_shape<float, bf16, PrecF32>(a, stream);
  return launch_scan_shape<float, float, PrecF32>(a, stream);
}

}  // namespace gdr
