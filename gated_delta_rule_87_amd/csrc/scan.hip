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
//
// Pipelining.  The chunk loop is latency-bound (one workgroup per CU, one
// wave per SIMD), so every global operand of chunk c+1 is requested while
// chunk c computes: each prefetch register set is refilled right after its
// last use, a full chunk before it is needed.  LDS rows are padded by 16 bytes
// so the 16 rows one fragment read touches sit in different banks.  With
// C = 64 and d_k <= 128 the carried keys Khat^T are built once per chunk as
// split fragments (while the small E product runs) instead of per MFMA, and
// A_c / L_c rows are prefetched too.
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace gdr {

// ------------------------------------------------------------- LDS layout
template <int C, int DK, int BV, typename TIn>
struct ScanLayout {
  static constexpr bool kStage = (C == 64) && (DK <= 128);  // Khat^T staged, A/L prefetched
  // fp32 inputs at C = 128 only fit in LDS without the row padding of lam and ks
  static constexpr bool kPad = !(C == 128 && sizeof(TIn) == 4);
  static constexpr int KS_LD = kPad ? DK + 16 / (int)sizeof(TIn) : DK;   // staged k rows (elements)
  static constexpr int KH_LD = C + 8;                       // Khat^T rows
  static constexpr int S_LD = DK + 8;                       // S^T rows
  static constexpr int Y_LD = C + 8;                        // Y^T, E^T rows
  __host__ __device__ static int lam_ld(int G) { return (kPad && G >= 32) ? G + 4 : G; }
  __host__ __device__ static size_t lam_bytes(int G) { return 4 * (size_t)C * lam_ld(G); }
  static constexpr size_t ks_bytes = sizeof(TIn) * (size_t)C * KS_LD;
  static constexpr size_t kh_bytes = kStage ? 4 * (size_t)DK * KH_LD : 0;
  static constexpr size_t s_bytes = 4 * (size_t)BV * S_LD;
  static constexpr size_t y_bytes = 4 * (size_t)BV * Y_LD;
  __host__ __device__ static size_t total(int G) {
    return lam_bytes(G) + ks_bytes + kh_bytes + s_bytes + 2 * y_bytes + 4 * (size_t)C + 4 * (size_t)DK;
  }
};

template <typename TIn, typename TOut, class P, int C, int DK, int BV>
__global__ __launch_bounds__(256) void scan_kernel(ChunkArgs a) {
  using Lay = ScanLayout<C, DK, BV, TIn>;
  constexpr bool kStage = Lay::kStage;
  constexpr int RB = C / 64;                 // 16-row token blocks per wave
  constexpr int CB = DK / 64;                // 16-row channel blocks of S per wave
  constexpr int NT = BV / 16;                // 16-column tiles
  constexpr int KSTEPS = DK / 32;
  constexpr int NKV = C * DK / (8 * 256);    // 8-element k vectors staged per thread
  constexpr int MAX_AS = 2;                  // prefetched A/L k-steps per row block (C = 64)
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
  const int LAM_LD = Lay::lam_ld(G);

  unsigned char *base = smem_raw;
  float *lam = reinterpret_cast<float *>(base);
  base += Lay::lam_bytes(G);
  TIn *ks = reinterpret_cast<TIn *>(base);
  base += Lay::ks_bytes;
  OperandLds<P> khT, sT, yT, eT;
  if constexpr (kStage) {
    khT.init(base, DK, Lay::KH_LD);
    base += Lay::kh_bytes;
  }
  sT.init(base, BV, Lay::S_LD);
  base += Lay::s_bytes;
  yT.init(base, BV, Lay::Y_LD);
  base += Lay::y_bytes;
  eT.init(base, BV, Lay::Y_LD);
  base += Lay::y_bytes;
  float *bet = reinterpret_cast<float *>(base);
  float *gam = bet + C;

  const TIn *qp = reinterpret_cast<const TIn *>(a.q);
  const TIn *kp = reinterpret_cast<const TIn *>(a.k);
  const TIn *vp = reinterpret_cast<const TIn *>(a.v);
  const TIn *bp = reinterpret_cast<const TIn *>(a.beta);
  const TIn *lap = reinterpret_cast<const TIn *>(a.log_alpha);
  TOut *op = reinterpret_cast<TOut *>(a.o);
  const size_t qk_row = (size_t)a.H_k * DK;   // token stride of q, k
  const size_t v_row = (size_t)a.H_v * a.d_v; // token stride of v, o
  const size_t la_row = (size_t)a.H_k * G;    // token stride of log alpha

  // ---------------------------------------------------- prefetch registers
  // Loads are unconditional: a token past T reads a clamped (valid) address
  // and is zeroed where the value is used, so no load sits behind a branch
  // that would force an early wait.  Raw input bits stay in registers until use.
  // G is a power of two (it divides d_k): row/column of a flat [C][G] index by shifts.
  const int lgG = __builtin_ctz(DK) - gs;
  const bool la_vec = G >= 8;                // log alpha rows in 8-element vectors
  Raw8<TIn> lav[NKV];                        // log alpha, flat [C][G] vectors (G >= 8)
  TIn las[NKV];                              // log alpha, flat [C][G] scalars (G < 8: C*G <= 512)
  Raw8<TIn> kr[NKV];                         // k chunk, flat [C][DK] in 8-element vectors
  TIn br;                                    // beta of token tid
  Raw8<TIn> qr[RB][KSTEPS];                  // q rows of this wave
  TIn vr[RB][NT][4];                         // v entries of this wave (D layout)
  float ar[RB][MAX_AS][8], lrow[RB][MAX_AS][8];   // A and L rows (C = 64 only)
  int kc = 0;                                // chunk the key-side registers hold

  auto row_ok = [&](int c, int t) __attribute__((always_inline)) { return c * C + t < T; };
  auto clamp_tok = [&](int c, int t) __attribute__((always_inline)) { return min(c * C + t, T - 1); };
  auto load_key_side = [&](int c) __attribute__((always_inline)) {          // log alpha, k, beta of chunk c
    kc = c;
    if (la_vec) {
#pragma unroll
      for (int j = 0; j < NKV; ++j) {
        const int e = min(8 * (tid + 256 * j), C * G - 8);
        const int t = e >> lgG, g = e & (G - 1);
        lav[j].load(lap + ((size_t)b * T + clamp_tok(c, t)) * la_row + (size_t)hk * G + g);
      }
    } else {
      // as many load instructions as the vector path: the count of memory
      // operations in flight must not depend on G
#pragma unroll
      for (int j = 0; j < NKV; ++j) {
        const int e = min(tid + 256 * j, C * G - 1);
        const int t = e >> lgG, g = e & (G - 1);
        las[j] = lap[((size_t)b * T + clamp_tok(c, t)) * la_row + (size_t)hk * G + g];
      }
    }
#pragma unroll
    for (int j = 0; j < NKV; ++j) {
      const int e = 8 * (tid + 256 * j);
      const int t = e / DK, ch = e % DK;
      kr[j].load(kp + ((size_t)b * T + clamp_tok(c, t)) * qk_row + hk * DK + ch);
    }
    br = bp[((size_t)b * T + clamp_tok(c, min(tid, C - 1))) * a.H_beta + hb];
  };
  auto store_key_side = [&]() __attribute__((always_inline)) {              // raw log alpha -> lam, k -> ks, beta -> bet
    if (la_vec) {
#pragma unroll
      for (int j = 0; j < NKV; ++j) {
        const int e = 8 * (tid + 256 * j);
        if (e < C * G) {
          const int t = e >> lgG, g = e & (G - 1);
          float x[8];
          lav[j].to_float(x);
          const float keep = row_ok(kc, t) ? 1.f : 0.f;
#pragma unroll
          for (int i = 0; i < 8; ++i) x[i] *= keep;
          *reinterpret_cast<float4 *>(lam + t * LAM_LD + g) = make_float4(x[0], x[1], x[2], x[3]);
          *reinterpret_cast<float4 *>(lam + t * LAM_LD + g + 4) = make_float4(x[4], x[5], x[6], x[7]);
        }
      }
    } else {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int e = tid + 256 * j;
        if (e < C * G) {
          const int t = e >> lgG;
          lam[t * LAM_LD + (e & (G - 1))] = row_ok(kc, t) ? static_cast<float>(las[j]) : 0.f;
        }
      }
    }
#pragma unroll
    for (int j = 0; j < NKV; ++j) {
      const int e = 8 * (tid + 256 * j);
      const int t = e / DK, ch = e % DK;
      Raw8<TIn> x = kr[j];
      if (!row_ok(kc, t)) x.zero();
      x.store(ks + t * Lay::KS_LD + ch);
    }
    if (tid < C) bet[tid] = row_ok(kc, tid) ? static_cast<float>(br) : 0.f;
  };
  auto load_rows = [&](int c) __attribute__((always_inline)) {              // q and v of this wave's token rows
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const int t = 16 * (w * RB + rb) + lr;
#pragma unroll
      for (int s = 0; s < KSTEPS; ++s)
        qr[rb][s].load(qp + ((size_t)b * T + clamp_tok(c, t)) * qk_row + hk * DK + 32 * s + 8 * lq);
#pragma unroll
      for (int n = 0; n < NT; ++n) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = 16 * (w * RB + rb) + 4 * lq + r;
          vr[rb][n][r] = vp[((size_t)b * T + clamp_tok(c, row)) * v_row + hv * a.d_v + c0 + 16 * n + lr];
        }
      }
    }
  };
  auto mat_ptr = [&](const float *ws, int heads, int head, int c) __attribute__((always_inline)) {
    return ws + (((size_t)b * heads + head) * a.N_c + c) * (size_t)(C * C);
  };
  auto load_rows_of = [&](const float *M, float (&dst)[RB][MAX_AS][8]) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const int I = w * RB + rb;
#pragma unroll
      for (int s = 0; s < MAX_AS; ++s) ld8(M + (16 * I + lr) * C + 32 * s + 8 * lq, dst[rb][s]);
    }
  };
  auto lambda_prefix = [&]() __attribute__((always_inline)) {
    for (int g = tid; g < G; g += blockDim.x) prefix_column<C>(lam + g, LAM_LD);
  };
  // exp(Lambda_t) for eight consecutive channels of row t
  auto decay8 = [&](int t, int ch0, float (&d)[8]) {
    if (gs == 0) {
      const float4 u = *reinterpret_cast<const float4 *>(lam + t * LAM_LD + ch0);
      const float4 v = *reinterpret_cast<const float4 *>(lam + t * LAM_LD + ch0 + 4);
      d[0] = u.x; d[1] = u.y; d[2] = u.z; d[3] = u.w; d[4] = v.x; d[5] = v.y; d[6] = v.z; d[7] = v.w;
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) d[e] = lam[t * LAM_LD + ((ch0 + e) >> gs)];
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) d[e] = __expf(d[e]);
  };

  // ---------------------------------------------------- state and prologue
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
  if (a.N_c > 0) {
    load_key_side(0);
    load_rows(0);
    if constexpr (kStage) {
      load_rows_of(mat_ptr(a.A_ws, a.H_beta, hb, 0), ar);
      load_rows_of(mat_ptr(a.L_ws, a.H_k, hk, 0), lrow);
      store_key_side();
      if (a.N_c > 1) load_key_side(1);
    }
  }
  __syncthreads();

  // One chunk.  Every memory instruction of a non-final chunk is
  // unconditional (prefetch indices are clamped to the last chunk), so the
  // number of memory operations in flight is the same on every path and the
  // compiler's wait counts stay exact across iterations; only the final,
  // possibly ragged chunk guards its output stores.
  auto step = [&](int c, auto tail_tag) __attribute__((always_inline)) {
    constexpr bool kTail = decltype(tail_tag)::value;
    const int t0 = c * C;
    const bool more = c + 1 < a.N_c;
    const int c1 = min(c + 1, a.N_c - 1), c2 = min(c + 2, a.N_c - 1);
    if constexpr (!kStage) {
      store_key_side();
      load_key_side(c1);
      __syncthreads();
    }
    lambda_prefix();
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
#pragma unroll
      for (int s = 0; s < KSTEPS; ++s) {
        const int ch0 = 32 * s + 8 * lq;
        float kv[8], qv[8], d[8];
        ld8(ks + t * Lay::KS_LD + ch0, kv);
        qr[rb][s].to_float(qv);
        if (!row_ok(c, t)) {
#pragma unroll
          for (int e = 0; e < 8; ++e) qv[e] = 0.f;
        }
        decay8(t, ch0, d);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          kv[e] *= d[e];
          qv[e] *= d[e];
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
        for (int r = 0; r < 4; ++r)
          y[r] = (row_ok(c, 16 * I + 4 * lq + r) ? static_cast<float>(vr[rb][n][r]) : 0.f) - accY[n][r];
        yT.put4(16 * n + lr, 16 * I + 4 * lq, y);
      }
    }
    load_rows(c1);
    __syncthreads();

    // ---- E = diag(beta) A Y;  (staged path) Khat^T;  gamma = exp(Lambda_C)
    {
      const float *Ac = mat_ptr(a.A_ws, a.H_beta, hb, c);
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        const int I = w * RB + rb;
        f32x4 accE[NT];
#pragma unroll
        for (int n = 0; n < NT; ++n) accE[n] = f32x4{0.f, 0.f, 0.f, 0.f};
        if constexpr (kStage) {
#pragma unroll
          for (int s = 0; s < MAX_AS; ++s) {
            if (s * 32 < 16 * I + 16) {
              const Plain fa = make_frag<Plain>(ar[rb][s]);
#pragma unroll
              for (int n = 0; n < NT; ++n) mma(accE[n], fa, yT.get(16 * n + lr, 32 * s + 8 * lq));
            }
          }
        } else {
          float av[C / 32][8];
#pragma unroll
          for (int s = 0; s < C / 32; ++s) ld8(Ac + (16 * I + lr) * C + 32 * s + 8 * lq, av[s]);
#pragma unroll
          for (int s = 0; s < C / 32; ++s) {
            if (s * 32 < 16 * I + 16) {
              const Plain fa = make_frag<Plain>(av[s]);
#pragma unroll
              for (int n = 0; n < NT; ++n) mma(accE[n], fa, yT.get(16 * n + lr, 32 * s + 8 * lq));
            }
          }
        }
#pragma unroll
        for (int n = 0; n < NT; ++n) {
          f32x4 e;
#pragma unroll
          for (int r = 0; r < 4; ++r) e[r] = bet[16 * I + 4 * lq + r] * accE[n][r];
          eT.put4(16 * n + lr, 16 * I + 4 * lq, e);
        }
      }
      if constexpr (kStage) {
        load_rows_of(mat_ptr(a.A_ws, a.H_beta, hb, c1), ar);
        // Khat^T[i][t] = k[t][i] exp(Lambda_C - Lambda_t): thread (channel i, token segment)
        constexpr int SEG = 256 / DK;
        constexpr int TPS = C / SEG;
        const int i = tid % DK, seg = tid / DK;
        const int gi = i >> gs;
        const float lamC = lam[(C - 1) * LAM_LD + gi];
#pragma unroll
        for (int t8 = 0; t8 < TPS; t8 += 8) {
          float kh[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int tt = seg * TPS + t8 + e;
            kh[e] = static_cast<float>(ks[tt * Lay::KS_LD + i]) * __expf(lamC - lam[tt * LAM_LD + gi]);
          }
          khT.put8(i, seg * TPS + t8, kh);
        }
      }
      for (int i = tid; i < DK; i += blockDim.x) gam[i] = __expf(lam[(C - 1) * LAM_LD + (i >> gs)]);
    }
    __syncthreads();

    // ---- O = Qbar S + L E
    {
      const float *Lc = mat_ptr(a.L_ws, a.H_k, hk, c);
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        const int I = w * RB + rb;
        if constexpr (kStage) {
#pragma unroll
          for (int s = 0; s < MAX_AS; ++s) {
            if (s * 32 < 16 * I + 16) {
              const Split fl = make_frag<Split>(lrow[rb][s]);
#pragma unroll
              for (int n = 0; n < NT; ++n) mma(accO[rb][n], fl, eT.get(16 * n + lr, 32 * s + 8 * lq));
            }
          }
        } else {
          float lv[C / 32][8];
#pragma unroll
          for (int s = 0; s < C / 32; ++s) ld8(Lc + (16 * I + lr) * C + 32 * s + 8 * lq, lv[s]);
#pragma unroll
          for (int s = 0; s < C / 32; ++s) {
            if (s * 32 < 16 * I + 16) {
              const Split fl = make_frag<Split>(lv[s]);
#pragma unroll
              for (int n = 0; n < NT; ++n) mma(accO[rb][n], fl, eT.get(16 * n + lr, 32 * s + 8 * lq));
            }
          }
        }
#pragma unroll
        for (int n = 0; n < NT; ++n) {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int tr = 16 * I + 4 * lq + r;
            if (!kTail || t0 + tr < T)
              st(op + (size_t)(b * T + t0 + tr) * v_row + hv * a.d_v + c0 + 16 * n + lr, accO[rb][n][r]);
          }
        }
      }
      if constexpr (kStage) {
        load_rows_of(mat_ptr(a.L_ws, a.H_k, hk, c1), lrow);
      }
    }

    // ---- S = F_c S + Khat^T E
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      const int i0 = (w * CB + cb) * 16;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float g_ = gam[i0 + 4 * lq + r];
#pragma unroll
        for (int n = 0; n < NT; ++n) S[cb][n][r] *= g_;
      }
      const int i = i0 + lr;
#pragma unroll
      for (int s = 0; s < C / 32; ++s) {
        const int tt0 = 32 * s + 8 * lq;
        Split fkh;
        if constexpr (kStage) {
          fkh = khT.get(i, tt0);
        } else {
          const float lamC = lam[(C - 1) * LAM_LD + (i >> gs)];
          float kh[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int tt = tt0 + e;
            kh[e] = static_cast<float>(ks[tt * Lay::KS_LD + i]) * __expf(lamC - lam[tt * LAM_LD + (i >> gs)]);
          }
          fkh = make_frag<Split>(kh);
        }
#pragma unroll
        for (int n = 0; n < NT; ++n) mma(S[cb][n], fkh, eT.get(16 * n + lr, tt0));
      }
#pragma unroll
      for (int n = 0; n < NT; ++n) sT.put4(16 * n + lr, i0 + 4 * lq, S[cb][n]);
    }
    if constexpr (kStage) {
      // Next chunk's key side into lam / ks / bet: their last readers (the
      // Khat^T build, the E product, gamma) ran before the previous barrier.
      if (more) store_key_side();
      load_key_side(c2);
    }
    __syncthreads();
  };
  for (int c = 0; c + 1 < a.N_c; ++c) step(c, std::integral_constant<bool, false>());
  if (a.N_c > 0) step(a.N_c - 1, std::integral_constant<bool, true>());


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

template <int C, int DK, int BV>
static size_t scan_lds_bytes_t(int G, bool in_bf16) {
  return in_bf16 ? ScanLayout<C, DK, BV, bf16>::total(G) : ScanLayout<C, DK, BV, float>::total(G);
}

static size_t scan_lds_bytes(int C, int d_k, int G, int BV, bool in_bf16) {
#define GDR_CASE(c_, dk_, bv_) \
  if (C == c_ && d_k == dk_ && BV == bv_) return scan_lds_bytes_t<c_, dk_, bv_>(G, in_bf16);
  GDR_CASE(64, 64, 16) GDR_CASE(64, 64, 32) GDR_CASE(64, 128, 16) GDR_CASE(64, 128, 32)
  GDR_CASE(64, 256, 16) GDR_CASE(64, 256, 32) GDR_CASE(128, 64, 16) GDR_CASE(128, 64, 32)
  GDR_CASE(128, 128, 16) GDR_CASE(128, 128, 32) GDR_CASE(128, 256, 16) GDR_CASE(128, 256, 32)
#undef GDR_CASE
  return (size_t)1 << 40;
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
  const size_t lds = ScanLayout<C, DK, BV, TIn>::total(a.G);
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
