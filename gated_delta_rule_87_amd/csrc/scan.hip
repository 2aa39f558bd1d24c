// State scan + output: per (batch, value head, tile of BV value columns) walk
// the chunks in order, carrying the d_k x BV slice of the state S in MFMA
// accumulators.  Per chunk c (Systolic Linear Attention, Table 2, section 2.3
// and the WY equivalence proof of section 2.4.2):
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
// Organisation.  Eight waves, two per SIMD, so one wave's memory and LDS
// latency hides behind the other's arithmetic.  Per chunk:
//   stage  wave w takes d_k/8 key channels with lane = token: the in-chunk
//          prefix Lambda of each gate column is a DPP scan across the wave
//          (no serial pass over the chunk), and the raw k rows, the decay
//          factors (exp(Lambda) with C = 64 and d_k <= 128, else Lambda) and,
//          in that case, the split Khat^T fragments go to LDS;
//   Y      jobs (16-token row block, 16-column tile);
//   E      the same jobs;
//   O, S   the same jobs, then (16-channel block, tile) jobs for S.
// A wave that owns several tiles of one row (or channel) block builds the
// block's A fragments once.  Every global operand of chunk c+1 is requested
// while chunk c computes; all loads of a non-final chunk are unconditional
// (clamped indices, bounds masking at use) so the compiler's memory-wait
// counts stay exact across iterations, and the final, possibly ragged chunk
// is peeled.  LDS rows are padded by 16 bytes so the 16 rows one fragment
// read touches sit in different banks.
//
// Gates: per-channel (G = d_k) or grouped with at most 8 groups (each wave's
// channels then share one group); other groupings are rejected on the host.
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace gdr {

constexpr int kScanWaves = 8;
enum ScanGate { kGatePerChannel = 0, kGateGrouped = 1 };

template <int C, int DK, int BV, typename TIn, int GK>
struct ScanLayout {
  static constexpr bool kStage = (C == 64) && (DK <= 128);  // exp(Lambda) + Khat^T staged; A/L prefetched
  static constexpr int KS_LD = DK + 16 / (int)sizeof(TIn);  // raw k rows (elements)
  static constexpr int LAM_LD = GK == kGatePerChannel ? DK + 4 : 8;   // decay rows (floats)
  static constexpr int KH_LD = C + 8;                       // Khat^T rows
  static constexpr int S_LD = DK + 8;                       // S^T rows
  static constexpr int Y_LD = C + 8;                        // Y^T, E^T rows
  static constexpr size_t lam_bytes = 4 * (size_t)C * LAM_LD;
  static constexpr size_t ks_bytes = sizeof(TIn) * (size_t)C * KS_LD;
  static constexpr size_t kh_bytes = kStage ? 4 * (size_t)DK * KH_LD : 0;
  static constexpr size_t s_bytes = 4 * (size_t)BV * S_LD;
  static constexpr size_t y_bytes = 4 * (size_t)BV * Y_LD;
  static constexpr size_t total = lam_bytes + ks_bytes + kh_bytes + s_bytes + 2 * y_bytes + 4 * (size_t)C +
                                  4 * (size_t)DK;
};

// Distribution of (block, tile) jobs over the eight waves: with at least
// eight blocks a wave owns blocks w, w+8, ... and every tile of each; with
// fewer, NW/NBLK waves share a block and split its tiles.
template <int NBLK, int NT>
struct WaveJobs {
  static constexpr bool kWide = NBLK >= kScanWaves;
  static constexpr int RPW = kWide ? NBLK / kScanWaves : 1;   // blocks per wave
  static constexpr int WPR = kWide ? 1 : kScanWaves / NBLK;   // waves per block
  static constexpr int TPW = (NT + WPR - 1) / WPR;            // tiles per wave and block
  __device__ static int blk(int w, int r) { return kWide ? w + kScanWaves * r : w % NBLK; }
  __device__ static int tile(int w, int u) { return (kWide ? 0 : w / NBLK) + WPR * u; }
};

// Row-shifted copy of x inside each 16-lane row, or a row broadcast (DPP);
// lanes with no source or outside ROW_MASK receive 0.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_take(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, ROW_MASK, 0xf, true));
}
// Inclusive prefix sum across the 64 lanes of a wave: shifts by 1, 2, 4, 8
// inside each row, then the last lane of row 0 (2) is added to row 1 (3) and
// the last lane of row 1 to rows 2 and 3.
__device__ __forceinline__ float wave_prefix(float x) {
  x += dpp_take<0x111, 0xf>(x);
  x += dpp_take<0x112, 0xf>(x);
  x += dpp_take<0x114, 0xf>(x);
  x += dpp_take<0x118, 0xf>(x);
  x += dpp_take<0x142, 0xa>(x);
  x += dpp_take<0x143, 0xc>(x);
  return x;
}
__device__ __forceinline__ float lane63(float x) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 63));
}

template <typename TIn, typename TOut, class P, int C, int DK, int BV, int GK>
__global__ __launch_bounds__(64 * kScanWaves) void scan_kernel(ChunkArgs a) {
  using Lay = ScanLayout<C, DK, BV, TIn, GK>;
  constexpr bool kStage = Lay::kStage;
  constexpr bool kPC = GK == kGatePerChannel;
  constexpr int NW = kScanWaves;
  constexpr int NB = C / 16;                  // token row blocks
  constexpr int NT = BV / 16;                 // column tiles
  using J = WaveJobs<NB, NT>;                 // Y / E / O jobs
  using SJ = WaveJobs<DK / 16, NT>;           // S jobs
  constexpr int KSTEPS = DK / 32;
  constexpr int CPW = DK / NW;                // staging channels per wave
  constexpr int GW = kPC ? CPW : 1;           // gate columns scanned per wave
  constexpr int TPL = C / 64;                 // staging tokens per lane
  constexpr int MAX_AS = 2;                   // prefetched A/L k-steps per row block (C = 64)
  static_assert(CPW % 8 == 0, "staging channels per wave must be a multiple of 8");
  using Plain = typename P::Plain;
  using Split = typename P::Split;

  extern __shared__ __align__(16) unsigned char smem_raw[];
  const int G = a.G, gs = a.gshift, T = a.T;
  const int c0 = blockIdx.x * BV, hv = blockIdx.y, b = blockIdx.z;
  const int R = a.H_v / a.H_k;
  const int hk = hv / R;
  const int hb = a.beta_per_key_head ? hk : hv;
  const int w = wave_id(), l = lane_id();
  const int lr = l & 15, lq = l >> 4;
  // grouped gates: this wave's channels all lie in gate group gw; the first
  // wave of each group writes the group's shared values
  const int gw = kPC ? 0 : (CPW * w) >> gs;
  const bool g_owner = kPC || ((CPW * w) & ((1 << gs) - 1)) == 0;

  unsigned char *base = smem_raw;
  float *lam = reinterpret_cast<float *>(base);   // kStage: exp(Lambda_t); else Lambda_t  [C][LAM_LD]
  base += Lay::lam_bytes;
  TIn *ks = reinterpret_cast<TIn *>(base);        // raw k [C][KS_LD]
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
  float *bet = reinterpret_cast<float *>(base);   // beta of each token [C]
  float *gam = bet + C;                           // exp(Lambda_C) per gate column

  const TIn *qp = reinterpret_cast<const TIn *>(a.q);
  const TIn *kp = reinterpret_cast<const TIn *>(a.k);
  const TIn *vp = reinterpret_cast<const TIn *>(a.v);
  const TIn *bp = reinterpret_cast<const TIn *>(a.beta);
  const TIn *lap = reinterpret_cast<const TIn *>(a.log_alpha);
  TOut *op = reinterpret_cast<TOut *>(a.o);
  const size_t qk_row = (size_t)a.H_k * DK;   // token stride of q, k
  const size_t v_row = (size_t)a.H_v * a.d_v; // token stride of v, o
  const size_t la_row = (size_t)a.H_k * G;    // token stride of log alpha

  auto row_ok = [&](int c, int t) { return c * C + t < T; };
  auto tok = [&](int c, int t) { return (size_t)b * T + min(c * C + t, T - 1); };
  auto mat_ptr = [&](const float *ws, int heads, int head, int c) {
    return ws + (((size_t)b * heads + head) * a.N_c + c) * (size_t)(C * C);
  };
  auto gcol = [&](int ch) { return kPC ? ch : ch >> gs; };   // gate column of key channel ch

  // ---------------------------------------------------- prefetch registers
  // key side, staging layout (lane = token; channels CPW w .. CPW w + CPW - 1)
  Raw8<TIn> lav[TPL][kPC ? CPW / 8 : 1];     // log alpha, per-channel gates
  TIn las[TPL];                              // log alpha of the wave's group, grouped gates
  Raw8<TIn> kv8[TPL][CPW / 8];               // k
  TIn br[TPL];                               // beta
  // row-block jobs
  Raw8<TIn> qr[J::RPW][KSTEPS];                          // q rows
  TIn vr[J::RPW][J::TPW][4];                             // v entries (D layout)
  float ar[J::RPW][MAX_AS][8], lrow[J::RPW][MAX_AS][8];  // A_c and L_c rows (kStage)

  auto load_key_side = [&](int c) __attribute__((always_inline)) {
#pragma unroll
    for (int h = 0; h < TPL; ++h) {
      const size_t trow = tok(c, 64 * h + l);
      if constexpr (kPC) {
#pragma unroll
        for (int v8 = 0; v8 < CPW / 8; ++v8) lav[h][v8].load(lap + trow * la_row + (size_t)hk * G + CPW * w + 8 * v8);
      } else {
        las[h] = lap[trow * la_row + (size_t)hk * G + gw];
      }
#pragma unroll
      for (int v8 = 0; v8 < CPW / 8; ++v8) kv8[h][v8].load(kp + trow * qk_row + hk * DK + CPW * w + 8 * v8);
      br[h] = bp[trow * a.H_beta + hb];
    }
  };
  auto load_jobs = [&](int c) __attribute__((always_inline)) {
#pragma unroll
    for (int r = 0; r < J::RPW; ++r) {
      const int I = J::blk(w, r);
#pragma unroll
      for (int s = 0; s < KSTEPS; ++s) qr[r][s].load(qp + tok(c, 16 * I + lr) * qk_row + hk * DK + 32 * s + 8 * lq);
#pragma unroll
      for (int u = 0; u < J::TPW; ++u) {
        const int col = min(c0 + 16 * J::tile(w, u) + lr, a.d_v - 1);
#pragma unroll
        for (int e = 0; e < 4; ++e) vr[r][u][e] = vp[tok(c, 16 * I + 4 * lq + e) * v_row + hv * a.d_v + col];
      }
    }
  };
  auto load_mat_rows = [&](const float *M, float (&dst)[J::RPW][MAX_AS][8]) __attribute__((always_inline)) {
#pragma unroll
    for (int r = 0; r < J::RPW; ++r) {
      const int I = J::blk(w, r);
#pragma unroll
      for (int s = 0; s < MAX_AS; ++s) ld8(M + (16 * I + lr) * C + 32 * s + 8 * lq, dst[r][s]);
    }
  };

  // Stage chunk c from the key-side registers.
  auto stage = [&](int c) __attribute__((always_inline)) {
    float lamv[TPL][GW];
#pragma unroll
    for (int h = 0; h < TPL; ++h) {
      const float keep = row_ok(c, 64 * h + l) ? 1.f : 0.f;   // Lambda stays flat past T
      if constexpr (kPC) {
#pragma unroll
        for (int v8 = 0; v8 < CPW / 8; ++v8) {
          float x[8];
          lav[h][v8].to_float(x);
#pragma unroll
          for (int e = 0; e < 8; ++e) lamv[h][8 * v8 + e] = x[e] * keep;
        }
      } else {
        lamv[h][0] = static_cast<float>(las[h]) * keep;
      }
#pragma unroll
      for (int g = 0; g < GW; ++g) lamv[h][g] = wave_prefix(lamv[h][g]);
    }
#pragma unroll
    for (int h = 1; h < TPL; ++h) {
#pragma unroll
      for (int g = 0; g < GW; ++g) lamv[h][g] += lane63(lamv[h - 1][g]);
    }
    float lamC[GW];
#pragma unroll
    for (int g = 0; g < GW; ++g) lamC[g] = lane63(lamv[TPL - 1][g]);
#pragma unroll
    for (int h = 0; h < TPL; ++h) {
      const int t = 64 * h + l;
      float kx[CPW];
#pragma unroll
      for (int v8 = 0; v8 < CPW / 8; ++v8) {
        Raw8<TIn> z = kv8[h][v8];
        if (!row_ok(c, t)) z.zero();
        z.store(ks + t * Lay::KS_LD + CPW * w + 8 * v8);
        float x[8];
        z.to_float(x);
#pragma unroll
        for (int e = 0; e < 8; ++e) kx[8 * v8 + e] = x[e];
      }
      if constexpr (kPC) {
#pragma unroll
        for (int v4 = 0; v4 < CPW / 4; ++v4) {
          float u[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) u[e] = kStage ? __expf(lamv[h][4 * v4 + e]) : lamv[h][4 * v4 + e];
          *reinterpret_cast<float4 *>(lam + t * Lay::LAM_LD + CPW * w + 4 * v4) = make_float4(u[0], u[1], u[2], u[3]);
        }
      } else {
        if (g_owner) lam[t * Lay::LAM_LD + gw] = kStage ? __expf(lamv[h][0]) : lamv[h][0];
      }
      if constexpr (kStage) {
        float dec[GW];
#pragma unroll
        for (int g = 0; g < GW; ++g) dec[g] = __expf(lamC[g] - lamv[h][g]);
#pragma unroll
        for (int e = 0; e < CPW; ++e) khT.put(CPW * w + e, t, kx[e] * dec[kPC ? e : 0]);
      }
      if (w == 0) bet[t] = row_ok(c, t) ? static_cast<float>(br[h]) : 0.f;
    }
    if constexpr (kPC) {
      float gsel = 0.f;
#pragma unroll
      for (int e = 0; e < CPW; ++e)
        if (e == l) gsel = lamC[e];
      if (l < CPW) gam[CPW * w + l] = __expf(gsel);
    } else {
      if (g_owner && l == 0) gam[gw] = __expf(lamC[0]);
    }
  };
  // exp(Lambda_t) for channels ch0 .. ch0 + 7 of token row t
  auto decay8 = [&](int t, int ch0, float (&d)[8]) __attribute__((always_inline)) {
    if constexpr (kPC) {
      const float4 u = *reinterpret_cast<const float4 *>(lam + t * Lay::LAM_LD + ch0);
      const float4 v = *reinterpret_cast<const float4 *>(lam + t * Lay::LAM_LD + ch0 + 4);
      d[0] = u.x; d[1] = u.y; d[2] = u.z; d[3] = u.w; d[4] = v.x; d[5] = v.y; d[6] = v.z; d[7] = v.w;
      if constexpr (!kStage) {
#pragma unroll
        for (int e = 0; e < 8; ++e) d[e] = __expf(d[e]);
      }
    } else {
      float x = lam[t * Lay::LAM_LD + (ch0 >> gs)];
      if constexpr (!kStage) x = __expf(x);
#pragma unroll
      for (int e = 0; e < 8; ++e) d[e] = x;
    }
  };

  // ---------------------------------------------------- state and prologue
  f32x4 S[SJ::RPW][SJ::TPW];
  const size_t sbase = ((size_t)b * a.H_v + hv) * DK * a.d_v;
#pragma unroll
  for (int r = 0; r < SJ::RPW; ++r) {
    const int i0 = 16 * SJ::blk(w, r);
#pragma unroll
    for (int u = 0; u < SJ::TPW; ++u) {
      const int n = SJ::tile(w, u);
      if (n >= NT) continue;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = i0 + 4 * lq + e, col = c0 + 16 * n + lr;
        S[r][u][e] = a.h0 ? a.h0[sbase + (size_t)i * a.d_v + col] : 0.f;
      }
      sT.put4(16 * n + lr, i0 + 4 * lq, S[r][u]);
    }
  }
  if (a.N_c > 0) {
    load_key_side(0);
    load_jobs(0);
    if constexpr (kStage) {
      load_mat_rows(mat_ptr(a.A_ws, a.H_beta, hb, 0), ar);
      load_mat_rows(mat_ptr(a.L_ws, a.H_k, hk, 0), lrow);
    }
  }

  // One chunk.  Every memory instruction of a non-final chunk is
  // unconditional (prefetch indices are clamped to the last chunk); only the
  // final, possibly ragged chunk guards its output stores.
  auto step = [&](int c, auto tail_tag) __attribute__((always_inline)) {
    constexpr bool kTail = decltype(tail_tag)::value;
    const int t0 = c * C;
    const int c1 = min(c + 1, a.N_c - 1);

    // ---- stage (the previous chunk's readers of lam, ks, khT, bet and gam
    //      finished before the barrier that ended it)
    stage(c);
    load_key_side(c1);
    __syncthreads();

    // ---- Y = V - Kbar S and Qbar S
    f32x4 accO[J::RPW][J::TPW];
#pragma unroll
    for (int r = 0; r < J::RPW; ++r) {
      const int I = J::blk(w, r);
      const int t = 16 * I + lr;
      const float qkeep = row_ok(c, t) ? 1.f : 0.f;
      f32x4 accY[J::TPW];
#pragma unroll
      for (int u = 0; u < J::TPW; ++u) accY[u] = accO[r][u] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < KSTEPS; ++s) {
        const int ch0 = 32 * s + 8 * lq;
        float kv[8], qv[8], d[8];
        ld8(ks + t * Lay::KS_LD + ch0, kv);
        qr[r][s].to_float(qv);
        decay8(t, ch0, d);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          kv[e] *= d[e];
          qv[e] *= d[e] * qkeep;
        }
        const Plain fk = make_frag<Plain>(kv);
        const Split fq = make_frag<Split>(qv);
#pragma unroll
        for (int u = 0; u < J::TPW; ++u) {
          const int n = J::tile(w, u);
          if (n >= NT) continue;
          const Split fs = sT.get(16 * n + lr, ch0);
          mma(accY[u], fk, fs);
          mma(accO[r][u], fq, fs);
        }
      }
#pragma unroll
      for (int u = 0; u < J::TPW; ++u) {
        const int n = J::tile(w, u);
        if (n >= NT) continue;
        f32x4 y;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          y[e] = (row_ok(c, 16 * I + 4 * lq + e) ? static_cast<float>(vr[r][u][e]) : 0.f) - accY[u][e];
        yT.put4(16 * n + lr, 16 * I + 4 * lq, y);
      }
    }
    load_jobs(c1);
    __syncthreads();

    // ---- E = diag(beta) A Y
    {
      const float *Ac = mat_ptr(a.A_ws, a.H_beta, hb, c);
#pragma unroll
      for (int r = 0; r < J::RPW; ++r) {
        const int I = J::blk(w, r);
        f32x4 accE[J::TPW];
#pragma unroll
        for (int u = 0; u < J::TPW; ++u) accE[u] = f32x4{0.f, 0.f, 0.f, 0.f};
        float av[kStage ? 1 : C / 32][8];
        if constexpr (!kStage) {
#pragma unroll
          for (int s = 0; s < C / 32; ++s) ld8(Ac + (16 * I + lr) * C + 32 * s + 8 * lq, av[s]);
        }
#pragma unroll
        for (int s = 0; s < C / 32; ++s) {
          if (s * 32 >= 16 * I + 16) continue;   // A_c is lower triangular
          Plain fa;
          if constexpr (kStage) fa = make_frag<Plain>(ar[r][s]);
          else fa = make_frag<Plain>(av[s]);
#pragma unroll
          for (int u = 0; u < J::TPW; ++u) {
            const int n = J::tile(w, u);
            if (n < NT) mma(accE[u], fa, yT.get(16 * n + lr, 32 * s + 8 * lq));
          }
        }
#pragma unroll
        for (int u = 0; u < J::TPW; ++u) {
          const int n = J::tile(w, u);
          if (n >= NT) continue;
          f32x4 e;
#pragma unroll
          for (int x = 0; x < 4; ++x) e[x] = bet[16 * I + 4 * lq + x] * accE[u][x];
          eT.put4(16 * n + lr, 16 * I + 4 * lq, e);
        }
      }
      if constexpr (kStage) load_mat_rows(mat_ptr(a.A_ws, a.H_beta, hb, c1), ar);
    }
    __syncthreads();

    // ---- O = Qbar S + L E
    {
      const float *Lc = mat_ptr(a.L_ws, a.H_k, hk, c);
#pragma unroll
      for (int r = 0; r < J::RPW; ++r) {
        const int I = J::blk(w, r);
        float lv[kStage ? 1 : C / 32][8];
        if constexpr (!kStage) {
#pragma unroll
          for (int s = 0; s < C / 32; ++s) ld8(Lc + (16 * I + lr) * C + 32 * s + 8 * lq, lv[s]);
        }
#pragma unroll
        for (int s = 0; s < C / 32; ++s) {
          if (s * 32 >= 16 * I + 16) continue;   // L_c is lower triangular
          Split fl;
          if constexpr (kStage) fl = make_frag<Split>(lrow[r][s]);
          else fl = make_frag<Split>(lv[s]);
#pragma unroll
          for (int u = 0; u < J::TPW; ++u) {
            const int n = J::tile(w, u);
            if (n < NT) mma(accO[r][u], fl, eT.get(16 * n + lr, 32 * s + 8 * lq));
          }
        }
        TOut *orow = op + ((size_t)b * T + t0 + 16 * I + 4 * lq) * v_row + hv * a.d_v + c0 + lr;
#pragma unroll
        for (int u = 0; u < J::TPW; ++u) {
          const int n = J::tile(w, u);
          if (n >= NT) continue;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            if (!kTail || t0 + 16 * I + 4 * lq + e < T) st(orow + e * v_row + 16 * n, accO[r][u][e]);
          }
        }
      }
      if constexpr (kStage) load_mat_rows(mat_ptr(a.L_ws, a.H_k, hk, c1), lrow);
    }

    // ---- S = F_c S + Khat^T E
#pragma unroll
    for (int r = 0; r < SJ::RPW; ++r) {
      const int i0 = 16 * SJ::blk(w, r);
#pragma unroll
      for (int u = 0; u < SJ::TPW; ++u) {
        if (SJ::tile(w, u) >= NT) continue;
#pragma unroll
        for (int e = 0; e < 4; ++e) S[r][u][e] *= gam[gcol(i0 + 4 * lq + e)];
      }
      const int i = i0 + lr;
#pragma unroll
      for (int s = 0; s < C / 32; ++s) {
        const int tt0 = 32 * s + 8 * lq;
        Split fkh;
        if constexpr (kStage) {
          fkh = khT.get(i, tt0);
        } else {
          const float lC = lam[(C - 1) * Lay::LAM_LD + gcol(i)];
          float kh[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int tt = tt0 + e;
            kh[e] = static_cast<float>(ks[tt * Lay::KS_LD + i]) * __expf(lC - lam[tt * Lay::LAM_LD + gcol(i)]);
          }
          fkh = make_frag<Split>(kh);
        }
#pragma unroll
        for (int u = 0; u < SJ::TPW; ++u) {
          const int n = SJ::tile(w, u);
          if (n < NT) mma(S[r][u], fkh, eT.get(16 * n + lr, tt0));
        }
      }
#pragma unroll
      for (int u = 0; u < SJ::TPW; ++u) {
        const int n = SJ::tile(w, u);
        if (n < NT) sT.put4(16 * n + lr, i0 + 4 * lq, S[r][u]);
      }
    }
    __syncthreads();
  };
  for (int c = 0; c + 1 < a.N_c; ++c) step(c, std::integral_constant<bool, false>());
  if (a.N_c > 0) step(a.N_c - 1, std::integral_constant<bool, true>());

  if (a.hT) {
#pragma unroll
    for (int r = 0; r < SJ::RPW; ++r) {
      const int i0 = 16 * SJ::blk(w, r);
#pragma unroll
      for (int u = 0; u < SJ::TPW; ++u) {
        const int n = SJ::tile(w, u);
        if (n >= NT) continue;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int i = i0 + 4 * lq + e, col = c0 + 16 * n + lr;
          a.hT[sbase + (size_t)i * a.d_v + col] = S[r][u][e];
        }
      }
    }
  }
}

static size_t scan_lds_bytes(int C, int d_k, int BV, bool in_bf16, int gk) {
#define GDR_CASE(c_, dk_, bv_)                                                                        \
  if (C == c_ && d_k == dk_ && BV == bv_) {                                                           \
    if (in_bf16)                                                                                      \
      return gk ? ScanLayout<c_, dk_, bv_, bf16, 1>::total : ScanLayout<c_, dk_, bv_, bf16, 0>::total; \
    return gk ? ScanLayout<c_, dk_, bv_, float, 1>::total : ScanLayout<c_, dk_, bv_, float, 0>::total; \
  }
  GDR_CASE(64, 64, 16) GDR_CASE(64, 64, 32) GDR_CASE(64, 128, 16) GDR_CASE(64, 128, 32)
  GDR_CASE(64, 256, 16) GDR_CASE(64, 256, 32) GDR_CASE(128, 64, 16) GDR_CASE(128, 64, 32)
  GDR_CASE(128, 128, 16) GDR_CASE(128, 128, 32) GDR_CASE(128, 256, 16) GDR_CASE(128, 256, 32)
#undef GDR_CASE
  return (size_t)1 << 40;
}

static int scan_gate_kind(int d_k, int G) {
  if (G == d_k) return kGatePerChannel;
  if (G >= 1 && G <= kScanWaves && d_k % G == 0) return kGateGrouped;
  return -1;
}

// Value-column tile width: 32 when that already gives a workgroup per CU
// (256 of them), else 16 for more parallelism; 0 if the shape is not
// supported or neither fits in LDS.
int scan_choose_bv(int B, int H_v, int C, int d_k, int d_v, int G, bool in_bf16) {
  if (!(C == 64 || C == 128) || !(d_k == 64 || d_k == 128 || d_k == 256) || d_v % 16 != 0) return 0;
  const int gk = scan_gate_kind(d_k, G);
  if (gk < 0) return 0;
  const size_t cap = 160 * 1024;
  const bool fit32 = d_v % 32 == 0 && scan_lds_bytes(C, d_k, 32, in_bf16, gk) <= cap;
  const bool fit16 = scan_lds_bytes(C, d_k, 16, in_bf16, gk) <= cap;
  const long n32 = (long)B * H_v * (d_v / 32);
  if (fit32 && (n32 >= 256 || !fit16)) return 32;
  return fit16 ? 16 : 0;
}

template <typename TIn, typename TOut, class P, int C, int DK, int BV, int GK>
static hipError_t launch_scan_t(const ChunkArgs &a, hipStream_t stream) {
  const size_t lds = ScanLayout<C, DK, BV, TIn, GK>::total;
  auto kern = scan_kernel<TIn, TOut, P, C, DK, BV, GK>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  dim3 grid(a.d_v / BV, a.H_v, a.B);
  hipLaunchKernelGGL(kern, grid, dim3(64 * kScanWaves), lds, stream, a);
  return hipGetLastError();
}

template <typename TIn, typename TOut, class P, int C, int DK>
static hipError_t launch_scan_bv(const ChunkArgs &a, hipStream_t s) {
  const int bv = scan_choose_bv(a.B, a.H_v, C, DK, a.d_v, a.G, sizeof(TIn) == 2);
  const int gk = scan_gate_kind(DK, a.G);
  if (bv == 32 && gk == kGatePerChannel) return launch_scan_t<TIn, TOut, P, C, DK, 32, kGatePerChannel>(a, s);
  if (bv == 32 && gk == kGateGrouped) return launch_scan_t<TIn, TOut, P, C, DK, 32, kGateGrouped>(a, s);
  if (bv == 16 && gk == kGatePerChannel) return launch_scan_t<TIn, TOut, P, C, DK, 16, kGatePerChannel>(a, s);
  if (bv == 16 && gk == kGateGrouped) return launch_scan_t<TIn, TOut, P, C, DK, 16, kGateGrouped>(a, s);
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
