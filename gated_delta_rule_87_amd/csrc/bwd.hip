// Backward pass of the chunkwise gated delta rule (Systolic Linear Attention,
// section 2.5, custom VJP by recomputation): the forward keeps only the
// state entering every chunk, S_{c-1}; the backward recomputes the chunk
// quantities of Table 2 and runs two kernels after the prep kernels (which,
// in backward mode, write the reverse scan's operands and fp32 copies of
// A_c and of the beta-free Gram G_c):
//
// 1. Reverse state scan (bscan_kernel), sequential over the chunks from the
//    last, parallel over (batch, value head, 32 value columns).  With the
//    upstream gradients dO_c and dS_c (of the state leaving chunk c; dS of
//    the last chunk = dhT):
//      X_c       = L_c^T dO_c + Khat_c dS_c            (the gradient of E_c)
//      D_c       = A_c^T diag(beta) X_c                 (section 2.5; = dv_c)
//      dS_{c-1}  = F_c dS_c + Qbar_c^T dO_c - Kbar_c^T D_c.
//    A_c^T and L_c^T are upper triangular; with the tokens of the chunk in
//    reverse order (J the reversal) J A^T J and J L^T J are lower triangular
//    again, so the scan reads them, J Khat, (J Qbar)^T and (J Kbar)^T as
//    ready MFMA operands in the forward's tile format and multiplies only.
//    It writes dv, X_c, every dS_c, and dh0.
//
// 2. Gradient kernel (bgrad_kernel), one workgroup per (batch, key head,
//    chunk), all chunks at once.  Per value head of the key head, over
//    32-column slabs of d_v:
//      Y = V - Kbar S_{c-1},  E~ = A Y,  E = diag(beta) E~,
//      dQbar += dO S_{c-1}^T,  dKbar -= D S_{c-1}^T,  dKhat += E dS_c^T,
//      dL += tril(dO E^T),  dG -= tril_{-1}(D E^T)   (= dM diag(beta), section 2.5),
//      dgamma += rowsum(S_{c-1} (.) dS_c),
//      dbeta_j = sum_v E~_jv (X_jv - (G^T D)_jv)     (dM = -tril_{-1}(D E~^T) through M = G diag(beta));
//    then, per key head, the decayed pair sums of dL and dG with
//    P_tj = exp(Lambda_t - Lambda_j) (t >= j):
//      dq  = dQbar (.) e^Lambda + sum_j dL_tj k_j P_tj,
//      dk  = dKbar (.) e^Lambda + dKhat (.) e^(Lambda_C - Lambda)
//            + sum_j dG_tj k_j P_tj + sum_t (dG_tj k_t + dL_tj q_t) P_tj,
//    the gradient of Lambda (each pair term also differentiated in its
//    exponent; Qbar, Kbar, Khat and F_c through e^(+-Lambda)), and its
//    reverse prefix sum over the chunk, summed over each gate group's
//    channels, is dlog_alpha.  A chunk whose total decay stays within
//    kPairRange (and whose log alpha are all <= 0) takes the pair sums as
//    fp32 MFMA products with the chunk's first token as pivot
//    (P_tj = e^{Lambda_t} e^{-Lambda_j}, every factor in [e^-64, e^64]);
//    any other chunk forms each pair's exponential on its own.
//
// Scope: chunk 64, d_k in {64, 128}, d_v a multiple of 32, exact solve,
// no document resets or momentum.
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace gdr {

constexpr int kBwdC = 64;
constexpr int kBScanWaves = 8;
constexpr float kPairRange = 64.f;   // exp(64) ~ 6e27: every pivoted factor and partial sum stays finite

bool bwd_supported(int C, int d_k, int d_v) { return C == kBwdC && (d_k == 64 || d_k == 128) && d_v % 32 == 0; }

// ------------------------------------------------------------ reverse scan
// LDS: the dS operand (B fragments of dS^T), the reversed dO, X and -D of
// the chunk (split operands), and the nonzero blocks of J A^T J and J L^T J
// followed by a zero block each.
template <int DK, int FB>
struct BScanLayout {
  static constexpr int C = kBwdC, BV = 32;
  static constexpr int S_LD = DK + 8, Y_LD = C + 8;
  static constexpr size_t s_bytes = 4 * (size_t)BV * S_LD;
  static constexpr size_t y_bytes = 4 * (size_t)BV * Y_LD;
  static constexpr int NZ = tri_blocks(C / 16);
  static constexpr size_t total = s_bytes + 3 * y_bytes + 2 * (size_t)(NZ + 1) * FB;
};

typedef unsigned u32x2b __attribute__((ext_vector_type(2)));
typedef unsigned u32x4b __attribute__((ext_vector_type(4)));

// Operands of chunk c come from the workspace tiles the backward prep wrote
// (regions named as in the forward: A = J (diag(beta) A)^T J, L = J L^T J,
// KB = J Khat, QB = (J Qbar)^T, KH = (J Kbar)^T, GM = exp(Lambda_C)).  Row t'
// of a reversed chunk is token C - 1 - t'.  Jobs: X and D over (16-row
// block, 16-column tile) = 4 x 2 = one per wave; dS over (16-channel block,
// tile).  Operands of chunk c - 1 are requested while chunk c computes.
template <typename TG, class P, int DK>
__global__ __launch_bounds__(64 * kBScanWaves) void bscan_kernel(ChunkArgs a, BwdArgs g) {
  constexpr int C = kBwdC, BV = 32, NB = C / 16, NT = BV / 16;
  constexpr int KSTEPS = DK / 32, CSTEPS = C / 32;
  constexpr int FB = P::kF32 ? 2048 : 1024;
  using Lay = BScanLayout<DK, FB>;
  constexpr int NZ = Lay::NZ;
  constexpr int NCB = DK / 16;                         // channel blocks of dS
  constexpr int SPW = NCB * NT / kBScanWaves;          // dS jobs per wave
  constexpr int NTH = 64 * kBScanWaves;
  static_assert(NB * NT == kBScanWaves && SPW * kBScanWaves == NCB * NT, "job split");
  using IO = TileIO<P>;
  using Plain = typename P::Plain;
  using WT = typename std::conditional<P::kF32, float, f16>::type;   // X and dS_c in the workspace

  extern __shared__ __align__(16) unsigned char smem_raw[];
  StateLds<P> sT;
  OperandLds<P> dT, xT, nT;
  sT.init(smem_raw, BV, Lay::S_LD);
  dT.init(smem_raw + Lay::s_bytes, BV, Lay::Y_LD);
  xT.init(smem_raw + Lay::s_bytes + Lay::y_bytes, BV, Lay::Y_LD);
  nT.init(smem_raw + Lay::s_bytes + 2 * Lay::y_bytes, BV, Lay::Y_LD);
  unsigned char *alA = smem_raw + Lay::s_bytes + 3 * Lay::y_bytes;
  unsigned char *alL = alA + (NZ + 1) * FB;

  const int tid = threadIdx.x, w = wave_id(), l = lane_id(), lr = l & 15, lq = l >> 4;
  const int T = a.T, NC = a.N_c;
  const int NX = a.d_v / BV;
  int unit = blockIdx.x;   // units of one head on one XCD (they read the same operand tiles)
  if (gridDim.x % 8 == 0) unit = (blockIdx.x % 8) * (gridDim.x / 8) + blockIdx.x / 8;
  const int c0 = (unit % NX) * BV, hv = (unit / NX) % a.H_v, b = unit / (NX * a.H_v);
  const int hk = hv / (a.H_v / a.H_k), hb = a.beta_per_key_head ? hk : hv;
  const int XI = w % NB, Xn = w / NB;                  // X / D job
  const size_t vrow = (size_t)a.H_v * a.d_v;           // token stride of dO, X, dv
  const size_t sbase = ((size_t)b * a.H_v + hv) * DK * a.d_v;
  auto al_slot = [&](int I, int s) { return s <= I / 2 ? tri_index(I, s) : NZ; };
  auto tile = [&](int r, int heads, int head, int c) -> const void * { return ws_tile(a, r, heads, head, b, c); };
  auto sb = [&](int r) { return (w + kBScanWaves * r) % NCB; };   // dS job r: channel block
  auto sn = [&](int r) { return (w + kBScanWaves * r) / NCB; };   //            column tile
  const TG *dop = reinterpret_cast<const TG *>(g.d_o);

  // the nonzero blocks of J A^T J and J L^T J, moved by all threads in pieces
  constexpr int AL_BYTES = 2 * NZ * FB / NTH;
  constexpr int AW = AL_BYTES % 16 == 0 ? 16 : AL_BYTES % 8 == 0 ? 8 : 4;
  constexpr int ANREP = AL_BYTES / AW;
  static_assert(AL_BYTES % AW == 0 && FB % AW == 0 && ANREP * AW * NTH == 2 * NZ * FB, "operand block pieces");
  using AVec = typename std::conditional<AW == 4, unsigned,
               typename std::conditional<AW == 8, u32x2b, u32x4b>::type>::type;
  AVec alseg[ANREP];
  unsigned al_src[ANREP], al_dst[ANREP];
  bool al_isl[ANREP];
#pragma unroll
  for (int k = 0; k < ANREP; ++k) {
    const int byte = (k * NTH + tid) * AW;
    int j = byte / FB;
    const int off = byte % FB;
    al_isl[k] = j >= NZ;
    if (al_isl[k]) j -= NZ;
    int I = 0;
#pragma unroll
    for (int i = 1; i < NB; ++i) I = tri_index(i, 0) <= j ? i : I;
    al_src[k] = (I * CSTEPS + (j - tri_index(I, 0))) * FB + off;
    al_dst[k] = (al_isl[k] ? (NZ + 1) * FB : 0) + j * FB + off;
  }
  auto load_al = [&](int c) {
    const unsigned char *ta = static_cast<const unsigned char *>(tile(kWsA, a.H_beta, hb, c));
    const unsigned char *tl = static_cast<const unsigned char *>(tile(kWsL, a.H_k, hk, c));
#pragma unroll
    for (int k = 0; k < ANREP; ++k) alseg[k] = *reinterpret_cast<const AVec *>((al_isl[k] ? tl : ta) + al_src[k]);
  };
  auto put_al = [&]() {
#pragma unroll
    for (int k = 0; k < ANREP; ++k) *reinterpret_cast<AVec *>(alA + al_dst[k]) = alseg[k];
  };
  // dO of the chunk, reversed: thread -> column dn, reversed rows 4 dq4 ..
  const int dn = tid % BV, dq4 = tid / BV;
  float dov[4];
  auto load_do = [&](int c) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int row = c * C + C - 1 - (4 * dq4 + e);
      const float x = ldf(dop + ((size_t)b * T + min(row, T - 1)) * vrow + (size_t)hv * a.d_v + c0 + dn);
      dov[e] = row < T ? x : 0.f;
    }
  };
  auto put_do = [&]() { dT.put4(dn, 4 * dq4, f32x4{dov[0], dov[1], dov[2], dov[3]}); };
  Plain fkb[KSTEPS];                                   // J Khat rows of block XI
  Plain fqh[SPW][CSTEPS], fkh[SPW][CSTEPS];            // (J Qbar)^T, (J Kbar)^T rows of each dS job
  float gmv[SPW][4];                                   // exp(Lambda_C) of the job's rows
  auto load_kb = [&](int c) {
    const void *t = tile(kWsKB, a.H_k, hk, c);
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) fkb[s] = IO::get_plain(t, XI * KSTEPS + s, l);
  };
  auto load_sh = [&](int c) {
    const void *tq = tile(kWsQB, a.H_k, hk, c), *tk = tile(kWsKH, a.H_k, hk, c);
    const float *tg = static_cast<const float *>(tile(kWsGM, a.H_k, hk, c));
#pragma unroll
    for (int r = 0; r < SPW; ++r) {
#pragma unroll
      for (int s = 0; s < CSTEPS; ++s) {
        fqh[r][s] = IO::get_plain(tq, sb(r) * CSTEPS + s, l);
        fkh[r][s] = IO::get_plain(tk, sb(r) * CSTEPS + s, l);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) gmv[r][e] = tg[16 * sb(r) + 4 * lq + e];
    }
  };

  // ---- dS of the last chunk = dhT
  f32x4 dS[SPW];
#pragma unroll
  for (int r = 0; r < SPW; ++r) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int i = 16 * sb(r) + 4 * lq + e, col = c0 + 16 * sn(r) + lr;
      dS[r][e] = g.dhT ? g.dhT[sbase + (size_t)i * a.d_v + col] : 0.f;
    }
    sT.put4(16 * sn(r) + lr, 16 * sb(r) + 4 * lq, dS[r]);
  }
  for (int i = tid; i < FB / 16; i += NTH) {
    reinterpret_cast<u32x4b *>(alA + NZ * FB)[i] = u32x4b{0u, 0u, 0u, 0u};
    reinterpret_cast<u32x4b *>(alL + NZ * FB)[i] = u32x4b{0u, 0u, 0u, 0u};
  }
  if (NC > 0) {
    load_al(NC - 1);
    load_do(NC - 1);
    load_kb(NC - 1);
    load_sh(NC - 1);
  }

  for (int c = NC - 1; c >= 0; --c) {
    const int cn = c > 0 ? c - 1 : 0;
    put_al();                                          // last readers (previous chunk) were before its final barrier
    put_do();
    {
      WT *ds = static_cast<WT *>(g.dstates) + (((size_t)b * a.H_v + hv) * NC + c) * DK * a.d_v;
#pragma unroll
      for (int r = 0; r < SPW; ++r) {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          __builtin_nontemporal_store(static_cast<WT>(dS[r][e]),
                                      ds + (size_t)(16 * sb(r) + 4 * lq + e) * a.d_v + c0 + 16 * sn(r) + lr);
      }
    }
    __syncthreads();
    load_al(cn);
    load_do(cn);

    // ---- X' = (J L^T J)(J dO) + (J Khat) dS
    {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < CSTEPS; ++s) mma(acc, IO::get_plain(alL, al_slot(XI, s), l), dT.get(16 * Xn + lr, 32 * s + 8 * lq));
#pragma unroll
      for (int s = 0; s < KSTEPS; ++s) mma(acc, fkb[s], sT.get(16 * Xn + lr, 32 * s + 8 * lq));
      xT.put4(16 * Xn + lr, 16 * XI + 4 * lq, acc);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int row = c * C + C - 1 - (16 * XI + 4 * lq + e);
        if (row < T)
          static_cast<WT *>(g.x)[((size_t)b * T + row) * vrow + (size_t)hv * a.d_v + c0 + 16 * Xn + lr] =
              static_cast<WT>(acc[e]);
      }
    }
    load_kb(cn);
    __syncthreads();

    // ---- D' = (J A^T diag(beta) J) X' = J dv_c
    {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < CSTEPS; ++s) mma(acc, IO::get_plain(alA, al_slot(XI, s), l), xT.get(16 * Xn + lr, 32 * s + 8 * lq));
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int row = c * C + C - 1 - (16 * XI + 4 * lq + e);
        if (row < T) g.dv[((size_t)b * T + row) * vrow + (size_t)hv * a.d_v + c0 + 16 * Xn + lr] = acc[e];
      }
      nT.put4(16 * Xn + lr, 16 * XI + 4 * lq, -acc);
    }
    __syncthreads();

    // ---- dS <- F_c dS + (J Qbar)^T (J dO) - (J Kbar)^T D'
#pragma unroll
    for (int r = 0; r < SPW; ++r) {
#pragma unroll
      for (int e = 0; e < 4; ++e) dS[r][e] *= gmv[r][e];
#pragma unroll
      for (int s = 0; s < CSTEPS; ++s) {
        mma(dS[r], fqh[r][s], dT.get(16 * sn(r) + lr, 32 * s + 8 * lq));
        mma(dS[r], fkh[r][s], nT.get(16 * sn(r) + lr, 32 * s + 8 * lq));
      }
      sT.put4(16 * sn(r) + lr, 16 * sb(r) + 4 * lq, dS[r]);
    }
    load_sh(cn);
    __syncthreads();
  }
  if (g.dh0) {
#pragma unroll
    for (int r = 0; r < SPW; ++r) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = 16 * sb(r) + 4 * lq + e, col = c0 + 16 * sn(r) + lr;
        g.dh0[sbase + (size_t)i * a.d_v + col] = dS[r][e];
      }
    }
  }
}

// --------------------------------------------------------- gradient kernel
// LDS (floats).  Lambda for the whole item; A_c and G_c (later dL and dG);
// the value-slab region (S_{c-1}, dS_c, dO, V -> Y, X, D, E~), which holds
// the K and Q rows before and after the slabs, and finally dLambda.
template <int DK>
struct GradLayout {
  static constexpr int C = kBwdC, VS = 32;
  static constexpr int LDK = DK + 4, LDC = C + 4, LDV = VS + 4;
  static constexpr int lam = 0;
  static constexpr int au = lam + C * LDK;
  static constexpr int gu = au + C * LDC;
  static constexpr int slab = gu + C * LDC;
  static constexpr int sp = slab;
  static constexpr int ds = sp + DK * LDV;
  static constexpr int dO = ds + DK * LDV;
  static constexpr int vy = dO + C * LDV;
  static constexpr int xs = vy + C * LDV;
  static constexpr int dd = xs + C * LDV;
  static constexpr int es = dd + C * LDV;
  static constexpr int slab_end = es + C * LDV;
  static constexpr int ks = slab, qs = slab + C * LDK;
  static constexpr int pair_end = qs + C * LDK;
  static constexpr int misc = slab_end > pair_end ? slab_end : pair_end;
  static constexpr int bet = misc;
  static constexpr int dbp = bet + C;
  static constexpr int dgam = dbp + 2 * C;
  static constexpr int dlast = dgam + DK;
  static constexpr int flag = dlast + DK;
  static constexpr int total = flag + 4;
  static constexpr size_t bytes = 4 * (size_t)total;
  static_assert(bytes <= 160 * 1024, "gradient kernel LDS");
  static_assert(C * DK <= slab_end - slab, "log alpha staging fits the slab region");
};

// Rows t < nv of a [.., C rows, head stride DK] q or k slice as fp32 [C][LDK]
// (zero past T).
template <typename TIn, int DK>
__device__ __forceinline__ void load_key_rows(float *dst, const TIn *src, size_t row0, size_t rstride, int nv) {
  constexpr int C = kBwdC, LDK = DK + 4;
  for (int i = threadIdx.x; i < C * DK / 4; i += blockDim.x) {
    const int t = i / (DK / 4), ch = 4 * (i % (DK / 4));
    const TIn *p = src + (row0 + (size_t)min(t, nv - 1)) * rstride + ch;
    const float m = t < nv ? 1.f : 0.f;
    *reinterpret_cast<float4 *>(dst + t * LDK + ch) = make_float4(ldf(p) * m, ldf(p + 1) * m, ldf(p + 2) * m, ldf(p + 3) * m);
  }
}

// Grid (N_c, H_k, B); eight waves: wave w owns row block I = w % 4 and half
// h = w / 4 of the columns of every product.
template <typename TIn, typename TG, int DK>
__global__ __launch_bounds__(512) void bgrad_kernel(ChunkArgs a, BwdArgs g) {
  constexpr int C = kBwdC, VS = 32, NB = C / 16;
  constexpr int HCT = DK / 32;                         // channel tiles per half
  using Lay = GradLayout<DK>;
  constexpr int LDK = Lay::LDK, LDC = Lay::LDC, LDV = Lay::LDV;
  extern __shared__ __align__(16) float sm[];
  float *lam = sm + Lay::lam, *au = sm + Lay::au, *gu = sm + Lay::gu;
  float *sp = sm + Lay::sp, *dss = sm + Lay::ds, *dO = sm + Lay::dO, *vy = sm + Lay::vy, *xs = sm + Lay::xs;
  float *dd = sm + Lay::dd, *es = sm + Lay::es, *ks = sm + Lay::ks, *qs = sm + Lay::qs;
  float *bet = sm + Lay::bet, *dbp = sm + Lay::dbp, *dgam = sm + Lay::dgam, *dlast = sm + Lay::dlast;
  int *flag = reinterpret_cast<int *>(sm + Lay::flag);

  const int c = blockIdx.x, hk = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, w = wave_id(), l = lane_id(), lr = l & 15, lq = l >> 4;
  const int I = w & 3, h = w >> 2;
  const int T = a.T, t0 = c * C, nv = min(C, T - t0);
  const int R = a.H_v / a.H_k, G = a.G, gs = a.gshift;
  const TIn *qp = reinterpret_cast<const TIn *>(a.q) + (size_t)hk * DK;
  const TIn *kp = reinterpret_cast<const TIn *>(a.k) + (size_t)hk * DK;
  const TIn *vp = reinterpret_cast<const TIn *>(a.v);
  const TIn *bp = reinterpret_cast<const TIn *>(a.beta);
  const TIn *lap = reinterpret_cast<const TIn *>(a.log_alpha);
  const TG *dop = reinterpret_cast<const TG *>(g.d_o);
  const size_t krow = (size_t)a.H_k * DK, vrow = (size_t)a.H_v * a.d_v;
  const size_t row0 = (size_t)b * T + t0;
  auto trow = [&](int t) { return row0 + (size_t)min(t, nv - 1); };   // clamped token row

  // ---- Lambda: in-chunk prefix of log alpha per channel (zero past T);
  // flag: a positive log alpha or a total decay beyond kPairRange
  float *las = sm + Lay::slab;
  for (int i = tid; i < C * G; i += 512) {
    const int t = i / G, q = i % G;
    const float x = ldf(lap + (trow(t) * a.H_k + hk) * G + q);
    las[i] = t < nv ? x : 0.f;
  }
  if (tid == 0) flag[0] = 0;
  __syncthreads();
  if (tid < DK) {
    const int q = tid >> gs;
    float run = 0.f;
    bool wide = false;
    for (int t = 0; t < C; ++t) {
      const float x = las[t * G + q];
      wide |= x > 0.f;
      run += x;
      lam[t * LDK + tid] = run;
    }
    if (wide || !(-run <= kPairRange)) flag[0] = 1;    // several threads may store the same 1
  }
  __syncthreads();
  // ---- Kbar rows of block I as fp32 A operands (lane: row lr, channels 4 u + lq)
  load_key_rows<TIn, DK>(ks, kp, row0, krow, nv);
  {
    const float *gsrc = a.gu + (((size_t)b * a.H_k + hk) * a.N_c + c) * (C * C);
    for (int i = tid; i < C * C / 4; i += 512) {
      const int r = i / (C / 4), cc = 4 * (i % (C / 4));
      *reinterpret_cast<float4 *>(gu + r * LDC + cc) = *reinterpret_cast<const float4 *>(gsrc + r * C + cc);
    }
  }
  __syncthreads();
  float kbf[DK / 4];
#pragma unroll
  for (int u = 0; u < DK / 4; ++u) {
    const int t = 16 * I + lr, ch = 4 * u + lq;
    kbf[u] = ks[t * LDK + ch] * __expf(lam[t * LDK + ch]);
  }

  f32x4 aQ[HCT], aKb[HCT], aKh[HCT], aL[2], aG[2];
#pragma unroll
  for (int n = 0; n < HCT; ++n) aQ[n] = aKb[n] = aKh[n] = f32x4{0.f, 0.f, 0.f, 0.f};
  aL[0] = aL[1] = aG[0] = aG[1] = f32x4{0.f, 0.f, 0.f, 0.f};
  float dgacc = 0.f, dbk = 0.f;

  for (int r = 0; r < R; ++r) {
    const int hv = hk * R + r, hb = a.beta_per_key_head ? hk : hv;
    __syncthreads();                                   // the previous head's readers of A, beta and the slabs are done
    if (r == 0 || !a.beta_per_key_head) {
      const float *asrc = a.au + (((size_t)b * a.H_beta + hb) * a.N_c + c) * (C * C);
      for (int i = tid; i < C * C / 4; i += 512) {
        const int rr = i / (C / 4), cc = 4 * (i % (C / 4));
        *reinterpret_cast<float4 *>(au + rr * LDC + cc) = *reinterpret_cast<const float4 *>(asrc + rr * C + cc);
      }
      if (tid < C) {
        const float x = ldf(bp + trow(tid) * a.H_beta + hb);
        bet[tid] = tid < nv ? x : 0.f;
      }
    }
    float dbl[4] = {0.f, 0.f, 0.f, 0.f};
    const size_t sidx = (((size_t)b * a.H_v + hv) * a.N_c + c) * DK * a.d_v;
    for (int v0 = 0; v0 < a.d_v; v0 += VS) {
      __syncthreads();                                 // the previous slab's readers are done
      for (int i = tid; i < DK * VS / 4; i += 512) {
        const int rr = i / (VS / 4), cc = 4 * (i % (VS / 4));
        const size_t o = sidx + (size_t)rr * a.d_v + v0 + cc;
        *reinterpret_cast<float4 *>(sp + rr * LDV + cc) = *reinterpret_cast<const float4 *>(static_cast<const float *>(g.states) + o);
        *reinterpret_cast<float4 *>(dss + rr * LDV + cc) = *reinterpret_cast<const float4 *>(static_cast<const float *>(g.dstates) + o);
      }
      for (int i = tid; i < C * VS / 4; i += 512) {
        const int t = i / (VS / 4), cc = 4 * (i % (VS / 4));
        const size_t o = trow(t) * vrow + (size_t)hv * a.d_v + v0 + cc;
        const float m = t < nv ? 1.f : 0.f;
        const TG *pg = dop + o;
        const TIn *pv = vp + o;
        *reinterpret_cast<float4 *>(dO + t * LDV + cc) =
            make_float4(ldf(pg) * m, ldf(pg + 1) * m, ldf(pg + 2) * m, ldf(pg + 3) * m);
        *reinterpret_cast<float4 *>(vy + t * LDV + cc) =
            make_float4(ldf(pv) * m, ldf(pv + 1) * m, ldf(pv + 2) * m, ldf(pv + 3) * m);
        const float4 xv = *reinterpret_cast<const float4 *>(static_cast<const float *>(g.x) + o);
        const float4 dv = *reinterpret_cast<const float4 *>(g.dv + o);
        *reinterpret_cast<float4 *>(xs + t * LDV + cc) = make_float4(xv.x * m, xv.y * m, xv.z * m, xv.w * m);
        *reinterpret_cast<float4 *>(dd + t * LDV + cc) = make_float4(dv.x * m, dv.y * m, dv.z * m, dv.w * m);
      }
      __syncthreads();
      {                                                // Y = V - Kbar S_{c-1}, tile (I, h)
        f32x4 y = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int u = 0; u < DK / 4; ++u) y = mfma_f32(kbf[u], sp[(4 * u + lq) * LDV + 16 * h + lr], y);
#pragma unroll
        for (int e = 0; e < 4; ++e) vy[(16 * I + 4 * lq + e) * LDV + 16 * h + lr] -= y[e];
      }
      __syncthreads();
      {                                                // E~ = A Y; Z = X - G^T D; dbeta partials
        f32x4 et = {0.f, 0.f, 0.f, 0.f}, z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int J = 0; J < NB; ++J) {
          if (J <= I)
            tile_f32_n<1>(et, [&](int i, int k) { return au[(16 * I + i) * LDC + k]; },
                          [&](int k, int j) { return vy[k * LDV + 16 * h + j]; }, 16 * J);
          if (J >= I)
            tile_f32_n<1>(z, [&](int i, int k) { return gu[k * LDC + 16 * I + i]; },
                          [&](int k, int j) { return dd[k * LDV + 16 * h + j]; }, 16 * J);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int row = 16 * I + 4 * lq + e, col = 16 * h + lr;
          es[row * LDV + col] = et[e];
          dbl[e] += et[e] * (xs[row * LDV + col] - z[e]);
        }
      }
      __syncthreads();
      // products over the slab's value columns
#pragma unroll
      for (int n = 0; n < HCT; ++n) {
        const int n8 = h * HCT + n;
        auto ysp = [&](int k, int j) { return sp[(16 * n8 + j) * LDV + k]; };
        tile_f32_n<2>(aQ[n], [&](int i, int k) { return dO[(16 * I + i) * LDV + k]; }, ysp, 0);
        tile_f32_n<2>(aKb[n], [&](int i, int k) { return dd[(16 * I + i) * LDV + k]; }, ysp, 0);
        tile_f32_n<2>(aKh[n], [&](int i, int k) { return bet[16 * I + i] * es[(16 * I + i) * LDV + k]; },
                      [&](int k, int j) { return dss[(16 * n8 + j) * LDV + k]; }, 0);
      }
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) {
        const int J = 2 * jj + h;
        if (J > I) continue;
        auto ye = [&](int k, int j) { return bet[16 * J + j] * es[(16 * J + j) * LDV + k]; };
        tile_f32_n<2>(aL[jj], [&](int i, int k) { return dO[(16 * I + i) * LDV + k]; }, ye, 0);
        tile_f32_n<2>(aG[jj], [&](int i, int k) { return dd[(16 * I + i) * LDV + k]; }, ye, 0);
      }
      if (tid < DK) {
#pragma unroll 8
        for (int v = 0; v < VS; ++v) dgacc += sp[tid * LDV + v] * dss[tid * LDV + v];
      }
    }
    // dbeta of this head: sum of the partials over the 16 column lanes and both halves
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float x = dbl[e];
      x += __shfl_xor(x, 1);
      x += __shfl_xor(x, 2);
      x += __shfl_xor(x, 4);
      x += __shfl_xor(x, 8);
      dbl[e] = x;
    }
    if (lr == 0) {
#pragma unroll
      for (int e = 0; e < 4; ++e) dbp[h * C + 16 * I + 4 * lq + e] = dbl[e];
    }
    __syncthreads();
    if (tid < C) {
      const float d = dbp[tid] + dbp[C + tid];
      if (a.beta_per_key_head) {
        dbk += d;
      } else if (tid < nv) {
        g.dbeta[trow(tid) * a.H_v + hv] = d;
      }
    }
  }
  if (a.beta_per_key_head && tid < nv) g.dbeta[trow(tid) * a.H_k + hk] = dbk;

  // ---- pair sums: K, Q rows; dL (lower) and dG (strictly lower) over A and G
  __syncthreads();
  float *dls = au, *dgs = gu;
  load_key_rows<TIn, DK>(ks, kp, row0, krow, nv);
  load_key_rows<TIn, DK>(qs, qp, row0, krow, nv);
#pragma unroll
  for (int jj = 0; jj < 2; ++jj) {
    const int J = 2 * jj + h;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int row = 16 * I + 4 * lq + e, col = 16 * J + lr;
      dls[row * LDC + col] = (J <= I && row >= col) ? aL[jj][e] : 0.f;
      dgs[row * LDC + col] = (J <= I && row > col) ? -aG[jj][e] : 0.f;
    }
  }
  if (tid < DK) {
    dgam[tid] = dgacc;
    dlast[tid] = 0.f;
  }
  __syncthreads();
  const bool wide = flag[0] != 0;
  f32x4 pq[HCT], pr[HCT], pc[HCT];                      // sum_j dL P k, sum_j dG P k, sum_t (dG k + dL q) P
#pragma unroll
  for (int n = 0; n < HCT; ++n) {
    const int ch = 16 * (h * HCT + n) + lr;            // this lane's channel (B operand column / D column)
    pq[n] = pr[n] = pc[n] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (!wide) {
      // pivot = first token: P_tj = e^{Lambda_t} e^{-Lambda_j}
#pragma unroll
      for (int J = 0; J < NB; ++J) {
        if (J <= I) {                                  // row side: j in block J
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const int k = 16 * J + 4 * u + lq;
            const float yv = ks[k * LDK + ch] * __expf(-lam[k * LDK + ch]);
            pq[n] = mfma_f32(dls[(16 * I + lr) * LDC + k], yv, pq[n]);
            pr[n] = mfma_f32(dgs[(16 * I + lr) * LDC + k], yv, pr[n]);
          }
        }
        if (J >= I) {                                  // column side: t in block J
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const int k = 16 * J + 4 * u + lq;
            const float ex = __expf(lam[k * LDK + ch]);
            pc[n] = mfma_f32(dgs[k * LDC + 16 * I + lr], ks[k * LDK + ch] * ex, pc[n]);
            pc[n] = mfma_f32(dls[k * LDC + 16 * I + lr], qs[k * LDK + ch] * ex, pc[n]);
          }
        }
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float lt = lam[(16 * I + 4 * lq + e) * LDK + ch];
        const float ex = __expf(lt), exi = __expf(-lt);
        pq[n][e] *= ex;
        pr[n][e] *= ex;
        pc[n][e] *= exi;
      }
    } else {
      // each pair's exponential on its own, causal side only (t >= j)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int t = 16 * I + 4 * lq + e;
        const float lt = lam[t * LDK + ch];
        float sq = 0.f, sr = 0.f, sc = 0.f;
        for (int j = 0; j <= t; ++j) {
          const float kj = ks[j * LDK + ch] * __expf(lt - lam[j * LDK + ch]);
          sq += dls[t * LDC + j] * kj;
          sr += dgs[t * LDC + j] * kj;
        }
        for (int s = t; s < C; ++s) {
          const float p = __expf(lam[s * LDK + ch] - lt);
          sc += (dgs[s * LDC + t] * ks[s * LDK + ch] + dls[s * LDC + t] * qs[s * LDK + ch]) * p;
        }
        pq[n][e] = sq;
        pr[n][e] = sr;
        pc[n][e] = sc;
      }
    }
  }
  // ---- dq, dk and dLambda of the lane's entries
  float dl[HCT][4];
#pragma unroll
  for (int n = 0; n < HCT; ++n) {
    const int ch = 16 * (h * HCT + n) + lr;
    const float lc = lam[(C - 1) * LDK + ch];
    float last = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int t = 16 * I + 4 * lq + e;
      const float lt = lam[t * LDK + ch];
      const float ex = __expf(lt), hx = __expf(lc - lt);
      const float kv = ks[t * LDK + ch], qv = qs[t * LDK + ch];
      const float dQb = aQ[n][e], dKb = -aKb[n][e], dKh = aKh[n][e];
      const float dqv = dQb * ex + pq[n][e];
      const float dkv = dKb * ex + dKh * hx + pr[n][e] + pc[n][e];
      dl[n][e] = qv * dqv + kv * (dKb * ex + pr[n][e] - pc[n][e] - dKh * hx);
      last += kv * dKh * hx;                           // Khat's exponent Lambda_C - Lambda_t: its Lambda_C side
      if (t < nv) {
        const size_t o = (trow(t) * a.H_k + hk) * DK + ch;
        g.dq[o] = dqv;
        g.dk[o] = dkv;
      }
    }
    atomicAdd(dlast + ch, last);
  }
  __syncthreads();                                     // every read of the K and Q rows is done
  float *dlam = ks;
#pragma unroll
  for (int n = 0; n < HCT; ++n) {
    const int ch = 16 * (h * HCT + n) + lr;
#pragma unroll
    for (int e = 0; e < 4; ++e) dlam[(16 * I + 4 * lq + e) * LDK + ch] = dl[n][e];
  }
  __syncthreads();
  if (tid < DK) {
    // Lambda_C also enters F_c = diag(e^{Lambda_C}); then Lambda_t = sum_{s<=t} log alpha_s
    float run = dlast[tid] + dgam[tid] * __expf(lam[(C - 1) * LDK + tid]);
    for (int t = C - 1; t >= 0; --t) {
      run += dlam[t * LDK + tid];
      dlam[t * LDK + tid] = run;
    }
  }
  __syncthreads();
  const int cpg = DK / G;
  for (int i = tid; i < nv * G; i += 512) {
    const int t = i / G, q = i % G;
    float s = 0.f;
    for (int j = 0; j < cpg; ++j) s += dlam[t * LDK + q * cpg + j];
    g.dla[(trow(t) * a.H_k + hk) * G + q] = s;
  }
}

// ------------------------------------------- gradient kernel, fp16 operands
// The same computation for bf16 inputs with every product on fp16 MFMA
// (fp32 accumulation): operands are rounded once to fp16 in LDS, as the
// forward's scan operands are.  The d_v products use 16x16x32 tiles; the
// pair sums go over 16-token blocks (16x16x16 tiles) with block pivots, so
// that every fp16 operand stays in range whatever the decay:
//   row side   (t in block I, j in block J <= I): pivot p = first token of I,
//              P_tj = e^{Lambda_t - Lambda_p} e^{Lambda_p - Lambda_j};
//   column side (j in block J, t in block I >= J): pivot p' = last token of
//              J, P_tj = e^{Lambda_t - Lambda_p'} e^{Lambda_p' - Lambda_j}.
// Off the diagonal both factors are <= 1 (log alpha <= 0); on a diagonal
// block one factor is at most e^{range of Lambda over the block}, so a block
// whose range exceeds kDiagRange in some channel is summed entry by entry,
// and a chunk with a positive log alpha is summed entry by entry throughout.
typedef f16 f16x4 __attribute__((ext_vector_type(4)));
constexpr float kDiagRange = 8.f;   // e^8 ~ 3e3: pivoted unit-norm keys stay far inside fp16

__device__ __forceinline__ f32x4 mfma_k16(const f16x4 &a, const f16x4 &b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
}

// Inclusive prefix sum over the 64 lanes of a wave: within each 16-lane DPP
// row, then the row totals (read from lanes 15, 31, 47) added to the rows
// after them.
__device__ __forceinline__ float wave_prefix64(float x) {
  x = row_prefix16(x);
  const float t0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 15));
  const float t1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 31));
  const float t2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 47));
  const int row = lane_id() >> 4;
  return x + (row >= 1 ? t0 : 0.f) + (row >= 2 ? t1 : 0.f) + (row >= 3 ? t2 : 0.f);
}

template <int DK>
struct Grad16Layout {
  static constexpr int C = kBwdC, VS = 32;
  static constexpr int LDK = DK + 4;          // fp32 rows of Lambda, K, Q
  static constexpr int KLD = DK + 8;          // fp16 rows of Kbar and S^T
  static constexpr int CLD = C + 8;           // fp16 rows of A, G, Y^T
  static constexpr int SLD = VS + 8;          // fp16 rows of the slab operands
  static constexpr int PLD = C + 4;           // fp16 rows of dL, dG and their transposes
  static constexpr int VLD = VS + 4;          // fp32 rows of V
  static constexpr size_t lam = 0;
  static constexpr size_t kb = lam + 4 * (size_t)C * LDK;
  static constexpr size_t au = kb + 2 * (size_t)C * KLD;
  static constexpr size_t gu = au + 2 * (size_t)C * CLD;
  static constexpr size_t mats_end = gu + 2 * (size_t)C * CLD;
  static constexpr size_t pm = kb;            // after the slabs: dL, dG, dL^T, dG^T
  static constexpr size_t pm_end = pm + 4 * 2 * (size_t)C * PLD;
  static constexpr size_t slab = mats_end > pm_end ? mats_end : pm_end;
  static constexpr size_t sa = slab;                          // S_{c-1}[:, slab]   [DK][SLD]
  static constexpr size_t sb = sa + 2 * (size_t)DK * SLD;     // its transpose      [VS][KLD]
  static constexpr size_t dsa = sb + 2 * (size_t)VS * KLD;    // dS_c[:, slab]      [DK][SLD]
  static constexpr size_t doh = dsa + 2 * (size_t)DK * SLD;   // dO, D, E~, E, X    [C][SLD] each
  static constexpr size_t dh = doh + 2 * (size_t)C * SLD;
  static constexpr size_t eth = dh + 2 * (size_t)C * SLD;
  static constexpr size_t eh = eth + 2 * (size_t)C * SLD;
  static constexpr size_t xh = eh + 2 * (size_t)C * SLD;
  static constexpr size_t yt = xh + 2 * (size_t)C * SLD;      // Y^T [VS][CLD]
  static constexpr size_t vf = yt + 2 * (size_t)VS * CLD;     // V fp32 [C][VLD]
  static constexpr size_t slab_end = vf + 4 * (size_t)C * VLD;
  static constexpr size_t ks = slab, qs = ks + 4 * (size_t)C * LDK;   // after the slabs: K, Q rows fp32
  static constexpr size_t kq_end = qs + 4 * (size_t)C * LDK;
  static constexpr size_t misc = slab_end > kq_end ? slab_end : kq_end;
  static constexpr size_t bet = misc;                         // floats: beta [C], dbeta parts [2][C],
  static constexpr size_t dbp = bet + 4 * C;                  //   column sums [C], dgamma [DK],
  static constexpr size_t dbcol = dbp + 4 * 2 * C;            //   Lambda_C terms [DK], flags
  static constexpr size_t dgam = dbcol + 4 * C;
  static constexpr size_t dlast = dgam + 4 * DK;
  static constexpr size_t flags = dlast + 4 * DK;
  static constexpr size_t bytes = flags + 4 * 8;
  static_assert(bytes <= 160 * 1024, "gradient kernel LDS");
  static_assert(4 * (size_t)C * DK <= slab_end - slab, "log alpha staging fits the slab region");
};

template <typename TIn, typename TG, int DK>
__global__ __launch_bounds__(512) void bgrad16_kernel(ChunkArgs a, BwdArgs g) {
  constexpr int C = kBwdC, VS = 32, NB = C / 16;
  constexpr int HCT = DK / 32;                         // channel tiles per half
  using Lay = Grad16Layout<DK>;
  constexpr int LDK = Lay::LDK, KLD = Lay::KLD, CLD = Lay::CLD, SLD = Lay::SLD, PLD = Lay::PLD, VLD = Lay::VLD;
  extern __shared__ __align__(16) unsigned char sm8[];
  float *lam = reinterpret_cast<float *>(sm8 + Lay::lam);
  f16 *kb = reinterpret_cast<f16 *>(sm8 + Lay::kb), *au = reinterpret_cast<f16 *>(sm8 + Lay::au);
  f16 *gu = reinterpret_cast<f16 *>(sm8 + Lay::gu);
  f16 *dLh = reinterpret_cast<f16 *>(sm8 + Lay::pm), *dGh = dLh + C * PLD, *dLt = dGh + C * PLD, *dGt = dLt + C * PLD;
  f16 *sa = reinterpret_cast<f16 *>(sm8 + Lay::sa), *sb = reinterpret_cast<f16 *>(sm8 + Lay::sb);
  f16 *dsa = reinterpret_cast<f16 *>(sm8 + Lay::dsa), *doh = reinterpret_cast<f16 *>(sm8 + Lay::doh);
  f16 *dh = reinterpret_cast<f16 *>(sm8 + Lay::dh), *eth = reinterpret_cast<f16 *>(sm8 + Lay::eth);
  f16 *eh = reinterpret_cast<f16 *>(sm8 + Lay::eh), *xh = reinterpret_cast<f16 *>(sm8 + Lay::xh);
  f16 *yt = reinterpret_cast<f16 *>(sm8 + Lay::yt);
  float *vf = reinterpret_cast<float *>(sm8 + Lay::vf);
  float *ks = reinterpret_cast<float *>(sm8 + Lay::ks), *qs = reinterpret_cast<float *>(sm8 + Lay::qs);
  float *bet = reinterpret_cast<float *>(sm8 + Lay::bet), *dbp = reinterpret_cast<float *>(sm8 + Lay::dbp);
  float *dbcol = reinterpret_cast<float *>(sm8 + Lay::dbcol), *dgam = reinterpret_cast<float *>(sm8 + Lay::dgam);
  float *dlast = reinterpret_cast<float *>(sm8 + Lay::dlast);
  int *flags = reinterpret_cast<int *>(sm8 + Lay::flags);   // [0]: a positive log alpha; [1 + I]: block I too wide

  const int c = blockIdx.x, hk = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, w = wave_id(), l = lane_id(), lr = l & 15, lq = l >> 4;
  const int I = w & 3, h = w >> 2;
  const int T = a.T, t0 = c * C, nv = min(C, T - t0);
  const int R = a.H_v / a.H_k, G = a.G, gs = a.gshift;
  const TIn *qp = reinterpret_cast<const TIn *>(a.q) + (size_t)hk * DK;
  const TIn *kp = reinterpret_cast<const TIn *>(a.k) + (size_t)hk * DK;
  const TIn *vp = reinterpret_cast<const TIn *>(a.v);
  const TIn *bp = reinterpret_cast<const TIn *>(a.beta);
  const TIn *lap = reinterpret_cast<const TIn *>(a.log_alpha);
  const TG *dop = reinterpret_cast<const TG *>(g.d_o);
  const f16 *xg = static_cast<const f16 *>(g.x);
  const f16 *dsg = static_cast<const f16 *>(g.dstates);
  const size_t krow = (size_t)a.H_k * DK, vrow = (size_t)a.H_v * a.d_v;
  const size_t row0 = (size_t)b * T + t0;
  auto trow = [&](int t) { return row0 + (size_t)min(t, nv - 1); };
  auto f4 = [](float x0, float x1, float x2, float x3) {
    f16x4 r;
    r[0] = static_cast<f16>(x0); r[1] = static_cast<f16>(x1); r[2] = static_cast<f16>(x2); r[3] = static_cast<f16>(x3);
    return r;
  };

  // One slab's inputs, fetched into registers one slab ahead: 4-column
  // pieces of S_{c-1} and dS_c (SQ per thread) and of the dO, D, X and V rows
  // (one per thread).
  constexpr int SQ = DK * VS / 4 / 512;
  static_assert(SQ >= 1 && SQ * 512 * 4 == DK * VS && C * VS / 4 == 512, "slab pieces");
  const f16 *stg = static_cast<const f16 *>(g.states);
  f16x4 rS[SQ], rdS[SQ], rX;
  float4 rdO, rD, rV;
  const int pt = tid / (VS / 4), pv = 4 * (tid % (VS / 4));
  auto fetch = [&](int hv, int v0) {
    const size_t sidx = (((size_t)b * a.H_v + hv) * a.N_c + c) * DK * a.d_v;
#pragma unroll
    for (int q = 0; q < SQ; ++q) {
      const int i = tid + 512 * q, rr = i / (VS / 4), vq = 4 * (i % (VS / 4));
      const size_t o = sidx + (size_t)rr * a.d_v + v0 + vq;
      rS[q] = *reinterpret_cast<const f16x4 *>(stg + o);
      rdS[q] = *reinterpret_cast<const f16x4 *>(dsg + o);
    }
    const size_t o = trow(pt) * vrow + (size_t)hv * a.d_v + v0 + pv;
    rdO = make_float4(ldf(dop + o), ldf(dop + o + 1), ldf(dop + o + 2), ldf(dop + o + 3));
    rD = *reinterpret_cast<const float4 *>(g.dv + o);
    rX = *reinterpret_cast<const f16x4 *>(xg + o);
    rV = make_float4(ldf(vp + o), ldf(vp + o + 1), ldf(vp + o + 2), ldf(vp + o + 3));
  };
  auto stage = [&]() {
#pragma unroll
    for (int q = 0; q < SQ; ++q) {
      const int i = tid + 512 * q, rr = i / (VS / 4), vq = 4 * (i % (VS / 4));
      *reinterpret_cast<f16x4 *>(sa + rr * SLD + vq) = rS[q];
#pragma unroll
      for (int e = 0; e < 4; ++e) sb[(vq + e) * KLD + rr] = rS[q][e];
      *reinterpret_cast<f16x4 *>(dsa + rr * SLD + vq) = rdS[q];
    }
    const float m = pt < nv ? 1.f : 0.f;             // rows past T: zero
    *reinterpret_cast<f16x4 *>(doh + pt * SLD + pv) = f4(rdO.x * m, rdO.y * m, rdO.z * m, rdO.w * m);
    *reinterpret_cast<f16x4 *>(dh + pt * SLD + pv) = f4(rD.x * m, rD.y * m, rD.z * m, rD.w * m);
    *reinterpret_cast<f16x4 *>(xh + pt * SLD + pv) = pt < nv ? rX : f16x4{};
    *reinterpret_cast<float4 *>(vf + pt * VLD + pv) = make_float4(rV.x * m, rV.y * m, rV.z * m, rV.w * m);
  };
  // dgamma: TPR threads per state row, VPT columns each
  constexpr int TPR = 512 / DK, VPT = VS / TPR;
  const int gr = tid / TPR, gc = (tid % TPR) * VPT;

  // ---- every load the item starts with, issued together: log alpha of the
  // lane's token (the 64 lanes of a wave are the chunk's tokens; wave w takes
  // channels w CPW ..), the K rows, G_c, A_c and beta of the first head, and
  // the first value slab
  constexpr int CPW = DK / 8;                          // channels per wave in the Lambda prefix
  constexpr int EPT = C * DK / 512;                    // K (and Q) row elements per thread: 8 or 16
  constexpr int TPRW = DK / EPT;                       // threads per token row
  const int kt = tid / TPRW, kc = (tid % TPRW) * EPT;
  float lav[CPW];
  {
    const TIn *lrow = lap + (trow(l) * a.H_k + hk) * G;
#pragma unroll
    for (int c2 = 0; c2 < CPW; ++c2) lav[c2] = ldf(lrow + ((w * CPW + c2) >> gs));
  }
  Raw8<TIn> kraw[EPT / 8], qraw[EPT / 8];
#pragma unroll
  for (int e = 0; e < EPT / 8; ++e) kraw[e].load(kp + trow(kt) * krow + kc + 8 * e);
  const int hb0 = a.beta_per_key_head ? hk : hk * R;
  const float *gsrc = a.gu + (((size_t)b * a.H_k + hk) * a.N_c + c) * (C * C);
  const float *asrc0 = a.au + (((size_t)b * a.H_beta + hb0) * a.N_c + c) * (C * C);
  float4 graw[2], araw[2];
#pragma unroll
  for (int q2 = 0; q2 < 2; ++q2) {
    const int i = tid + 512 * q2, rr = i / (C / 4), cc = 4 * (i % (C / 4));
    graw[q2] = *reinterpret_cast<const float4 *>(gsrc + rr * C + cc);
    araw[q2] = *reinterpret_cast<const float4 *>(asrc0 + rr * C + cc);
  }
  const float bet0 = ldf(bp + trow(tid % C) * a.H_beta + hb0);
  fetch(hk * R, 0);
  if (tid < 8) flags[tid] = 0;
  __syncthreads();
  // ---- Lambda: inclusive prefix over the wave's lanes per channel (zero log
  // decay past T); the rising flag and the diagonal blocks' decay ranges
  {
    const float mt = l < nv ? 1.f : 0.f;
    bool rising = false;
    bool wide = false;
#pragma unroll
    for (int c2 = 0; c2 < CPW; ++c2) {
      const float a0 = lav[c2] * mt;
      rising |= a0 > 0.f;
      const float x = wave_prefix64(a0);
      lam[l * LDK + w * CPW + c2] = x;
      // the block's range of Lambda when log alpha <= 0 (a chunk with a
      // positive one is summed entry by entry whatever its ranges)
      wide |= !(dpp_row_bcast<0>(x) - dpp_row_bcast<15>(x) <= kDiagRange);
    }
    if (wide && (l & 15) == 0) flags[1 + (l >> 4)] = 1;   // several waves may store the same 1
    if (__ballot(rising) != 0 && l == 0) flags[0] = 1;
  }
  __syncthreads();
  // ---- Kbar = K (.) e^Lambda, G_c, A_c and beta of the first head as LDS operands
#pragma unroll
  for (int e = 0; e < EPT / 8; ++e) {
    float x[8];
    kraw[e].to_float(x);
    const int ch = kc + 8 * e;
    const float m = kt < nv ? 1.f : 0.f;
    f16x8 y;
#pragma unroll
    for (int j = 0; j < 8; ++j) y[j] = static_cast<f16>(x[j] * m * __expf(lam[kt * LDK + ch + j]));
    *reinterpret_cast<f16x8 *>(kb + kt * KLD + ch) = y;
  }
#pragma unroll
  for (int q2 = 0; q2 < 2; ++q2) {
    const int i = tid + 512 * q2, rr = i / (C / 4), cc = 4 * (i % (C / 4));
    *reinterpret_cast<f16x4 *>(gu + rr * CLD + cc) = f4(graw[q2].x, graw[q2].y, graw[q2].z, graw[q2].w);
    *reinterpret_cast<f16x4 *>(au + rr * CLD + cc) = f4(araw[q2].x, araw[q2].y, araw[q2].z, araw[q2].w);
  }
  if (tid < C) bet[tid] = tid < nv ? bet0 : 0.f;

  f32x4 aQ[HCT], aKb[HCT], aKh[HCT], aL[2], aG[2];
#pragma unroll
  for (int n = 0; n < HCT; ++n) aQ[n] = aKb[n] = aKh[n] = f32x4{0.f, 0.f, 0.f, 0.f};
  aL[0] = aL[1] = aG[0] = aG[1] = f32x4{0.f, 0.f, 0.f, 0.f};
  float dgacc = 0.f, dbk = 0.f;

  for (int r = 0; r < R; ++r) {
    const int hv = hk * R + r, hb = a.beta_per_key_head ? hk : hv;
    __syncthreads();                                   // the previous head's readers are done
    if (r > 0 && !a.beta_per_key_head) {              // the first head's A and beta are staged already
      const float *asrc = a.au + (((size_t)b * a.H_beta + hb) * a.N_c + c) * (C * C);
      for (int i = tid; i < C * C / 4; i += 512) {
        const int rr = i / (C / 4), cc = 4 * (i % (C / 4));
        const float4 x = *reinterpret_cast<const float4 *>(asrc + rr * C + cc);
        *reinterpret_cast<f16x4 *>(au + rr * CLD + cc) = f4(x.x, x.y, x.z, x.w);
      }
      if (tid < C) {
        const float x = ldf(bp + trow(tid) * a.H_beta + hb);
        bet[tid] = tid < nv ? x : 0.f;
      }
    }
    if (tid < C) dbcol[tid] = 0.f;
    f32x4 aP[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};   // D E~^T of this head
    float dbl = 0.f;                                   // sum_v E~ X of token 16 I + lr (this lane's rows)
    for (int v0 = 0; v0 < a.d_v; v0 += VS) {
      __syncthreads();                                 // the previous slab's readers are done
      stage();
      if (v0 + VS < a.d_v) {
        fetch(hv, v0 + VS);
      } else if (r + 1 < R) {
        fetch(hv + 1, 0);
      } else {                                         // the pair sums' K and Q rows
#pragma unroll
        for (int e = 0; e < EPT / 8; ++e) {
          kraw[e].load(kp + trow(kt) * krow + kc + 8 * e);
          qraw[e].load(qp + trow(kt) * krow + kc + 8 * e);
        }
      }
      __syncthreads();
      {                                                // Y = V - Kbar S_{c-1}: tile (t block I, v tile h) -> Y^T
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < DK / 32; ++s)
          acc = mfma_f16(*reinterpret_cast<const f16x8 *>(kb + (16 * I + lr) * KLD + 32 * s + 8 * lq),
                         *reinterpret_cast<const f16x8 *>(sb + (16 * h + lr) * KLD + 32 * s + 8 * lq), acc);
        const int t = 16 * I + 4 * lq, v = 16 * h + lr;
        *reinterpret_cast<f16x4 *>(yt + v * CLD + t) =
            f4(vf[t * VLD + v] - acc[0], vf[(t + 1) * VLD + v] - acc[1], vf[(t + 2) * VLD + v] - acc[2],
               vf[(t + 3) * VLD + v] - acc[3]);
      }
      __syncthreads();
      {                                                // E~^T = Y^T A^T: tile (v tile h, t block I)
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < C / 32; ++s) {
          if (2 * s > I) continue;                     // A is lower triangular
          acc = mfma_f16(*reinterpret_cast<const f16x8 *>(yt + (16 * h + lr) * CLD + 32 * s + 8 * lq),
                         *reinterpret_cast<const f16x8 *>(au + (16 * I + lr) * CLD + 32 * s + 8 * lq), acc);
        }
        const int t = 16 * I + lr, v = 16 * h + 4 * lq;
        const float bt = bet[t];
        const f16x4 xv = *reinterpret_cast<const f16x4 *>(xh + t * SLD + v);
        *reinterpret_cast<f16x4 *>(eth + t * SLD + v) = f4(acc[0], acc[1], acc[2], acc[3]);
        *reinterpret_cast<f16x4 *>(eh + t * SLD + v) = f4(bt * acc[0], bt * acc[1], bt * acc[2], bt * acc[3]);
        dbl += acc[0] * static_cast<float>(xv[0]) + acc[1] * static_cast<float>(xv[1]) +
               acc[2] * static_cast<float>(xv[2]) + acc[3] * static_cast<float>(xv[3]);
      }
      __syncthreads();
      {                                                // products over the slab's 32 value columns
        const f16x8 adO = *reinterpret_cast<const f16x8 *>(doh + (16 * I + lr) * SLD + 8 * lq);
        const f16x8 aD = *reinterpret_cast<const f16x8 *>(dh + (16 * I + lr) * SLD + 8 * lq);
        const f16x8 aE = *reinterpret_cast<const f16x8 *>(eh + (16 * I + lr) * SLD + 8 * lq);
#pragma unroll
        for (int n = 0; n < HCT; ++n) {
          const int nt = h * HCT + n;
          const f16x8 bS = *reinterpret_cast<const f16x8 *>(sa + (16 * nt + lr) * SLD + 8 * lq);
          const f16x8 bdS = *reinterpret_cast<const f16x8 *>(dsa + (16 * nt + lr) * SLD + 8 * lq);
          aQ[n] = mfma_f16(adO, bS, aQ[n]);
          aKb[n] = mfma_f16(aD, bS, aKb[n]);
          aKh[n] = mfma_f16(aE, bdS, aKh[n]);
        }
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
          const int J = 2 * jj + h;
          if (J > I) continue;
          const f16x8 bE = *reinterpret_cast<const f16x8 *>(eh + (16 * J + lr) * SLD + 8 * lq);
          const f16x8 bEt = *reinterpret_cast<const f16x8 *>(eth + (16 * J + lr) * SLD + 8 * lq);
          aL[jj] = mfma_f16(adO, bE, aL[jj]);
          aP[jj] = mfma_f16(aD, bEt, aP[jj]);
        }
#pragma unroll
        for (int v = 0; v < VPT; ++v)
          dgacc += static_cast<float>(sa[gr * SLD + gc + v]) * static_cast<float>(dsa[gr * SLD + gc + v]);
      }
    }
    // dbeta_j = sum_v E~_jv X_jv - sum_{t>j} G_tj (D E~^T)_tj; dG -= (D E~^T) diag(beta), strictly lower
    dbl += __shfl_xor(dbl, 16);
    dbl += __shfl_xor(dbl, 32);
    if (lq == 0) dbp[h * C + 16 * I + lr] = dbl;
#pragma unroll
    for (int jj = 0; jj < 2; ++jj) {
      const int J = 2 * jj + h;
      if (J > I) continue;
      const int j = 16 * J + lr;
      const float bj = bet[j];
      float s2 = 0.f;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int t = 16 * I + 4 * lq + e;
        const bool below = t > j;
        const float pv = aP[jj][e];
        s2 += below ? static_cast<float>(gu[t * CLD + j]) * pv : 0.f;
        aG[jj][e] -= below ? pv * bj : 0.f;
      }
      atomicAdd(dbcol + j, s2);
    }
    __syncthreads();
    if (tid < C) {
      const float d = dbp[tid] + dbp[C + tid] - dbcol[tid];
      if (a.beta_per_key_head) {
        dbk += d;
      } else if (tid < nv) {
        g.dbeta[trow(tid) * a.H_v + hv] = d;
      }
    }
  }
  if (a.beta_per_key_head && tid < nv) g.dbeta[trow(tid) * a.H_k + hk] = dbk;

  // ---- pair sums
  __syncthreads();                                     // slab operands, Kbar, A and G are dead
#pragma unroll
  for (int e = 0; e < EPT / 8; ++e) {
    float xk[8], xq[8];
    kraw[e].to_float(xk);
    qraw[e].to_float(xq);
    const float m = kt < nv ? 1.f : 0.f;
    float *pk = ks + kt * LDK + kc + 8 * e, *pq = qs + kt * LDK + kc + 8 * e;
    *reinterpret_cast<float4 *>(pk) = make_float4(xk[0] * m, xk[1] * m, xk[2] * m, xk[3] * m);
    *reinterpret_cast<float4 *>(pk + 4) = make_float4(xk[4] * m, xk[5] * m, xk[6] * m, xk[7] * m);
    *reinterpret_cast<float4 *>(pq) = make_float4(xq[0] * m, xq[1] * m, xq[2] * m, xq[3] * m);
    *reinterpret_cast<float4 *>(pq + 4) = make_float4(xq[4] * m, xq[5] * m, xq[6] * m, xq[7] * m);
  }
#pragma unroll
  for (int jj = 0; jj < 2; ++jj) {
    const int J = 2 * jj + h, j = 16 * J + lr;
    f16x4 lv, gv;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int t = 16 * I + 4 * lq + e;
      lv[e] = static_cast<f16>((J <= I && t >= j) ? aL[jj][e] : 0.f);
      gv[e] = static_cast<f16>((J <= I && t > j) ? aG[jj][e] : 0.f);
      dLh[t * PLD + j] = lv[e];
      dGh[t * PLD + j] = gv[e];
    }
    *reinterpret_cast<f16x4 *>(dLt + j * PLD + 16 * I + 4 * lq) = lv;
    *reinterpret_cast<f16x4 *>(dGt + j * PLD + 16 * I + 4 * lq) = gv;
  }
#pragma unroll
  for (int m = 1; m < TPR; m <<= 1) dgacc += __shfl_xor(dgacc, m);
  if (tid % TPR == 0) dgam[gr] = dgacc;
  if (tid < DK) dlast[tid] = 0.f;
  __syncthreads();
  const bool rising = flags[0] != 0;
  const bool diag_wide = flags[1 + I] != 0;
  f32x4 pq[HCT], pr[HCT], pc[HCT];                      // sum_j dL P k, sum_j dG P k, sum_t (dG k + dL q) P
#pragma unroll
  for (int n = 0; n < HCT; ++n) {
    const int ch = 16 * (h * HCT + n) + lr;
    pq[n] = pr[n] = pc[n] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (!rising) {
      const float lp = lam[16 * I * LDK + ch], lpc = lam[(16 * I + 15) * LDK + ch];
      f32x4 aq = {0.f, 0.f, 0.f, 0.f}, ar = aq, ac = aq;
#pragma unroll
      for (int J = 0; J < NB; ++J) {
        if (J < I || (J == I && !diag_wide)) {         // row side: j in block J
          f16x4 bk;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int j = 16 * J + 4 * lq + e;
            bk[e] = static_cast<f16>(ks[j * LDK + ch] * __expf(lp - lam[j * LDK + ch]));
          }
          aq = mfma_k16(*reinterpret_cast<const f16x4 *>(dLh + (16 * I + lr) * PLD + 16 * J + 4 * lq), bk, aq);
          ar = mfma_k16(*reinterpret_cast<const f16x4 *>(dGh + (16 * I + lr) * PLD + 16 * J + 4 * lq), bk, ar);
        }
        if (J > I || (J == I && !diag_wide)) {         // column side: t in block J
          f16x4 bk, bq;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int t = 16 * J + 4 * lq + e;
            const float f = __expf(lam[t * LDK + ch] - lpc);
            bk[e] = static_cast<f16>(ks[t * LDK + ch] * f);
            bq[e] = static_cast<f16>(qs[t * LDK + ch] * f);
          }
          ac = mfma_k16(*reinterpret_cast<const f16x4 *>(dGt + (16 * I + lr) * PLD + 16 * J + 4 * lq), bk, ac);
          ac = mfma_k16(*reinterpret_cast<const f16x4 *>(dLt + (16 * I + lr) * PLD + 16 * J + 4 * lq), bq, ac);
        }
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float lt = lam[(16 * I + 4 * lq + e) * LDK + ch];
        const float rf = __expf(lt - lp), cf = __expf(lpc - lt);
        pq[n][e] = aq[e] * rf;
        pr[n][e] = ar[e] * rf;
        pc[n][e] = ac[e] * cf;
      }
    }
    if (rising || diag_wide) {
      // pairs summed entry by entry, causal side only: all pairs of the chunk
      // (rising), or those inside this row block's diagonal block
      const int lo = rising ? 0 : 16 * I, hi = rising ? C : 16 * I + 16;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int t = 16 * I + 4 * lq + e;
        const float lt = lam[t * LDK + ch];
        float sq = 0.f, sr = 0.f, sc = 0.f;
        for (int j = lo; j <= t; ++j) {
          const float kj = ks[j * LDK + ch] * __expf(lt - lam[j * LDK + ch]);
          sq += static_cast<float>(dLh[t * PLD + j]) * kj;
          sr += static_cast<float>(dGh[t * PLD + j]) * kj;
        }
        for (int s = t; s < hi; ++s) {
          const float p = __expf(lam[s * LDK + ch] - lt);
          sc += (static_cast<float>(dGh[s * PLD + t]) * ks[s * LDK + ch] +
                 static_cast<float>(dLh[s * PLD + t]) * qs[s * LDK + ch]) * p;
        }
        pq[n][e] += sq;
        pr[n][e] += sr;
        pc[n][e] += sc;
      }
    }
  }
  // ---- dq, dk and dLambda of the lane's entries
  float dl[HCT][4];
#pragma unroll
  for (int n = 0; n < HCT; ++n) {
    const int ch = 16 * (h * HCT + n) + lr;
    const float lc = lam[(C - 1) * LDK + ch];
    float last = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int t = 16 * I + 4 * lq + e;
      const float lt = lam[t * LDK + ch];
      const float ex = __expf(lt), hx = __expf(lc - lt);
      const float kv = ks[t * LDK + ch], qv = qs[t * LDK + ch];
      const float dQb = aQ[n][e], dKb = -aKb[n][e], dKh = aKh[n][e];
      const float dqv = dQb * ex + pq[n][e];
      const float dkv = dKb * ex + dKh * hx + pr[n][e] + pc[n][e];
      dl[n][e] = qv * dqv + kv * (dKb * ex + pr[n][e] - pc[n][e] - dKh * hx);
      last += kv * dKh * hx;
      if (t < nv) {
        const size_t o = (trow(t) * a.H_k + hk) * DK + ch;
        g.dq[o] = dqv;
        g.dk[o] = dkv;
      }
    }
    atomicAdd(dlast + ch, last);
  }
  __syncthreads();                                     // every read of the K and Q rows is done
  float *dlam = ks;
#pragma unroll
  for (int n = 0; n < HCT; ++n) {
    const int ch = 16 * (h * HCT + n) + lr;
#pragma unroll
    for (int e = 0; e < 4; ++e) dlam[(16 * I + 4 * lq + e) * LDK + ch] = dl[n][e];
  }
  __syncthreads();
  // Lambda_C also enters F_c = diag(e^{Lambda_C}); Lambda_t = sum_{s<=t} log alpha_s,
  // so dlog alpha_t is the suffix sum of dLambda over the chunk: over the
  // wave's lanes (tokens), wave w taking channels w CPW ..
  const int cpg = DK / G;                              // channels per gate group
  float sv[CPW];
#pragma unroll
  for (int c2 = 0; c2 < CPW; ++c2) {
    const int ch = w * CPW + c2;
    float x = dlam[l * LDK + ch];
    if (l == C - 1) x += dlast[ch] + dgam[ch] * __expf(lam[(C - 1) * LDK + ch]);
    const float p = wave_prefix64(x);
    const float tot = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, p), 63));
    sv[c2] = tot - p + x;                              // sum over tokens l .. C - 1
  }
  if (cpg <= CPW) {
    // each gate group within the wave's channels: summed in registers, one row per lane
    if (l < nv) {
      float *drow = g.dla + (trow(l) * a.H_k + hk) * G + (w * CPW) / cpg;
      if (cpg == 1 && CPW % 4 == 0) {
#pragma unroll
        for (int c2 = 0; c2 < CPW; c2 += 4)
          *reinterpret_cast<float4 *>(drow + c2) = make_float4(sv[c2], sv[c2 + 1], sv[c2 + 2], sv[c2 + 3]);
      } else {
        float x = 0.f;                                 // cpg a power of two: groups end at c2 + 1 = k cpg
#pragma unroll
        for (int c2 = 0; c2 < CPW; ++c2) {
          x += sv[c2];
          if (((c2 + 1) & (cpg - 1)) == 0) {
            drow[c2 / cpg] = x;
            x = 0.f;
          }
        }
      }
    }
  } else {
    // groups spanning several waves' channels: through LDS
#pragma unroll
    for (int c2 = 0; c2 < CPW; ++c2) dlam[l * LDK + w * CPW + c2] = sv[c2];
    __syncthreads();
    for (int i = tid; i < nv * G; i += 512) {
      const int t = i / G, q = i % G;
      float x = 0.f;
      for (int j = 0; j < cpg; ++j) x += dlam[t * LDK + q * cpg + j];
      g.dla[(trow(t) * a.H_k + hk) * G + q] = x;
    }
  }
}

// ---------------------------------------------------------------- launchers
template <typename TG, class P, int DK>
static hipError_t launch_bscan_t(const ChunkArgs &a, const BwdArgs &g, hipStream_t s) {
  const size_t lds = BScanLayout<DK, P::kF32 ? 2048 : 1024>::total;
  auto kern = bscan_kernel<TG, P, DK>;
  hipError_t e = allow_full_lds(reinterpret_cast<const void *>(kern));
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3((a.d_v / 32) * a.H_v * a.B), dim3(64 * kBScanWaves), lds, s, a, g);
  return hipGetLastError();
}

template <typename TG, class P>
static hipError_t launch_bscan_dk(const ChunkArgs &a, const BwdArgs &g, hipStream_t s) {
  if (a.d_k == 64) return launch_bscan_t<TG, P, 64>(a, g, s);
  if (a.d_k == 128) return launch_bscan_t<TG, P, 128>(a, g, s);
  return hipErrorInvalidValue;
}

hipError_t launch_bwd_scan(const ChunkArgs &a, const BwdArgs &g, bool in_bf16, bool g_bf16, hipStream_t s) {
  if (!bwd_supported(a.C, a.d_k, a.d_v)) return hipErrorInvalidValue;
  if (in_bf16) return g_bf16 ? launch_bscan_dk<bf16, PrecF16>(a, g, s) : launch_bscan_dk<float, PrecF16>(a, g, s);
  return g_bf16 ? launch_bscan_dk<bf16, PrecF32>(a, g, s) : launch_bscan_dk<float, PrecF32>(a, g, s);
}

template <typename TIn, typename TG, int DK>
static hipError_t launch_grad_t(const ChunkArgs &a, const BwdArgs &g, hipStream_t s) {
  // fp32 inputs: every product in fp32; bf16 inputs: fp16 operands
  void (*kern)(ChunkArgs, BwdArgs);
  size_t lds;
  if constexpr (std::is_same<TIn, float>::value) {
    kern = bgrad_kernel<TIn, TG, DK>;
    lds = GradLayout<DK>::bytes;
  } else {
    kern = bgrad16_kernel<TIn, TG, DK>;
    lds = Grad16Layout<DK>::bytes;
  }
  hipError_t e = allow_full_lds(reinterpret_cast<const void *>(kern));
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3(a.N_c, a.H_k, a.B), dim3(512), lds, s, a, g);
  return hipGetLastError();
}

template <typename TIn, typename TG>
static hipError_t launch_grad_dk(const ChunkArgs &a, const BwdArgs &g, hipStream_t s) {
  if (a.d_k == 64) return launch_grad_t<TIn, TG, 64>(a, g, s);
  if (a.d_k == 128) return launch_grad_t<TIn, TG, 128>(a, g, s);
  return hipErrorInvalidValue;
}

hipError_t launch_bwd_grad(const ChunkArgs &a, const BwdArgs &g, bool in_bf16, bool g_bf16, hipStream_t s) {
  if (!bwd_supported(a.C, a.d_k, a.d_v)) return hipErrorInvalidValue;
  if (in_bf16) return g_bf16 ? launch_grad_dk<bf16, bf16>(a, g, s) : launch_grad_dk<bf16, float>(a, g, s);
  return g_bf16 ? launch_grad_dk<float, bf16>(a, g, s) : launch_grad_dk<float, float>(a, g, s);
}

}  // namespace gdr
