// Chunk preparation: per (batch, key head, chunk) build the beta-free Gram
// G_c (strictly lower) and the score matrix L_c (lower, diagonal included)
// with division-free relative decay, then for every beta head solve
// A_c = (I + G_c diag(beta))^{-1}.  Everything the sequential scan needs from
// q, k, beta and log alpha is written to the workspace here, where all
// chunks are processed in parallel, as ready MFMA operands (fp16 tiles for
// bf16 inputs, fp32 for fp32 inputs): diag(beta) A_c, L_c, Kbar_c, Qbar_c,
// Khat_c^T, and exp(Lambda_C).
//
// Systolic Linear Attention: Co-Designing Tile-Grouped Gated Delta Attention
// for TPUs:
//  - cumulative log-decay Lambda and the chunk matrices: Table 2;
//  - the Gram entries M_{t,j} = 1[t>j] beta_j sum_i exp(Lambda_{t,i} -
//    Lambda_{j,i}) k_{t,i} k_{j,i}: section 2.2, "Bottleneck 2";
//  - exp(+-Lambda) leaves fp32 once |Lambda| > 88.7: section 2.4.2;
//  - the exact inverse by recursive block doubling: section 2.4.3.
// Muir: Linear Attention with Sensitivity-Allocated Gating and Matched-Filter
// Readout, "Key Contributions": relative decays are split at chunk-internal
// boundaries instead of dividing by cumulative decay.
// When Good Enough Is Optimal: Multiplication-Only Matrix Inversion
// Approximation for Quantized Gated DeltaNet: truncated Neumann series with
// residual correction.
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
//
// Chunk pivot.  When no log alpha of the chunk is positive and the chunk's
// total decay -Lambda_{C-1} is within kPivotRange in every channel (true for
// any chunk of mild decay), the first token of the chunk serves as the pivot
// of every pair: the row operand K_t (.) exp(Lambda_t - Lambda_0) and the
// column operand K_j (.) exp(Lambda_0 - Lambda_j) then no longer depend on
// the pair, each block builds both once, and a pair is MFMA work only.  Every
// Lambda_t lies in [-kPivotRange, 0], so exp(+-Lambda_t) and all the factors
// formed from them stay in [exp(-kPivotRange), exp(kPivotRange)]: none
// overflows or underflows in fp32, every product keeps its relative
// precision, and entries with j > t can be large but are masked.
#include <algorithm>
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace gdr {

constexpr float kPivotRange = 64.f;  // exp(64) ~ 6e27 keeps every partial sum finite

// LDS rows of the C x C matrices are padded to C + 4 floats, so the 16 rows a
// column-strided fragment read touches fall into different banks.
__host__ __device__ inline int prep_ld(int C) { return C + 4; }
__host__ __device__ inline int prep_region0_floats(int C, int G) {
  return (C * G > C * prep_ld(C)) ? C * G : C * prep_ld(C);
}
__host__ __device__ inline int prep_tmp_floats(int C) {
  const int merge = C * (C / 2 + 4) / 2, neumann = C * 20;
  return merge > neumann ? merge : neumann;
}

constexpr int kXbLd = 20;   // row stride (floats) of the per-wave transpose buffers
constexpr int kChunkWide = 8;  // flags slot: the chunk's decay range exceeds kPivotRange

// Chunk-pivot column operands of blocks 0 .. NB - 2 (split fragments, two
// 1 KiB planes per block and channel step); only C = 64 (one row block per
// wave) takes the chunk-pivot route.
__host__ __device__ inline int prep_colop_floats(int C, int DK) {
  return C == 64 ? (C / 16 - 1) * DK * 16 : 0;
}
// The region after Lambda: G (slow route) or the solve's A (chunk-pivot
// route), followed by the solve's scratch; the chunk-pivot column operands
// overlay it before the solve.
__host__ __device__ inline int prep_union_floats(int C, int DK) {
  const int solve = C * prep_ld(C) + prep_tmp_floats(C), colop = prep_colop_floats(C, DK);
  return solve > colop ? solve : colop;
}

size_t prep_lds_bytes(int C, int DK, int G) {
  return sizeof(float) * (size_t)(prep_region0_floats(C, G) + prep_union_floats(C, DK) + C) +
         sizeof(int) * 16 + sizeof(float) * 4 * 32 * kXbLd;
}
// The chunk-pivot kernel keeps Lambda in registers: region 0 holds the
// block totals of Lambda during the build and G after it.
__host__ __device__ inline int prep_chunk_region0_floats(int C) { return C * prep_ld(C); }
size_t prep_chunk_lds_bytes(int C, int DK) {
  return sizeof(float) * (size_t)(prep_chunk_region0_floats(C) + prep_union_floats(C, DK) + C) +
         sizeof(int) * 16 + sizeof(float) * 4 * 32 * kXbLd;
}

// One lane's 32-byte fragment in LDS as two planes of 16 bytes per lane, so
// a wave's read of a plane is 1 KiB of consecutive bytes.
template <class F>
__device__ __forceinline__ void lds_put_frag(unsigned char *base, int idx, const F &f) {
  static_assert(sizeof(F) == 32, "two 16-byte planes");
  uint4 u[2];
  __builtin_memcpy(u, &f, sizeof(F));
  *reinterpret_cast<uint4 *>(base + 2048 * idx + 16 * lane_id()) = u[0];
  *reinterpret_cast<uint4 *>(base + 2048 * idx + 1024 + 16 * lane_id()) = u[1];
}
template <class F>
__device__ __forceinline__ F lds_get_frag(const unsigned char *base, int idx) {
  uint4 u[2];
  u[0] = *reinterpret_cast<const uint4 *>(base + 2048 * idx + 16 * lane_id());
  u[1] = *reinterpret_cast<const uint4 *>(base + 2048 * idx + 1024 + 16 * lane_id());
  F f;
  __builtin_memcpy(&f, u, sizeof(F));
  return f;
}

// --------------------------------------------------------------- fp32 tiles
// acc += X[i, k] * Y[k, j] for one 16x16 tile over k in [k0, k0 + 16 N)
// (element accessors; fp32 MFMA, lane l supplies X[i = l%16][k + l/16] and
// Y[k + l/16][j = l%16]).  The length is a template constant so the loop
// unrolls and its LDS reads are issued ahead of the MFMAs.
template <int N, class FX, class FY>
__device__ __forceinline__ void tile_f32_n(f32x4 &acc, const FX &x, const FY &y, int k0) {
  const int l = lane_id();
  const int i = l & 15, kk = l >> 4;
  float xa[4 * N], yb[4 * N];
#pragma unroll
  for (int u = 0; u < 4 * N; ++u) {
    xa[u] = x(i, k0 + 4 * u + kk);
    yb[u] = y(k0 + 4 * u + kk, i);
  }
#pragma unroll
  for (int u = 0; u < 4 * N; ++u) acc = mfma_f32(xa[u], yb[u], acc);
}

// Same over [k0, k1), k1 - k0 a multiple of 16 up to 16 NMAX (the longest
// contraction the caller can reach; the registers of the unrolled loads are
// sized for it).
template <int NMAX, class FX, class FY>
__device__ __forceinline__ void tile_f32(f32x4 &acc, const FX &x, const FY &y, int k0, int k1) {
  static_assert(NMAX >= 1 && NMAX <= 8, "contraction of 16 to 128");
  switch ((k1 - k0) >> 4) {
    case 1: tile_f32_n<1>(acc, x, y, k0); break;
    case 2: if constexpr (NMAX >= 2) tile_f32_n<2>(acc, x, y, k0); break;
    case 3: if constexpr (NMAX >= 3) tile_f32_n<3>(acc, x, y, k0); break;
    case 4: if constexpr (NMAX >= 4) tile_f32_n<4>(acc, x, y, k0); break;
    case 5: if constexpr (NMAX >= 5) tile_f32_n<5>(acc, x, y, k0); break;
    case 6: if constexpr (NMAX >= 6) tile_f32_n<6>(acc, x, y, k0); break;
    case 7: if constexpr (NMAX >= 7) tile_f32_n<7>(acc, x, y, k0); break;
    case 8: if constexpr (NMAX >= 8) tile_f32_n<8>(acc, x, y, k0); break;
    default: break;
  }
}

// ------------------------------------------------------------- exact solve
// amat <- (I + M)^{-1}, M = gmat diag(bet): 16x16 diagonal blocks by forward
// substitution (one lane per column), then block-doubling merges
// A[B,T] = -A[B,B] (M[B,T] A[T,T]) with fp32 MFMA.  Only the diagonal and
// lower 16x16 blocks of amat are written (and read): the blocks above the
// diagonal are zero by construction and left to the caller.
template <int C>
__device__ __forceinline__ void solve_exact(const float *gmat, const float *bet, float *amat, float *tmp) {
  constexpr int NB = C / 16;
  constexpr int LD = C + 4;
  const int tid = threadIdx.x, w = wave_id(), l = lane_id();
  if (tid < NB * 16) {
    const int base = 16 * (tid >> 4), cc = tid & 15;
    float bl[16], x[16];
#pragma unroll
    for (int m = 0; m < 16; m += 4) {
      const float4 v = *reinterpret_cast<const float4 *>(bet + base + m);
      bl[m] = v.x; bl[m + 1] = v.y; bl[m + 2] = v.z; bl[m + 3] = v.w;
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float row[16];
#pragma unroll
      for (int m = 0; m < 16; m += 4) {
        const float4 v = *reinterpret_cast<const float4 *>(gmat + (base + i) * LD + base + m);
        row[m] = v.x; row[m + 1] = v.y; row[m + 2] = v.z; row[m + 3] = v.w;
      }
      float s = (i == cc) ? 1.f : 0.f;
#pragma unroll
      for (int m = 0; m < i; ++m) s -= row[m] * bl[m] * x[m];
      x[i] = s;
      amat[(base + i) * LD + base + cc] = s;
    }
  }
  __syncthreads();
  // One job per (pair p, column tile tj): a wave forms the column tile of
  // X_p = M[bot, top] A[top, top] and then the same column of
  // A[bot, top] = -A[bot, bot] X_p, which needs only that column of X_p, so
  // the two products meet through the wave's own LDS writes, with no
  // workgroup barrier between them.
  for (int bs = 16; bs < C; bs *= 2) {
    const int tpb = bs / 16;                  // tiles per block side
    const int XLD = bs + 4;
    const int jobs = (C / (2 * bs)) * tpb;
    for (int job = w; job < jobs; job += blockDim.x / kWave) {
      const int p = job / tpb, tj = job % tpb;
      const int top = 2 * bs * p, bot = top + bs;
      const int c0 = top + 16 * tj;
      float *X = tmp + p * bs * XLD;          // pair p's X at tmp + p * bs * XLD
      for (int ti = 0; ti < tpb; ++ti) {
        const int r0 = bot + 16 * ti;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        tile_f32<C / 32>(acc,
                 [&](int i, int k) { return gmat[(r0 + i) * LD + k] * bet[k]; },
                 [&](int k, int j) { return amat[k * LD + c0 + j]; },
                 c0, top + bs);               // A[top,top] is lower: rows k >= column
#pragma unroll
        for (int r = 0; r < 4; ++r) X[(16 * ti + 4 * (l >> 4) + r) * XLD + 16 * tj + (l & 15)] = acc[r];
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");   // this wave's X column before its reads
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      for (int ti = 0; ti < tpb; ++ti) {
        const int r0 = bot + 16 * ti;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        tile_f32<C / 32>(acc,
                 [&](int i, int k) { return amat[(r0 + i) * LD + k]; },
                 [&](int k, int j) { return X[(k - bot) * XLD + 16 * tj + j]; },
                 bot, r0 + 16);               // A[bot,bot] is lower: columns k <= row
#pragma unroll
        for (int r = 0; r < 4; ++r)
          amat[(r0 + 4 * (l >> 4) + r) * LD + top + 16 * tj + (l & 15)] = -acc[r];
      }
    }
    __syncthreads();
  }
}

// ----------------------------------------------------------- Neumann solve
// X = sum_{s=0}^{m} (-M)^s by Horner (X <- I - M X, m times), then r residual
// corrections X <- X + X (I - (I + M) X).  Horner steps update X in place by
// 16-column blocks, one wave per block: tile (I, J) of M X contracts over
// k in [16 J, 16 I + 16) (X is lower triangular), that is over the tiles of
// column block J at and above row block I, so a wave that goes up its column
// from the bottom overwrites only tiles nothing later in the column reads.
// One barrier per step.  The residual products go one 16-column block of
// the result at a time, X updated in place: (I + M) X[:, J] needs only
// column block J of X, and X Rm[:, J] needs the columns of X at and right of
// J, which are still the old ones.
constexpr int kPrepWaves = 4;                 // the prep kernels run 256 threads
template <int C>
__device__ __forceinline__ void solve_neumann(const float *gmat, const float *bet, float *amat, float *tmp, int order,
                              int residual) {
  constexpr int NB = C / 16;
  constexpr int LD = C + 4;
  constexpr int TLD = 20;                     // tmp rows: one 16-column block, padded
  constexpr int kMaxTiles = (NB + 3) / 4;
  const int tid = threadIdx.x, w = wave_id(), l = lane_id();
  const int nw = blockDim.x / kWave;
  for (int i = tid; i < C * LD; i += blockDim.x) amat[i] = ((i / LD) == (i % LD)) ? 1.f : 0.f;
  __syncthreads();
  auto Mx = [&](int i, int k, int r0) { return gmat[(r0 + i) * LD + k] * bet[k]; };
  // column blocks J and NB - 1 - J share a wave: long and short columns paired
  auto owner = [](int J) { return (J < NB / 2 ? J : NB - 1 - J) % kPrepWaves; };
  for (int it = 0; it < order; ++it) {
#pragma unroll 1
    for (int J = 0; J < NB; ++J) {
      if (owner(J) != w) continue;
#pragma unroll 1
      for (int I = NB - 1; I >= J; --I) {       // one tile's operands live at a time
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        tile_f32<C / 16>(acc, [&](int i, int k) { return Mx(i, k, 16 * I); },
                 [&](int k, int j) { return amat[k * LD + 16 * J + j]; }, 16 * J, 16 * I + 16);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = 16 * I + 4 * (l >> 4) + r, col = 16 * J + (l & 15);
          amat[row * LD + col] = ((row == col) ? 1.f : 0.f) - acc[r];
        }
      }
    }
    __syncthreads();
  }
  for (int it = 0; it < residual; ++it) {
    for (int J = 0; J < NB; ++J) {
      // Rm[:, J] = I - X[:, J] - (M X)[:, J] -> tmp[row * TLD + col - 16J]
      for (int I = J + w; I < NB; I += nw) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        const int r0 = 16 * I;
        tile_f32<C / 16>(acc, [&](int i, int k) { return Mx(i, k, r0); },
                 [&](int k, int j) { return amat[k * LD + 16 * J + j]; }, 16 * J, r0 + 16);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = 16 * I + 4 * (l >> 4) + r, col = 16 * J + (l & 15);
          tmp[row * TLD + (l & 15)] = ((row == col) ? 1.f : 0.f) - amat[row * LD + col] - acc[r];
        }
      }
      __syncthreads();
      f32x4 acc[kMaxTiles];
      int nt = 0;
      for (int I = J + w; I < NB; I += nw, ++nt) {
        acc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
        const int r0 = 16 * I;
        tile_f32<C / 16>(acc[nt], [&](int i, int k) { return amat[(r0 + i) * LD + k]; },
                 [&](int k, int j) { return tmp[k * TLD + j]; }, 16 * J, r0 + 16);
      }
      __syncthreads();
      nt = 0;
      for (int I = J + w; I < NB; I += nw, ++nt) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = 16 * I + 4 * (l >> 4) + r, col = 16 * J + (l & 15);
          amat[row * LD + col] += acc[nt][r];
        }
      }
      __syncthreads();
    }
  }
}

// ------------------------------------------------------------------ kernels
// Loads are unconditional (tokens past T read a clamped, valid address and
// are zeroed where used): a load behind a branch forces an early wait for
// every memory operation in flight.
//
// Two kernels share the per-chunk steps below.  The chunk-pivot kernel
// (C = 64) takes every chunk; a chunk whose decay range is too wide for the
// chunk pivot is left to the block-pivot kernel, which runs after it and
// finds such chunks by a mark in their exp(Lambda_C) row (a negative value,
// which an exponential never produces).  For C = 128 the block-pivot kernel
// takes every chunk.

constexpr float kWideMark = -1.f;

// One (batch, key head, chunk) work item: indices, LDS carve-up, pointers.
template <typename TIn, class P, int C, int DK>
struct PrepItem {
  static constexpr int NB = C / 16;
  static constexpr int NKV = C * DK / (8 * 256);  // bound on 8-element log-alpha vectors per thread
  static constexpr int KS = DK / 32;
  using Split = typename P::Split;
  // workspace tiles: fp16 for bf16 inputs, fp32 for fp32 inputs
  using IO = TileIO<typename std::conditional<P::kF32, PrecF32, PrecF16>::type>;

  const ChunkArgs &a;
  const int c, hk, b, G, gs, T, t0, tid, w, l, lr, lq, lgG, Rb;
  // Block-pivot route: Lambda, then A, over region 0; G in the union region.
  // Chunk-pivot route: the column operands in the union region until the
  // pairs are done, then G over region 0 (Lambda is dead by then) and A in
  // the union region.  The solve's scratch follows C (C + 4) floats into the
  // union region on both routes.
  float *const smem, *const lam, *const ureg, *const tmp, *const bet;
  int *const flags;                                    // [NB] block ranges, [kChunkWide]
  float *const xb;                                     // this wave's transpose buffer [32 channels][kXbLd]
  const TIn *const la, *const bp, *const kbase, *const qbase;
  const size_t row_stride, la_row;                     // token strides of q / k and of log alpha
  void *const tKB, *const tQB, *const tKH, *const tL;

  // region0: floats before the union region
  __device__ __forceinline__ PrepItem(const ChunkArgs &a_, int c_, int hk_, int b_, float *smem_, int region0)
      : a(a_), c(c_), hk(hk_), b(b_), G(a_.G), gs(a_.gshift), T(a_.T), t0(c_ * C), tid(threadIdx.x),
        w(wave_id()), l(lane_id()), lr(lane_id() & 15), lq(lane_id() >> 4),
        lgG(__builtin_ctz(DK) - a_.gshift), Rb(a_.H_beta / a_.H_k), smem(smem_), lam(smem_),
        ureg(smem_ + region0), tmp(ureg + C * prep_ld(C)),
        bet(ureg + prep_union_floats(C, DK)), flags(reinterpret_cast<int *>(bet + C)),
        xb(reinterpret_cast<float *>(flags + 16) + wave_id() * 32 * kXbLd),
        la(reinterpret_cast<const TIn *>(a_.log_alpha)), bp(reinterpret_cast<const TIn *>(a_.beta)),
        kbase(reinterpret_cast<const TIn *>(a_.k) + (size_t)hk_ * DK),
        qbase(reinterpret_cast<const TIn *>(a_.q) + (size_t)hk_ * DK), row_stride((size_t)a_.H_k * DK),
        la_row((size_t)a_.H_k * a_.G), tKB(ws_tile(a_, kWsKB, a_.H_k, hk_, b_, c_)),
        tQB(ws_tile(a_, kWsQB, a_.H_k, hk_, b_, c_)), tKH(ws_tile(a_, kWsKH, a_.H_k, hk_, b_, c_)),
        tL(ws_tile(a_, kWsL, a_.H_k, hk_, b_, c_)) {}

  __device__ __forceinline__ size_t tok(int t) const { return (size_t)b * T + min(t0 + t, T - 1); }

  // rows 16 blk + lr of a q / k head, channels 32 s + 8 lq ..
  __device__ __forceinline__ void load_rows(Raw8<TIn> (&dst)[KS], const TIn *base, int blk) const {
    const size_t rt = tok(16 * blk + lr) * row_stride;
#pragma unroll
    for (int s = 0; s < KS; ++s) dst[s].load(base + rt + 32 * s + 8 * lq);
  }

  // Raw log alpha of the chunk, in flight between issue and use.
  struct LaRegs {
    Raw8<TIn> v[NKV];
    TIn s[NKV];
  };
  __device__ __forceinline__ void issue_la(LaRegs &r) const {
    if (G >= 8) {
#pragma unroll
      for (int j = 0; j < NKV; ++j) {
        const int e = min(8 * (tid + 256 * j), C * G - 8);
        r.v[j].load(la + tok(e >> lgG) * la_row + (size_t)hk * G + (e & (G - 1)));
      }
    } else {
#pragma unroll
      for (int j = 0; j < NKV; ++j) {
        const int e = min(tid + 256 * j, C * G - 1);
        r.s[j] = la[tok(e >> lgG) * la_row + (size_t)hk * G + (e & (G - 1))];
      }
    }
  }

  // Lambda = in-chunk prefix sum of log alpha per decay group (Systolic
  // Linear Attention, Table 2), and the decay range flags: per 16-token block
  // and over the chunk.  Ends with a barrier.
  __device__ __forceinline__ void lambda(const LaRegs &r) {
    if (G >= 8) {
#pragma unroll
      for (int j = 0; j < NKV; ++j) {
        const int e = 8 * (tid + 256 * j);
        if (e < C * G) {
          const int t = e >> lgG, g = e & (G - 1);
          float x[8];
          r.v[j].to_float(x);
          const float keep = (t0 + t < T) ? 1.f : 0.f;
          *reinterpret_cast<float4 *>(lam + t * G + g) =
              make_float4(x[0] * keep, x[1] * keep, x[2] * keep, x[3] * keep);
          *reinterpret_cast<float4 *>(lam + t * G + g + 4) =
              make_float4(x[4] * keep, x[5] * keep, x[6] * keep, x[7] * keep);
        }
      }
    } else {
#pragma unroll
      for (int j = 0; j < NKV; ++j) {
        const int e = tid + 256 * j;
        if (e < C * G) lam[e] = (t0 + (e >> lgG) < T) ? static_cast<float>(r.s[j]) : 0.f;
      }
    }
    if (tid < 16) flags[tid] = 0;
    __syncthreads();
    for (int g = tid; g < G; g += blockDim.x) prefix_column<C>(lam + g, G);
    __syncthreads();
    // several threads may store the same 1
    for (int g = tid; g < G; g += blockDim.x) {
      float clo = lam[g], chi = clo;
#pragma unroll
      for (int I = 0; I < NB; ++I) {
        float lo = lam[(16 * I) * G + g], hi = lo;
#pragma unroll
        for (int q = 1; q < 16; ++q) {
          const float x = lam[(16 * I + q) * G + g];
          lo = fminf(lo, x);
          hi = fmaxf(hi, x);
        }
        if (!(hi - lo <= kPivotRange)) flags[I] = 1;
        clo = fminf(clo, lo);
        chi = fmaxf(chi, hi);
      }
      if (!(chi - clo <= kPivotRange)) flags[kChunkWide] = 1;
    }
    __syncthreads();
  }

  __device__ __forceinline__ float *gm_row() const {
    return reinterpret_cast<float *>(ws_tile(a, kWsGM, a.H_k, hk, b, c));
  }
  __device__ __forceinline__ void write_gm() const {
    if (tid < DK) gm_row()[tid] = __expf(lam[(C - 1) * G + (tid >> gs)]);
  }

  // Lambda of row t for eight consecutive channels (vector reads per channel,
  // one broadcast read when the eight share a decay group)
  __device__ __forceinline__ void lam8(int t, int ch0, float (&x)[8]) const {
    if (gs == 0) {
      const float4 u = *reinterpret_cast<const float4 *>(lam + t * G + ch0);
      const float4 v = *reinterpret_cast<const float4 *>(lam + t * G + ch0 + 4);
      x[0] = u.x; x[1] = u.y; x[2] = u.z; x[3] = u.w; x[4] = v.x; x[5] = v.y; x[6] = v.z; x[7] = v.w;
    } else if (gs >= 3) {
      const float u = lam[t * G + (ch0 >> gs)];
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = u;
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = lam[t * G + ((ch0 + e) >> gs)];
    }
  }

  // The scan operands of channel step s of block I (Systolic Linear
  // Attention, Table 2; lane: token 16 I + lr, channels 32 s + 8 lq ..):
  // kbar = K (.) exp(Lambda_t), qbar = Q (.) exp(Lambda_t) and
  // kh = K (.) exp(Lambda_C - Lambda_t), the last transposed through the
  // wave's LDS buffer into channel-row fragments.
  __device__ __forceinline__ void scan_operands(int I, int s, const float (&kbar)[8], const float (&qbar)[8],
                                                const float (&kh)[8]) const {
    IO::put_plain8(tKB, I * KS + s, l, kbar);
    IO::put_plain8(tQB, I * KS + s, l, qbar);
    // Khat^T: lane (token lr, channels 8 lq ..) writes, lane (channel
    // 16 (l >> 5) + (l & 15), tokens 8 g ..) reads back a fragment
#pragma unroll
    for (int e = 0; e < 8; ++e) xb[(8 * lq + e) * kXbLd + lr] = kh[e];
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    const int chl = 16 * (l >> 5) + (l & 15), g = (l >> 4) & 1;
    float xt[8];
    const float4 u0 = *reinterpret_cast<const float4 *>(xb + chl * kXbLd + 8 * g);
    const float4 u1 = *reinterpret_cast<const float4 *>(xb + chl * kXbLd + 8 * g + 4);
    xt[0] = u0.x; xt[1] = u0.y; xt[2] = u0.z; xt[3] = u0.w; xt[4] = u1.x; xt[5] = u1.y; xt[6] = u1.z; xt[7] = u1.w;
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    IO::put_plain8(tKH, (2 * s + (l >> 5)) * (C / 32) + I / 2, 16 * (2 * (I & 1) + g) + (l & 15), xt);
  }

  // The 16 x 16 block (I, J) of L from an MFMA accumulator (lane: rows
  // 4 lq .. 4 lq + 3, column lr), through the wave's LDS buffer, as 32
  // fragments of 8 columns; on the diagonal block the entries above the
  // diagonal are zero.
  __device__ __forceinline__ void store_L_block(int I, int J, const f32x4 &acc) const {
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const int r = 4 * lq + q4;
      xb[r * kXbLd + lr] = (I > J || r >= lr) ? acc[q4] : 0.f;
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    const int r = l & 15, h = (l >> 4) & 1;
    const float4 u0 = *reinterpret_cast<const float4 *>(xb + r * kXbLd + 8 * h);
    const float4 u1 = *reinterpret_cast<const float4 *>(xb + r * kXbLd + 8 * h + 4);
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    if (l < 32) {
      const float v[8] = {u0.x, u0.y, u0.z, u0.w, u1.x, u1.y, u1.z, u1.w};
      IO::put_plain8(tL, I * (C / 32) + J / 2, 16 * (2 * (J & 1) + h) + r, v);
    }
  }

  // Zeros in the upper half of each 16 x 32 block of L_c that straddles the
  // diagonal, one fragment (row, 8 columns) per store; blocks wholly above
  // it (2 kb > rb) are never read and not written.
  __device__ __forceinline__ void zero_upper_L() const {
    const float z[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int u = tid; u < (C / 16) * (C / 32) * 64; u += blockDim.x) {
      const int blk = u >> 6, f = u & 63;
      const int rb = blk / (C / 32), kb = blk % (C / 32);
      if (2 * kb + (f >> 5) > rb && 2 * kb <= rb) IO::put_plain8(tL, blk, f, z);   // column block 2 kb + (f >> 5)
    }
  }

  // beta of the chunk for every beta head of this key head: element e of
  // thread tid's register j is e = tid + 256 j = rb * C + t (up to 4 * 256
  // values, C * Rb)
  static constexpr int NBET = 4;
  __device__ __forceinline__ void load_betas(TIn (&bets)[NBET]) const {
#pragma unroll
    for (int j = 0; j < NBET; ++j) {
      const int e = min(tid + 256 * j, C * Rb - 1);
      bets[j] = bp[tok(e % C) * a.H_beta + hk * Rb + e / C];
    }
  }
  __device__ __forceinline__ void put_betas(const TIn (&bets)[NBET], int rb) const {
#pragma unroll
    for (int j = 0; j < NBET; ++j) {
      const int e = tid + 256 * j;
      if (e / C == rb && e < C * Rb) bet[e % C] = (t0 + e % C < T) ? static_cast<float>(bets[j]) : 0.f;
    }
  }

  // Per beta head: A = (I + G diag(beta))^{-1} from gsolve into asolve (row
  // stride C + 4 both), then diag(beta) A to the workspace: the upper half of
  // a 16 x 32 block that straddles the diagonal as zeros, blocks wholly above
  // it not at all.  bet0_ready: the first head's beta is already in LDS
  // (written before a barrier that precedes the call).
  __device__ __forceinline__ void solve_store(float *gsolve, float *asolve, const TIn (&bets)[NBET],
                                              bool bet0_ready) const {
    for (int rb = 0; rb < Rb; ++rb) {
      const int hb = hk * Rb + rb;
      __syncthreads();
      if (rb > 0 || !bet0_ready) {
        put_betas(bets, rb);
        __syncthreads();
      }
      if (a.solve == 0) {
        solve_exact<C>(gsolve, bet, asolve, tmp);
      } else {
        solve_neumann<C>(gsolve, bet, asolve, tmp, a.order, a.residual);
      }
      __syncthreads();
      // diag(beta) A_c: the scan's chunk writes are E_c = diag(beta) A_c Y
      void *tA = ws_tile(a, kWsA, a.H_beta, hb, b, c);
      for (int u = tid; u < C * C / 8; u += blockDim.x) {   // unit = fragment (row, col .. col + 7)
        const int blk = u >> 6, f = u & 63;
        if (2 * (blk % (C / 32)) > blk / (C / 32)) continue;   // block wholly above the diagonal: not written
        const int row = 16 * (blk / (C / 32)) + (f & 15), col = 32 * (blk % (C / 32)) + 8 * (f >> 4);
        const float4 a0 = *reinterpret_cast<const float4 *>(asolve + row * (C + 4) + col);
        const float4 a1 = *reinterpret_cast<const float4 *>(asolve + row * (C + 4) + col + 4);
        const bool upper = col / 16 > row / 16;             // the half of a straddling block above the diagonal
        const float bt = bet[row];
        float x[8] = {bt * a0.x, bt * a0.y, bt * a0.z, bt * a0.w, bt * a1.x, bt * a1.y, bt * a1.z, bt * a1.w};
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = upper ? 0.f : x[e];
        IO::put_plain8(tA, blk, f, x);
      }
    }
  }
};

// Per row block I owned by a wave, both routes build
//  (1) the scan operands of its 16 tokens (scan_operands);
//  (2) the pivot-decayed row operands K (.) exp(Lambda_t - Lambda_p) and
//      Q (.) exp(Lambda_t - Lambda_p), kept as split fragments;
//  (3) Gram and L for the pairs (I, J), J <= I, each one MFMA product with the
//      decayed keys K_J (.) exp(Lambda_p - Lambda_j) of block J.

// f[i] for a lane-varying i in [0, 8) by selects (no indexed register access)
__device__ __forceinline__ float pick(const float (&f)[8], int i) {
  const float a = (i & 1) ? f[1] : f[0], b = (i & 1) ? f[3] : f[2];
  const float c = (i & 1) ? f[5] : f[4], d = (i & 1) ? f[7] : f[6];
  const float lo = (i & 2) ? b : a, hi = (i & 2) ? d : c;
  return (i & 4) ? hi : lo;
}

// Chunk-pivot route, C = 64: p = 0 for every pair; wave w owns block w and
// builds its column operand once; the operands of blocks 0 .. 2 are shared
// through LDS.  Lambda never goes through LDS whole: each lane holds log
// alpha of its token for its channels, the in-block prefix runs over the
// 16 lanes of a DPP row, and only the block totals and the first token's
// values are exchanged.  kGate: how log alpha maps onto a lane's eight
// channels (one value per channel, one 8-vector of groups, or at most four
// groups read as scalars).
enum GateMode { kGatePerChannel, kGateGroupsVec, kGateGroupsFew };
template <typename TIn, class P, int DK, int kGate>
__global__ __launch_bounds__(256) void prep_chunk_kernel(ChunkArgs a) {
  constexpr int C = 64;
  using X = PrepItem<TIn, P, C, DK>;
  using Split = typename X::Split;
  constexpr int NB = X::NB, KS = X::KS, NBET = X::NBET;
  extern __shared__ __align__(16) unsigned char smem_raw[];
  const X x(a, blockIdx.x, blockIdx.y, blockIdx.z, reinterpret_cast<float *>(smem_raw),
            prep_chunk_region0_floats(C));
  const int I = x.w, lr = x.lr, lq = x.lq, gs = x.gs, G = x.G;
  const int tr = 16 * I + lr;
  const float mt = (x.t0 + tr < x.T) ? 1.f : 0.f;

  // ---- all loads of the item, issued together: log alpha of the lane's
  // token, its key and query rows, beta
  const TIn *larow = x.la + x.tok(tr) * x.la_row + (size_t)x.hk * G;
  constexpr bool kVecLa = kGate != kGateGroupsFew;      // G >= 8: log alpha read as 8-element vectors
  Raw8<TIn> lav[kVecLa ? KS : 1];
  TIn las[4];
  if constexpr (kVecLa) {
#pragma unroll
    for (int s = 0; s < KS; ++s) lav[s].load(larow + min((32 * s + 8 * lq) >> gs, G - 8));
  } else {
#pragma unroll
    for (int g = 0; g < 4; ++g) las[g] = larow[min(g, G - 1)];
  }
  Raw8<TIn> kt[KS], qt[KS];
  x.load_rows(kt, x.kbase, I);
  x.load_rows(qt, x.qbase, I);
  TIn bets[NBET];
  x.load_betas(bets);


  // ---- Lambda of the lane's token in log2 units (log2(e) Lambda): in-block
  // prefix, then block offsets
  constexpr float kLog2e = 1.4426950408889634f;
  const float scale = mt * kLog2e;                     // tokens past T: zero log decay
  float lt[KS][8];
  bool rising = false;                                 // a positive log alpha: Lambda not monotone
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    const int ch0 = 32 * s + 8 * lq;
    if constexpr (kGate == kGatePerChannel) {
      float f[8];
      lav[s].to_float(f);
#pragma unroll
      for (int e = 0; e < 8; ++e) lt[s][e] = f[e] * scale;
    } else if constexpr (kGate == kGateGroupsVec) {
      float f[8];
      lav[s].to_float(f);
      const int g0 = min(ch0 >> gs, G - 8);
      if (gs >= 3) {                                     // one group for the lane's eight channels
        const float v = pick(f, (ch0 >> gs) - g0) * scale;
#pragma unroll
        for (int e = 0; e < 8; ++e) lt[s][e] = v;
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) lt[s][e] = pick(f, ((ch0 + e) >> gs) - g0) * scale;
      }
    } else {
      // G < 8 < d_k / G: the lane's eight channels share one group
      const int g = ch0 >> gs;
      const float v = static_cast<float>(g == 0 ? las[0] : g == 1 ? las[1] : g == 2 ? las[2] : las[3]) * scale;
#pragma unroll
      for (int e = 0; e < 8; ++e) lt[s][e] = v;
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) rising |= lt[s][e] > 0.f;
  }
  // Block totals of log alpha -> LDS; then one thread per channel turns them
  // into exclusive block offsets and the per-channel factors
  // e0 = exp(Lambda_0), e0i = exp(-Lambda_0), gc = exp(Lambda_{C-1}).
  float *off = x.smem;                                 // [NB][DK] block totals, then block offsets
  float *row0 = off + NB * DK;                         // [DK] log2(e) Lambda_0, then e0
  float *e0i = row0 + DK;                              // [DK]
  float *gc = e0i + DK;                                // [DK]
  if (I == 0 && lr == 0) {
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      float *d = row0 + 32 * s + 8 * lq;
      *reinterpret_cast<float4 *>(d) = make_float4(lt[s][0], lt[s][1], lt[s][2], lt[s][3]);
      *reinterpret_cast<float4 *>(d + 4) = make_float4(lt[s][4], lt[s][5], lt[s][6], lt[s][7]);
    }
  }
#pragma unroll
  for (int s = 0; s < KS; ++s) {
#pragma unroll
    for (int e = 0; e < 8; ++e) lt[s][e] = row_prefix16(lt[s][e]);
  }
  if (lr == 15) {
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      float *d = off + I * DK + 32 * s + 8 * lq;
      *reinterpret_cast<float4 *>(d) = make_float4(lt[s][0], lt[s][1], lt[s][2], lt[s][3]);
      *reinterpret_cast<float4 *>(d + 4) = make_float4(lt[s][4], lt[s][5], lt[s][6], lt[s][7]);
    }
  }
  // flags[kChunkWide]: a positive log alpha (Lambda not monotone) or a total
  // decay -Lambda_{C-1} beyond kPivotRange.  Without either, every Lambda_t
  // lies in [-kPivotRange, 0] and all the factors below lie in
  // [exp(-kPivotRange), exp(kPivotRange)].
  if (x.tid == 0) x.flags[kChunkWide] = 0;
  const bool any_rising = __ballot(rising) != 0;
  __syncthreads();
  x.put_betas(bets, 0);                               // the solve's first beta head, read after later barriers
  if (lr == 0 && lq == 0 && any_rising) x.flags[kChunkWide] = 1;
  if (x.tid < DK) {
    const int ch = x.tid;
    float run = 0.f;
#pragma unroll
    for (int J = 0; J < NB; ++J) {
      const float t = off[J * DK + ch];
      off[J * DK + ch] = run;
      run += t;
    }
    if (!(-run <= kPivotRange * kLog2e)) x.flags[kChunkWide] = 1;   // several threads may store the same 1
    const float l0 = row0[ch];
    row0[ch] = __builtin_amdgcn_exp2f(l0);
    e0i[ch] = __builtin_amdgcn_exp2f(-l0);
    gc[ch] = __builtin_amdgcn_exp2f(run);
  }
  __syncthreads();
  const bool wide = __builtin_amdgcn_readfirstlane(x.flags[kChunkWide]) != 0;
  if (wide) {
    if (x.tid == 0) x.gm_row()[0] = kWideMark;         // left to the block-pivot kernel
    return;
  }
  if (x.tid < DK) x.gm_row()[x.tid] = gc[x.tid];
  auto load8 = [&](const float *p, float (&y)[8]) __attribute__((always_inline)) {
    const float4 u = *reinterpret_cast<const float4 *>(p);
    const float4 v = *reinterpret_cast<const float4 *>(p + 4);
    y[0] = u.x; y[1] = u.y; y[2] = u.z; y[3] = u.w; y[4] = v.x; y[5] = v.y; y[6] = v.z; y[7] = v.w;
  };
  // ---- row and column operands, scan operands, the diagonal pair
  unsigned char *colop = reinterpret_cast<unsigned char *>(x.ureg);
  Split ak[KS], aq[KS];
  f32x4 dG = {0.f, 0.f, 0.f, 0.f}, dL = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    const int ch0 = 32 * s + 8 * lq;
    float xk[8], xq[8], f0[8], f0i[8], fc[8], o[8];
    kt[s].to_float(xk);
    qt[s].to_float(xq);
    load8(row0 + ch0, f0);
    load8(e0i + ch0, f0i);
    load8(gc + ch0, fc);
    load8(off + I * DK + ch0, o);
    float yk[8], yq[8], yb[8], kbar[8], qbar[8], kh[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float l2 = lt[s][e] + o[e];                // log2(e) Lambda_t
      const float d = __builtin_amdgcn_exp2f(l2);      // exp(Lambda_t)
      const float ui = __builtin_amdgcn_exp2f(-l2);    // exp(-Lambda_t)
      const float k = xk[e] * mt, q = xq[e] * mt;       // tokens past T: zero rows
      yk[e] = k * (d * f0i[e]);                        // row side, exp(Lambda_t - Lambda_0)
      yq[e] = q * (d * f0i[e]);
      yb[e] = k * (ui * f0[e]);                        // column side, exp(Lambda_0 - Lambda_t)
      kbar[e] = k * d;
      qbar[e] = q * d;
      kh[e] = k * (ui * fc[e]);                        // exp(Lambda_C - Lambda_t)
    }
    ak[s] = make_frag<Split>(yk);
    aq[s] = make_frag<Split>(yq);
    const Split bk = make_frag<Split>(yb);
    mma(dG, ak[s], bk);
    mma(dL, aq[s], bk);
    if (I < NB - 1) lds_put_frag(colop, I * KS + s, bk);
    x.scan_operands(I, s, kbar, qbar, kh);
  }
  x.store_L_block(I, I, dL);
  __syncthreads();                                     // column operands complete, Lambda rows dead
  float *gsolve = x.smem;
#pragma unroll
  for (int q4 = 0; q4 < 4; ++q4) {
    const int row = 16 * I + 4 * lq + q4, col = 16 * I + lr;
    gsolve[row * (C + 4) + col] = row > col ? dG[q4] : 0.f;
  }
  for (int J = 0; J < I; ++J) {
    f32x4 accG = {0.f, 0.f, 0.f, 0.f}, accL = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const Split bj = lds_get_frag<Split>(colop, J * KS + s);
      mma(accG, ak[s], bj);
      mma(accL, aq[s], bj);
    }
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) gsolve[(16 * I + 4 * lq + q4) * (C + 4) + 16 * J + lr] = accG[q4];
    x.store_L_block(I, J, accL);
  }
  x.zero_upper_L();
  x.solve_store(gsolve, x.ureg, bets, true);
}

// Block-pivot route for one chunk: p = first token of the row block; every
// exponent on the causal side is <= 0, except on a diagonal block, where it
// is at most the block's decay range (<= kPivotRange unless the block is
// flagged and evaluated entry by entry).  Wave w owns blocks w (and 7 - w
// when C = 128).
template <typename TIn, class P, int C, int DK>
__device__ __forceinline__ void prep_block_item(const ChunkArgs &a, int c, int hk, int b, float *smem) {
  using X = PrepItem<TIn, P, C, DK>;
  using Split = typename X::Split;
  constexpr int NB = X::NB, KS = X::KS;
  constexpr int NR = NB / 4;                           // row blocks per wave
  X x(a, c, hk, b, smem, prep_region0_floats(C, a.G));
  const int w = x.w, lr = x.lr, lq = x.lq, T = x.T, t0 = x.t0;
  auto own = [&](int r) { return (r & 1) ? 4 * r + 3 - w : 4 * r + w; };
  typename X::LaRegs lar;
  x.issue_la(lar);
  Raw8<TIn> kt[KS], qt[KS], kj[KS];
  x.load_rows(kt, x.kbase, own(0));
  x.load_rows(qt, x.qbase, own(0));
  x.load_rows(kj, x.kbase, 0);
  x.lambda(lar);
  x.write_gm();
  float *gmat = x.ureg;
  for (int r = 0; r < NR; ++r) {
    const int I = own(r);
    const int tr = 16 * I + lr, piv = 16 * I;
    const float mt = (t0 + tr < T) ? 1.f : 0.f;
    Split ak[KS], aq[KS];
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const int ch0 = 32 * s + 8 * lq;
      float xk[8], xq[8], lt[8], lp[8], lc[8];
      kt[s].to_float(xk);
      qt[s].to_float(xq);
      x.lam8(tr, ch0, lt);
      x.lam8(piv, ch0, lp);
      x.lam8(C - 1, ch0, lc);
      float yk[8], yq[8], kbar[8], qbar[8], kh[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float ea = __expf(lt[e] - lp[e]) * mt;
        const float d = __expf(lt[e]) * mt;
        const float h = __expf(lc[e] - lt[e]) * mt;
        yk[e] = xk[e] * ea;
        yq[e] = xq[e] * ea;
        kbar[e] = xk[e] * d;
        qbar[e] = xq[e] * d;
        kh[e] = xk[e] * h;
      }
      ak[s] = make_frag<Split>(yk);
      aq[s] = make_frag<Split>(yq);
      x.scan_operands(I, s, kbar, qbar, kh);
    }
    if (r + 1 < NR) {                                  // next owned block's rows
      x.load_rows(kt, x.kbase, own(r + 1));
      x.load_rows(qt, x.qbase, own(r + 1));
    }
    for (int J = 0; J <= I; ++J) {
      Raw8<TIn> ckj[KS];
#pragma unroll
      for (int s = 0; s < KS; ++s) ckj[s] = kj[s];
      x.load_rows(kj, x.kbase, J < I ? J + 1 : 0);     // next pair's key rows (first block of the next round)
      f32x4 accG = {0.f, 0.f, 0.f, 0.f}, accL = {0.f, 0.f, 0.f, 0.f};
      const int jr = 16 * J + lr;
      const float mj = (t0 + jr < T) ? 1.f : 0.f;
      if (!(I == J && x.flags[I])) {
#pragma unroll
        for (int s = 0; s < KS; ++s) {
          const int ch0 = 32 * s + 8 * lq;
          float xj[8], lp[8], lj[8];
          ckj[s].to_float(xj);
          x.lam8(piv, ch0, lp);
          x.lam8(jr, ch0, lj);
#pragma unroll
          for (int e = 0; e < 8; ++e) xj[e] *= __expf(lp[e] - lj[e]) * mj;
          const Split fj = make_frag<Split>(xj);
          mma(accG, ak[s], fj);
          mma(accL, aq[s], fj);
        }
      } else {
        // Diagonal block whose decay range is too wide for one pivot: each
        // entry by its definition, causal mask before the exponential.
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const int row = 16 * I + 4 * lq + q4, col = 16 * J + lr;
          float sg = 0.f, sl = 0.f;
          if (row >= col && t0 + row < T) {
            const size_t rrow = x.tok(row) * x.row_stride, rcol = x.tok(col) * x.row_stride;
            for (int ch = 0; ch < DK; ++ch) {
              const int g = ch >> x.gs;
              const float d = __expf(x.lam[row * x.G + g] - x.lam[col * x.G + g]);
              const float kc = static_cast<float>(x.kbase[rcol + ch]);
              sg += static_cast<float>(x.kbase[rrow + ch]) * kc * d;
              sl += static_cast<float>(x.qbase[rrow + ch]) * kc * d;
            }
          }
          accG[q4] = sg;
          accL[q4] = sl;
        }
      }
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int row = 16 * I + 4 * lq + q4, col = 16 * J + lr;
        gmat[row * (C + 4) + col] = (I > J || row > col) ? accG[q4] : 0.f;
      }
      x.store_L_block(I, J, accL);
    }
  }
  x.zero_upper_L();
  TIn bets[X::NBET];                                   // beta loaded here: short-lived registers
  x.load_betas(bets);
  x.solve_store(gmat, x.smem, bets, false);
}

// Grid (N_c, H_k, B), one chunk per work group.
template <typename TIn, class P, int C, int DK>
__global__ __launch_bounds__(256) void prep_block_kernel(ChunkArgs a) {
  extern __shared__ __align__(16) unsigned char smem_raw[];
  prep_block_item<TIn, P, C, DK>(a, blockIdx.x, blockIdx.y, blockIdx.z, reinterpret_cast<float *>(smem_raw));
}

// 1-D grid: work group g checks the items g + j * gridDim.x (j < 256) for the
// chunk-pivot kernel's mark and runs the marked ones in turn.
template <typename TIn, class P, int C, int DK>
__global__ __launch_bounds__(256) void prep_block_listed_kernel(ChunkArgs a) {
  extern __shared__ __align__(16) unsigned char smem_raw[];
  float *smem = reinterpret_cast<float *>(smem_raw);
  const int n = a.N_c * a.H_k * a.B, tid = threadIdx.x;
  bool mine = false;
  {
    const int u = blockIdx.x + tid * gridDim.x;
    if (u < n) {
      const int c = u % a.N_c, hk = (u / a.N_c) % a.H_k, b = u / (a.N_c * a.H_k);
      mine = reinterpret_cast<const float *>(ws_tile(a, kWsGM, a.H_k, hk, b, c))[0] == kWideMark;
    }
  }
  // the 256 marks as four 64-bit wave masks, shared through LDS
  unsigned long long *masks = reinterpret_cast<unsigned long long *>(smem);
  const unsigned long long m = __ballot(mine);
  if (lane_id() == 0) masks[wave_id()] = m;
  __syncthreads();
  unsigned long long mk[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const unsigned long long v = masks[q];
    mk[q] = ((unsigned long long)__builtin_amdgcn_readfirstlane((unsigned)(v >> 32)) << 32) |
            (unsigned)__builtin_amdgcn_readfirstlane((unsigned)v);
  }
  __syncthreads();
  for (int q = 0; q < 4; ++q) {
    unsigned long long v = mk[q];
    while (v) {
      const int j = 64 * q + __builtin_ctzll(v);
      v &= v - 1;
      const int u = blockIdx.x + j * gridDim.x;
      const int c = u % a.N_c, hk = (u / a.N_c) % a.H_k, b = u / (a.N_c * a.H_k);
      prep_block_item<TIn, P, C, DK>(a, c, hk, b, smem);
      __syncthreads();
    }
  }
}

bool prep_supported(int C, int d_k, int G) {
  if (!(C == 64 || C == 128)) return false;
  if (!(d_k == 64 || d_k == 128 || d_k == 256)) return false;
  return prep_lds_bytes(C, d_k, G) <= 160 * 1024;
}

template <class K>
static hipError_t set_lds(K kern, size_t lds) {
  return hipFuncSetAttribute(reinterpret_cast<const void *>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                             (int)lds);
}

template <typename TIn, class P, int C, int DK>
static hipError_t launch_prep_t(const ChunkArgs &a, hipStream_t stream) {
  const size_t lds = prep_lds_bytes(C, DK, a.G);
  const dim3 grid(a.N_c, a.H_k, a.B);
  hipError_t e;
  if constexpr (C != 64) {
    auto block = prep_block_kernel<TIn, P, C, DK>;
    if ((e = set_lds(block, lds)) != hipSuccess) return e;
    hipLaunchKernelGGL(block, grid, dim3(256), lds, stream, a);
    return hipGetLastError();
  } else {
  auto chunk = a.G == DK  ? prep_chunk_kernel<TIn, P, DK, kGatePerChannel>
               : a.G >= 8 ? prep_chunk_kernel<TIn, P, DK, kGateGroupsVec>
                          : prep_chunk_kernel<TIn, P, DK, kGateGroupsFew>;
  auto listed = prep_block_listed_kernel<TIn, P, C, DK>;
  const size_t chunk_lds = prep_chunk_lds_bytes(C, DK);
  if ((e = set_lds(chunk, chunk_lds)) != hipSuccess) return e;
  if ((e = set_lds(listed, lds)) != hipSuccess) return e;
  hipLaunchKernelGGL(chunk, grid, dim3(256), chunk_lds, stream, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  // wide-range chunks, if any: two work groups per CU (the LDS of the block
  // route allows two), at most 256 items each
  const long n = (long)a.N_c * a.H_k * a.B;
  const long groups = std::max(std::min(n, 512L), (n + 255) / 256);
  hipLaunchKernelGGL(listed, dim3((unsigned)groups), dim3(256), lds, stream, a);
  return hipGetLastError();
  }
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
