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

#ifndef GDR_PREP_UNIT
#define GDR_PREP_UNIT 0
#endif

namespace gdr {

constexpr float kPivotRange = 64.f;  // exp(64) ~ 6e27 keeps every partial sum finite

// LDS rows of the C x C matrices are padded to C + 4 floats, so the 16 rows a
// column-strided fragment read touches fall into different banks.
__host__ __device__ inline int prep_ld(int C) { return C + 4; }
__host__ __device__ inline int prep_region0_floats(int C, int G) {
  return (C * G > C * prep_ld(C)) ? C * G : C * prep_ld(C);
}
__host__ __device__ constexpr int prep_tmp_floats(int C) {
  // block merges of the exact solve; one 16-column block of the Neumann
  // solve; four waves' 16 x 16 staging tiles of the block-Jacobi solve
  const int merge = C * (C / 2 + 4) / 2, neumann = C * 20 > 4 * 16 * 20 ? C * 20 : 4 * 16 * 20;
  return merge > neumann ? merge : neumann;
}

constexpr int kXbLd = 20;   // row stride (floats) of the per-wave transpose buffers
constexpr int kChunkWide = 8;  // flags slot: the chunk's decay range exceeds kPivotRange
constexpr int kHasReset = 9;   // flags slot: a document starts inside the chunk

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

// The block-pivot kernel of C = 32 and 128 runs eight waves; their transpose
// buffers take the solve's scratch (idle while the operands and pairs are
// built) instead of a region of their own.
__host__ __device__ inline int prep_union8_floats(int C, int DK) {
  const int scratch = prep_tmp_floats(C) > 8 * 32 * kXbLd ? prep_tmp_floats(C) : 8 * 32 * kXbLd;
  const int solve = C * prep_ld(C) + scratch, colop = prep_colop_floats(C, DK);
  return solve > colop ? solve : colop;
}
inline size_t prep_block8_lds_bytes(int C, int DK, int G) {
  return sizeof(float) * (size_t)(prep_region0_floats(C, G) + prep_union8_floats(C, DK) + C) + sizeof(int) * 16 + C;
}

// The block-pivot route also keeps each token's document segment (C bytes,
// after the transpose buffers).
#if !GDR_PREP_UNIT
size_t prep_lds_bytes(int C, int DK, int G) {
  return sizeof(float) * (size_t)(prep_region0_floats(C, G) + prep_union_floats(C, DK) + C) +
         sizeof(int) * 16 + sizeof(float) * 4 * 32 * kXbLd + C;
}
#endif
// The chunk-pivot kernel keeps Lambda in registers: region 0 holds the
// block totals of Lambda during the build and G after it.
__host__ __device__ inline int prep_chunk_region0_floats(int C) { return C * prep_ld(C); }
inline size_t prep_chunk_lds_bytes(int C, int DK) {
  return sizeof(float) * (size_t)(prep_chunk_region0_floats(C) + prep_union_floats(C, DK) + C) +
         sizeof(int) * 16 + sizeof(float) * 4 * 32 * kXbLd + C;
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

// ------------------------------------------------------------- exact solve
// amat <- (I + M)^{-1}, M = gmat diag(bet): 16x16 diagonal blocks by forward
// substitution (one lane per column), then block-doubling merges
// A[B,T] = -A[B,B] (M[B,T] A[T,T]) with fp32 MFMA.  Only the diagonal and
// lower 16x16 blocks of amat are written (and read): the blocks above the
// diagonal are zero by construction and left to the caller.
// The 16 x 16 diagonal blocks of (I + M)^{-1}, M = gmat diag(bet), by
// forward substitution: one thread per (block, column).
template <int C, bool kScaled = false>
__device__ __forceinline__ void invert_diag_blocks(const float *gmat, const float *bet, float *amat) {
  constexpr int NB = C / 16;
  constexpr int LD = C + 4;
  const int tid = threadIdx.x;
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
      amat[(base + i) * LD + base + cc] = kScaled ? bl[i] * s : s;
    }
  }
}

// kScaled: amat holds diag(beta) A throughout.  With Ahat = diag(beta) A the
// merge is Ahat[B,T] = -Ahat[B,B] (G[B,T] Ahat[T,T]) (it is diag(beta_B)
// A[B,B] M[B,T] A[T,T] with M = G diag(beta)), free of beta.
template <int C, bool kTiles = false, bool kScaled = false>
__device__ __forceinline__ void solve_exact(const float *gmat, const float *bet, float *amat, float *tmp) {
  constexpr int LD = C + 4;
  const int w = wave_id(), l = lane_id();
  auto mx = [&](int r, int k) __attribute__((always_inline)) { return kScaled ? gmat[r * LD + k] : gmat[r * LD + k] * bet[k]; };
  invert_diag_blocks<C, kScaled>(gmat, bet, amat);
  __syncthreads();
  if constexpr (kTiles) {
    // Eight waves: one job per 16 x 16 tile, the two products of a level
    // separated by a barrier.  In the second half of a level's tiles the
    // column (X) or row (A) index is mirrored, so a wave's two tiles have
    // contractions of complementary length.
    const int nw = blockDim.x / kWave;
    for (int bs = 16; bs < C; bs *= 2) {
      const int tpb = bs / 16, XLD = bs + 4;
      const int per = tpb * tpb, jobs = (C / (2 * bs)) * per;
      for (int job = w; job < jobs; job += nw) {
        const int p = job / per, u = job % per, ti = u / tpb;
        const int tj = ti >= (tpb + 1) / 2 ? tpb - 1 - u % tpb : u % tpb;
        const int top = 2 * bs * p, bot = top + bs, c0 = top + 16 * tj, r0 = bot + 16 * ti;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        tile_f32<C / 32>(acc,
                 [&](int i, int k) { return mx(r0 + i, k); },
                 [&](int k, int j) { return amat[k * LD + c0 + j]; },
                 c0, top + bs);               // A[top,top] is lower: rows k >= column
        float *X = tmp + p * bs * XLD;
#pragma unroll
        for (int r = 0; r < 4; ++r) X[(16 * ti + 4 * (l >> 4) + r) * XLD + 16 * tj + (l & 15)] = acc[r];
      }
      __syncthreads();
      for (int job = w; job < jobs; job += nw) {
        const int p = job / per, u = job % per, tj = u / tpb;
        const int ti = tj >= (tpb + 1) / 2 ? tpb - 1 - u % tpb : u % tpb;
        const int top = 2 * bs * p, bot = top + bs, r0 = bot + 16 * ti;
        const float *X = tmp + p * bs * XLD;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        tile_f32<C / 32>(acc,
                 [&](int i, int k) { return amat[(r0 + i) * LD + k]; },
                 [&](int k, int j) { return X[(k - bot) * XLD + 16 * tj + j]; },
                 bot, r0 + 16);               // A[bot,bot] is lower: columns k <= row
#pragma unroll
        for (int r = 0; r < 4; ++r)
          amat[(r0 + 4 * (l >> 4) + r) * LD + top + 16 * tj + (l & 15)] = -acc[r];
      }
      __syncthreads();
    }
    return;
  }
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
                 [&](int i, int k) { return mx(r0 + i, k); },
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

// ----------------------------------------------- block-Jacobi Neumann solve
// Systolic Linear Attention, section 2.4.3, "Block-doubling and block-Neumann
// factorization": with D the block diagonal of I + M (16-row blocks) and
// N = D^{-1} (I + M - D), X = sum_{s=0}^{m} (-N)^s D^{-1}; m = 1 is the
// pages' 1-Step Neumann A_N1 = (I - N) D^{-1}.  By Horner from X = D^{-1},
// m times X <- D^{-1} - D^{-1} O X (O = I + M - D: the blocks of M below the
// diagonal).  Block (I, J), I > J, of the update is -D_I^{-1} (O X)_IJ and
// reads column block J of X at block rows J .. I-1 only, so a wave updates
// its column block in place from the bottom up; the product (O X)_IJ goes
// through the wave's own 16 x 16 staging tile before D_I^{-1} multiplies it.
template <int C>
__device__ __forceinline__ void solve_block_neumann(const float *gmat, const float *bet, float *amat, float *tmp,
                                                    int order) {
  constexpr int NB = C / 16;
  constexpr int LD = C + 4;
  constexpr int SLD = 20;
  const int tid = threadIdx.x, w = wave_id(), l = lane_id();
  const int nw = blockDim.x / kWave;
  invert_diag_blocks<C>(gmat, bet, amat);
  float *st = tmp + w * 16 * SLD;
  if (order == 1) {
    // One step from X = D^{-1}: X[I,J] = -D_I^{-1} (M[I,J] D_J^{-1}) for
    // I > J, every block independent of the others, so the blocks are
    // shared out over the waves (the step below would contract over the
    // whole column, whose blocks other than J are still zero).
    __syncthreads();
    for (int job = w; job < NB * (NB - 1) / 2; job += nw) {
      int I = 1, J = job;                              // job = I (I - 1) / 2 + J, J < I
      while (J >= I) {
        J -= I;
        ++I;
      }
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      tile_f32_n<1>(acc, [&](int i, int k) { return gmat[(16 * I + i) * LD + k] * bet[k]; },
                    [&](int k, int j) { return amat[k * LD + 16 * J + j]; }, 16 * J);
#pragma unroll
      for (int r = 0; r < 4; ++r) st[(4 * (l >> 4) + r) * SLD + (l & 15)] = acc[r];
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      f32x4 acc2 = {0.f, 0.f, 0.f, 0.f};
      tile_f32_n<1>(acc2, [&](int i, int k) { return amat[(16 * I + i) * LD + 16 * I + k]; },
                    [&](int k, int j) { return st[k * SLD + j]; }, 0);
#pragma unroll
      for (int r = 0; r < 4; ++r) amat[(16 * I + 4 * (l >> 4) + r) * LD + 16 * J + (l & 15)] = -acc2[r];
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");   // the staging tile's reads before its next writes
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
    __syncthreads();
    return;
  }
  for (int i = tid; i < C * C; i += blockDim.x) {
    const int r = i / C, cc = i % C;
    if (r / 16 > cc / 16) amat[r * LD + cc] = 0.f;    // X = D^{-1}
  }
  __syncthreads();
  for (int it = 0; it < order; ++it) {
    for (int J = w; J < NB - 1; J += nw) {
      for (int I = NB - 1; I > J; --I) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        tile_f32<NB>(acc, [&](int i, int k) { return gmat[(16 * I + i) * LD + k] * bet[k]; },
                     [&](int k, int j) { return amat[k * LD + 16 * J + j]; }, 16 * J, 16 * I);
#pragma unroll
        for (int r = 0; r < 4; ++r) st[(4 * (l >> 4) + r) * SLD + (l & 15)] = acc[r];
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        f32x4 acc2 = {0.f, 0.f, 0.f, 0.f};
        tile_f32_n<1>(acc2, [&](int i, int k) { return amat[(16 * I + i) * LD + 16 * I + k]; },
                      [&](int k, int j) { return st[k * SLD + j]; }, 0);
#pragma unroll
        for (int r = 0; r < 4; ++r) amat[(16 * I + 4 * (l >> 4) + r) * LD + 16 * J + (l & 15)] = -acc2[r];
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");   // the staging tile's reads before its next writes
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      }
    }
    __syncthreads();
  }
}

// ----------------------------------------------------------- Neumann solve
// X = sum_{s=0}^{m} (-M)^s by Horner (X <- I - M X, m times from X = I; the
// first step needs no product: X = I - M), then r residual corrections
// X <- X + X R with R = I - (I + M) X.
//
// Products of lower-triangular C x C matrices go by 16 x 16 tiles (I, J),
// I >= J; tile (I, J) contracts over k in [16 J, 16 I + 16).  The tiles of
// one product are independent, so they are dealt to all waves (longest
// contraction first, dealt back and forth), each wave keeps its results in
// registers, and all waves write them after a barrier: two barriers per
// Horner step.  A residual correction needs R whole as the right operand of
// X R; the solve's scratch holds g 16-column blocks of it (g from the scratch
// size), so the correction goes by groups of g column blocks: R[:, group]
// into the scratch, barrier, (X R)[:, group] into registers, barrier, then
// added to X while the next group's R is formed (that reads only columns of
// X right of the group).  F: the MFMA operand kind -- split bf16 for bf16
// inputs (about 16 significant bits per operand, three bf16 MFMAs per
// 32-deep step), fp32 for fp32 inputs.

// Tile (I, J) of a lower-triangular product, contraction k in [16 J, 16 I + 16)
// in 32-deep steps (the second half of an odd last step is masked).
// yrow(r, k, y): y[e] = Y[r][k + e], e < 8; zcol(k, c) = Z[k][c].
template <class F, class FY, class FZ>
__device__ __forceinline__ f32x4 lower_tile(const FY &yrow, const FZ &zcol, int I, int J) {
  const int l = lane_id(), lr = l & 15, lq = l >> 4;
  const int kend = 16 * I + 16;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 1
  for (int k0 = 16 * J; k0 < kend; k0 += 32) {
    const int kk = k0 + 8 * lq;
    const bool ok = kk < kend;
    const int ks = ok ? kk : kk - 16;                  // a valid row, read and zeroed
    float y[8], z[8];
    yrow(16 * I + lr, ks, y);
#pragma unroll
    for (int e = 0; e < 8; ++e) z[e] = zcol(ks + e, 16 * J + lr);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      y[e] = ok ? y[e] : 0.f;
      z[e] = ok ? z[e] : 0.f;
    }
    mma(acc, make_frag<F>(y), make_frag<F>(z));
  }
  return acc;
}

// Tile `p` of the lower-triangular tiles of an NB x NB block matrix ordered
// by decreasing contraction (I - J descending, then J ascending).
__device__ __forceinline__ void lower_tile_at(int NB, int p, int &I, int &J) {
  int d = NB - 1;
  while (p >= NB - d) {
    p -= NB - d;
    --d;
  }
  J = p;
  I = p + d;
}

// Column blocks of R the scratch holds at a time.
template <int C, int NTH>
constexpr int neumann_res_cols() {
  constexpr int scratch = NTH == 512 ? (prep_tmp_floats(C) > 8 * 32 * kXbLd ? prep_tmp_floats(C) : 8 * 32 * kXbLd)
                                     : prep_tmp_floats(C);
  int g = C / 16;
  while (g > 1 && C * (16 * g + 4) > scratch) --g;
  return g;
}

template <int C, int NTH, class F>
__device__ __forceinline__ void solve_neumann(const float *gmat, const float *bet, float *amat, float *tmp, int order,
                                              int residual) {
  constexpr int NB = C / 16;
  constexpr int LD = C + 4;
  constexpr int NW = NTH / kWave;
  constexpr int NT = NB * (NB + 1) / 2;                // lower-triangular tiles
  constexpr int SL = (NT + NW - 1) / NW;               // tiles per wave (at most)
  constexpr int GR = neumann_res_cols<C, NTH>();       // column blocks per residual group
  constexpr int TLD = 16 * GR + 4;
  constexpr int SR = (GR * NB + NW - 1) / NW;
  static_assert(C * TLD <= (NTH == 512 ? (prep_tmp_floats(C) > 8 * 32 * kXbLd ? prep_tmp_floats(C) : 8 * 32 * kXbLd)
                                       : prep_tmp_floats(C)),
                "one column block of R fits the scratch");
  const int tid = threadIdx.x, w = wave_id(), l = lane_id(), lr = l & 15, lq = l >> 4;
  // M = G diag(beta), strictly lower (G's diagonal blocks hold zeros on and above the diagonal)
  auto mrow = [&](int r, int k, float (&y)[8]) __attribute__((always_inline)) {
    const float4 g0 = *reinterpret_cast<const float4 *>(gmat + r * LD + k);
    const float4 g1 = *reinterpret_cast<const float4 *>(gmat + r * LD + k + 4);
    const float4 b0 = *reinterpret_cast<const float4 *>(bet + k);
    const float4 b1 = *reinterpret_cast<const float4 *>(bet + k + 4);
    y[0] = g0.x * b0.x; y[1] = g0.y * b0.y; y[2] = g0.z * b0.z; y[3] = g0.w * b0.w;
    y[4] = g1.x * b1.x; y[5] = g1.y * b1.y; y[6] = g1.z * b1.z; y[7] = g1.w * b1.w;
  };
  auto xrow = [&](int r, int k, float (&y)[8]) __attribute__((always_inline)) {
    const float4 a0 = *reinterpret_cast<const float4 *>(amat + r * LD + k);
    const float4 a1 = *reinterpret_cast<const float4 *>(amat + r * LD + k + 4);
    y[0] = a0.x; y[1] = a0.y; y[2] = a0.z; y[3] = a0.w; y[4] = a1.x; y[5] = a1.y; y[6] = a1.z; y[7] = a1.w;
  };
  auto xcol = [&](int k, int c) __attribute__((always_inline)) { return amat[k * LD + c]; };
  // tile s of this wave: position s NW + w (s even) or s NW + NW - 1 - w (s odd)
  auto my_tile = [&](int s, int &I, int &J) __attribute__((always_inline)) {
    const int p = s * NW + ((s & 1) ? NW - 1 - w : w);
    if (p >= NT) return false;
    lower_tile_at(NB, p, I, J);
    return true;
  };

  // X = I (m = 0) or I - M
  for (int i = tid; i < C * LD; i += NTH) {
    const int r = i / LD, cc = i % LD;
    float x = (r == cc) ? 1.f : 0.f;
    if (order > 0 && cc < r) x -= gmat[i] * bet[cc];
    amat[i] = x;
  }
  __syncthreads();
  for (int it = 1; it < order; ++it) {
    f32x4 acc[SL];
#pragma unroll
    for (int s = 0; s < SL; ++s) {
      int I, J;
      if (my_tile(s, I, J)) acc[s] = lower_tile<F>(mrow, xcol, I, J);
    }
    __syncthreads();
#pragma unroll
    for (int s = 0; s < SL; ++s) {
      int I, J;
      if (!my_tile(s, I, J)) continue;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = 16 * I + 4 * lq + r, col = 16 * J + lr;
        amat[row * LD + col] = ((row == col) ? 1.f : 0.f) - acc[s][r];
      }
    }
    __syncthreads();
  }
  // residual: tile t of a group starting at column block J0 (rows from the
  // bottom, the group's columns left to right)
  auto res_tile = [&](int J0, int t, int &I, int &J) __attribute__((always_inline)) {
    const int g = min(GR, NB - J0);
    I = NB - 1;
    while (true) {
      const int n = min(g, I - J0 + 1);                // columns of the group at row block I
      if (t < n) break;
      t -= n;
      if (--I < J0) return false;
    }
    J = J0 + t;
    return true;
  };
  for (int it = 0; it < residual; ++it) {
    f32x4 acc[SR];
    int J0p = -1;
    for (int J0 = 0; J0 < NB; J0 += GR) {
      // R[:, group] = I - X - M X  (the scratch holds rows 0 .. C - 1 of the group's columns)
#pragma unroll
      for (int s = 0; s < SR; ++s) {
        int I, J;
        if (!res_tile(J0, s * NW + w, I, J)) continue;
        const f32x4 mx = lower_tile<F>(mrow, xcol, I, J);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = 16 * I + 4 * lq + r, col = 16 * J + lr;
          tmp[row * TLD + col - 16 * J0] = ((row == col) ? 1.f : 0.f) - amat[row * LD + col] - mx[r];
        }
      }
      // the previous group's X R, added now: its columns are left of this group
      if (J0p >= 0) {
#pragma unroll
        for (int s = 0; s < SR; ++s) {
          int I, J;
          if (!res_tile(J0p, s * NW + w, I, J)) continue;
#pragma unroll
          for (int r = 0; r < 4; ++r) amat[(16 * I + 4 * lq + r) * LD + 16 * J + lr] += acc[s][r];
        }
      }
      __syncthreads();
#pragma unroll
      for (int s = 0; s < SR; ++s) {
        int I, J;
        if (!res_tile(J0, s * NW + w, I, J)) continue;
        acc[s] = lower_tile<F>(xrow, [&](int k, int c) { return tmp[k * TLD + c - 16 * J0]; }, I, J);
      }
      __syncthreads();
      J0p = J0;
    }
#pragma unroll
    for (int s = 0; s < SR; ++s) {
      int I, J;
      if (!res_tile(J0p, s * NW + w, I, J)) continue;
#pragma unroll
      for (int r = 0; r < 4; ++r) amat[(16 * I + 4 * lq + r) * LD + 16 * J + lr] += acc[s][r];
    }
    __syncthreads();
  }
}

// ------------------------------------- Neumann solve on split-bf16 planes
// The same series and corrections for bf16 inputs with one beta head per
// key head (G is then not needed after the solve), in the transposed
// unknown Y = X^T: a Horner step is Y <- I - Y M^T, a residual correction
// R^T = I - Y - Y M^T, Y <- Y + R^T Y.  Y, M = G diag(beta) and the
// correction's R^T rows are kept in LDS as two bf16 planes (hi = bf16(x),
// lo = bf16(x - hi)), so an MFMA operand is two 16-byte reads with no
// conversion: every product is split-bf16 (three MFMAs per 32-deep step).
// Y M^T reads rows of both Y and M; only R^T Y reads Y down its columns.
// The MFMA takes M (or Y) as its row operand, so a lane's accumulator holds
// four consecutive columns of one row of the result, written as 8-byte
// pieces.  Both Y and R^T are upper triangular, M is strictly lower: their
// zero triangles are stored, so a contraction of an odd number of 16-blocks
// is padded with a zero block instead of masked.  M overwrites G.
//
// Plane layout: rows of C bf16 values, hi plane then lo plane; the 16-byte
// pieces of row r are XOR-swizzled by bits of r, so that the 16 rows of a
// fragment read fill the 16 16-byte bank slots of a 256-byte LDS line, and
// rows 8 and 16 apart (a read down a column) fall into different slots.
template <int C>
struct Planes {
  static constexpr int NCH = C / 8;                    // 16-byte pieces per row (4, 8 or 16)
  static constexpr int SH = NCH == 16 ? 0 : NCH == 8 ? 1 : 2;
  static __device__ __forceinline__ int off(int r, int k) {
    const int sw = ((r >> SH) ^ ((r >> 4) << 1)) & (NCH - 1);
    return r * C + ((((k >> 3) ^ sw) << 3) | (k & 7));
  }
};

__device__ __forceinline__ uint32_t bf16_bits(float x) { return __builtin_bit_cast(uint16_t, to_bf16(x)); }

// four values at (r, c .. c + 3), c % 4 == 0, as hi / lo planes
template <int C>
__device__ __forceinline__ void planes_put4(bf16 *hi, int rows, int r, int c, const float (&v)[4]) {
  uint32_t h[4], lo[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const bf16 hb = to_bf16(v[e]);
    h[e] = __builtin_bit_cast(uint16_t, hb);
    lo[e] = bf16_bits(v[e] - static_cast<float>(hb));
  }
  const int o = Planes<C>::off(r, c);
  *reinterpret_cast<uint2 *>(hi + o) = make_uint2(h[0] | (h[1] << 16), h[2] | (h[3] << 16));
  *reinterpret_cast<uint2 *>(hi + rows * C + o) = make_uint2(lo[0] | (lo[1] << 16), lo[2] | (lo[3] << 16));
}
template <int C>
__device__ __forceinline__ void planes_get4(const bf16 *hi, int rows, int r, int c, float (&v)[4]) {
  const int o = Planes<C>::off(r, c);
  const uint2 h = *reinterpret_cast<const uint2 *>(hi + o);
  const uint2 lo = *reinterpret_cast<const uint2 *>(hi + rows * C + o);
  const uint32_t hw[2] = {h.x, h.y}, lw[2] = {lo.x, lo.y};
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const uint32_t hb = (hw[e >> 1] >> (16 * (e & 1))) & 0xffffu, lb = (lw[e >> 1] >> (16 * (e & 1))) & 0xffffu;
    v[e] = __uint_as_float(hb << 16) + __uint_as_float(lb << 16);
  }
}
template <int C>
__device__ __forceinline__ float planes_get(const bf16 *hi, int rows, int r, int k) {
  const int o = Planes<C>::off(r, k);
  return static_cast<float>(hi[o]) + static_cast<float>(hi[rows * C + o]);
}
// 8 values (r, k .. k + 7), k % 8 == 0, as a split fragment
template <int C>
__device__ __forceinline__ FragS planes_row8(const bf16 *hi, int rows, int r, int k) {
  const int o = Planes<C>::off(r, k);
  FragS f;
  f.h = *reinterpret_cast<const bf16x8 *>(hi + o);
  f.l = *reinterpret_cast<const bf16x8 *>(hi + rows * C + o);
  return f;
}
// 8 values (k .. k + 7, c): down a column
template <int C>
__device__ __forceinline__ FragS planes_col8(const bf16 *hi, int rows, int k, int c) {
  FragS f;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int o = Planes<C>::off(k + e, c);
    f.h[e] = hi[o];
    f.l[e] = hi[rows * C + o];
  }
  return f;
}

// Contraction range of tile (I, J), I <= J, of a product of upper-triangular
// (or strictly upper, transposed strictly lower) block matrices: k in
// [16 I, 16 J + 16), padded to whole 32-deep steps by a zero 16-block below
// (I > 0) or above (I == 0: J + 1 < NB there, as NB is even).
__device__ __forceinline__ void upper_range(int I, int J, int &k0, int &k1) {
  k0 = 16 * I;
  k1 = 16 * J + 16;
  if ((J - I) % 2 == 0) {
    if (I > 0) k0 -= 16;
    else k1 += 16;
  }
}

template <int C, int NTH>
constexpr int neumann_plane_rows() {
  constexpr int scratch = NTH == 512 ? (prep_tmp_floats(C) > 8 * 32 * kXbLd ? prep_tmp_floats(C) : 8 * 32 * kXbLd)
                                     : prep_tmp_floats(C);
  int g = C / 16;
  while (g > 1 && 64 * g * C > 4 * scratch) --g;     // g row blocks of R^T: 2 planes x 16 g rows x C bf16
  return g;
}

template <int C, int NTH>
__device__ __forceinline__ void solve_neumann_planes(float *gmat, const float *bet, float *amat, float *tmp,
                                                     int order, int residual) {
  constexpr int NB = C / 16;
  constexpr int LD = C + 4;
  constexpr int NW = NTH / kWave;
  constexpr int NT = NB * (NB + 1) / 2;
  constexpr int SL = (NT + NW - 1) / NW;
  constexpr int GR = neumann_plane_rows<C, NTH>();
  constexpr int SR = (GR * NB + NW - 1) / NW;
  static_assert(64 * C <= 4 * prep_tmp_floats(C), "one row block of R^T fits the scratch");
  static_assert(4 * C * C <= 4 * C * LD, "planes fit the fp32 regions");
  const int tid = threadIdx.x, w = wave_id(), l = lane_id(), lr = l & 15, lq = l >> 4;
  bf16 *const Mp = reinterpret_cast<bf16 *>(gmat);
  bf16 *const Yp = reinterpret_cast<bf16 *>(amat);
  bf16 *const Rp = reinterpret_cast<bf16 *>(tmp);

  // Y = I (m = 0) or (I - M)^T, both triangles; M's planes after every read of G
  constexpr int NOCT = (C * C / 8 + NTH - 1) / NTH;   // octets of M per thread
  float gv[NOCT][8];
#pragma unroll
  for (int j = 0; j < NOCT; ++j) {
    const int u = min(tid + NTH * j, C * C / 8 - 1), c = u / (C / 8), k = 8 * (u % (C / 8));
    ld8(gmat + c * LD + k, gv[j]);
    const float4 b0 = *reinterpret_cast<const float4 *>(bet + k);
    const float4 b1 = *reinterpret_cast<const float4 *>(bet + k + 4);
    const float bb[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
#pragma unroll
    for (int e = 0; e < 8; ++e) gv[j][e] = (k + e < c) ? gv[j][e] * bb[e] : 0.f;   // M[c][k + e]
  }
  const float keep = order > 0 ? 1.f : 0.f;
#pragma unroll 4
  for (int u = tid; u < C * C / 4; u += NTH) {
    const int r = u % C, c = 4 * (u / C);              // neighbouring lanes read neighbouring G columns
    const float br = bet[r] * keep;
    float v[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float g = gmat[(c + e) * LD + r];          // read unconditionally: no branch, no wait per element
      v[e] = ((r == c + e) ? 1.f : 0.f) - ((c + e > r) ? g * br : 0.f);
    }
    planes_put4<C>(Yp, C, r, c, v);
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < NOCT; ++j) {
    const int u = tid + NTH * j, c = u / (C / 8), k = 8 * (u % (C / 8));
    if (u >= C * C / 8) break;
    const float lo4[4] = {gv[j][0], gv[j][1], gv[j][2], gv[j][3]}, hi4[4] = {gv[j][4], gv[j][5], gv[j][6], gv[j][7]};
    planes_put4<C>(Mp, C, c, k, lo4);
    planes_put4<C>(Mp, C, c, k + 4, hi4);
  }
  __syncthreads();

  // tile s of this wave (upper tiles, longest contraction first, dealt back and forth)
  auto my_tile = [&](int s, int &I, int &J) __attribute__((always_inline)) {
    const int p = s * NW + ((s & 1) ? NW - 1 - w : w);
    if (p >= NT) return false;
    lower_tile_at(NB, p, J, I);
    return true;
  };
  // (Y M^T)[16 I + lr][16 J + 4 lq + q]; the n = (k1 - k0) / 32 steps' reads
  // are all issued before the first MFMA
  auto ymt = [&](int I, int J) __attribute__((always_inline)) {
    int k0, k1;
    upper_range(I, J, k0, k1);
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    auto steps = [&](auto n) __attribute__((always_inline)) {
      constexpr int N = decltype(n)::value;
      FragS m[N], y[N];
#pragma unroll
      for (int u = 0; u < N; ++u) {
        m[u] = planes_row8<C>(Mp, C, 16 * J + lr, k0 + 32 * u + 8 * lq);
        y[u] = planes_row8<C>(Yp, C, 16 * I + lr, k0 + 32 * u + 8 * lq);
      }
#pragma unroll
      for (int u = 0; u < N; ++u) mma(acc, m[u], y[u]);
    };
    switch ((k1 - k0) >> 5) {
      case 1: steps(std::integral_constant<int, 1>()); break;
      case 2: if constexpr (NB >= 4) steps(std::integral_constant<int, 2>()); break;
      case 3: if constexpr (NB >= 6) steps(std::integral_constant<int, 3>()); break;
      case 4: if constexpr (NB >= 8) steps(std::integral_constant<int, 4>()); break;
      default: break;
    }
    return acc;
  };
  int tI[SL], tJ[SL];
  bool tv[SL];
#pragma unroll
  for (int s = 0; s < SL; ++s) tv[s] = my_tile(s, tI[s], tJ[s]);
  for (int it = 1; it < order; ++it) {
    f32x4 acc[SL];
#pragma unroll
    for (int s = 0; s < SL; ++s)
      if (tv[s]) acc[s] = ymt(tI[s], tJ[s]);
    __syncthreads();
#pragma unroll
    for (int s = 0; s < SL; ++s) {
      if (!tv[s]) continue;
      const int I = tI[s], J = tJ[s];
      const int r = 16 * I + lr, c = 16 * J + 4 * lq;
      float v[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) v[q] = ((r == c + q) ? 1.f : 0.f) - acc[s][q];
      planes_put4<C>(Yp, C, r, c, v);
    }
    __syncthreads();
  }

  // (R^T Y)[16 I + lr][16 J + 4 lq + q], R^T's rows I from planes Rt with
  // `rows` rows starting at row block I0: Y down its columns, R^T along its rows
  auto rty = [&](const bf16 *Rt, int rows, int I0, int I, int J) __attribute__((always_inline)) {
    int k0, k1;
    upper_range(I, J, k0, k1);
    f32x4 a = {0.f, 0.f, 0.f, 0.f};
    auto steps = [&](auto n) __attribute__((always_inline)) {
      constexpr int N = decltype(n)::value;
      FragS yc[N], rr[N];
#pragma unroll
      for (int u = 0; u < N; ++u) {
        yc[u] = planes_col8<C>(Yp, C, k0 + 32 * u + 8 * lq, 16 * J + lr);
        rr[u] = planes_row8<C>(Rt, rows, 16 * (I - I0) + lr, k0 + 32 * u + 8 * lq);
      }
#pragma unroll
      for (int u = 0; u < N; ++u) mma(a, yc[u], rr[u]);
    };
    switch ((k1 - k0) >> 5) {
      case 1: steps(std::integral_constant<int, 1>()); break;
      case 2: if constexpr (NB >= 4) steps(std::integral_constant<int, 2>()); break;
      case 3: if constexpr (NB >= 6) steps(std::integral_constant<int, 3>()); break;
      case 4: if constexpr (NB >= 8) steps(std::integral_constant<int, 4>()); break;
      default: break;
    }
    return a;
  };
  // R^T = I - Y - Y M^T at tile (I, J) (this lane's four entries)
  auto rt_tile = [&](int I, int J, float (&v)[4]) __attribute__((always_inline)) {
    const f32x4 p = ymt(I, J);
    const int r = 16 * I + lr, c = 16 * J + 4 * lq;
    float y[4];
    planes_get4<C>(Yp, C, r, c, y);
#pragma unroll
    for (int q = 0; q < 4; ++q) v[q] = ((r == c + q) ? 1.f : 0.f) - y[q] - p[q];
  };
  auto add_to_y = [&](int I, int J, const f32x4 &d) __attribute__((always_inline)) {
    const int r = 16 * I + lr, c = 16 * J + 4 * lq;
    float y[4];
    planes_get4<C>(Yp, C, r, c, y);
#pragma unroll
    for (int q = 0; q < 4; ++q) y[q] += d[q];
    planes_put4<C>(Yp, C, r, c, y);
  };
  // The last correction (the only one at r = 1): M is not read again, so
  // R^T goes whole into M's planes, its tiles dealt like the Horner step's;
  // four barriers.
  auto last_correction = [&]() __attribute__((always_inline)) {
    f32x4 acc[SL];
#pragma unroll
    for (int s = 0; s < SL; ++s) {
      if (!tv[s]) continue;
      float v[4];
      rt_tile(tI[s], tJ[s], v);
      acc[s] = f32x4{v[0], v[1], v[2], v[3]};
    }
    __syncthreads();                                   // every read of M done
#pragma unroll
    for (int s = 0; s < SL; ++s) {
      if (!tv[s]) continue;
      const int I = tI[s], J = tJ[s], r = 16 * I + lr, c = 16 * J + 4 * lq;
      const float v[4] = {acc[s][0], acc[s][1], acc[s][2], acc[s][3]};
      planes_put4<C>(Mp, C, r, c, v);
      if (I == J && I > 0) {                           // zero block left of the diagonal: R^T Y's padding
        const float z[4] = {0.f, 0.f, 0.f, 0.f};
        planes_put4<C>(Mp, C, r, c - 16, z);
      }
    }
    __syncthreads();
#pragma unroll
    for (int s = 0; s < SL; ++s)
      if (tv[s]) acc[s] = rty(Mp, C, 0, tI[s], tJ[s]);
    __syncthreads();
#pragma unroll
    for (int s = 0; s < SL; ++s)
      if (tv[s]) add_to_y(tI[s], tJ[s], acc[s]);
    __syncthreads();
  };

  // Earlier corrections (r > 1) by groups of GR row blocks of R^T (top to bottom):
  // tile t of the group at I0, longest contraction first; the block left of
  // each diagonal block of R^T is written as zeros (the padding of R^T Y)
  auto res_tile = [&](int I0, int t, int &I, int &J) __attribute__((always_inline)) {
    const int g = min(GR, NB - I0);
    for (int d = NB - 1 - I0; d >= 0; --d) {
      const int n = min(g, NB - d - I0);                 // group rows with I + d < NB
      if (t < n) {
        I = I0 + t;
        J = I + d;
        return true;
      }
      t -= n;
    }
    return false;
  };
  for (int it = 0; it < residual; ++it) {
    if (it == residual - 1) {
      last_correction();
      break;
    }
    f32x4 acc[SR];
    int pI[SR], pJ[SR];                                // the previous group's tiles
    bool pv[SR];
#pragma unroll
    for (int s = 0; s < SR; ++s) pv[s] = false;
    for (int I0 = 0; I0 < NB; I0 += GR) {
      int gI[SR], gJ[SR];
      bool gv2[SR];
#pragma unroll
      for (int s = 0; s < SR; ++s) gv2[s] = res_tile(I0, s * NW + w, gI[s], gJ[s]);
      // R^T rows of the group: I - Y - Y M^T
#pragma unroll
      for (int s = 0; s < SR; ++s) {
        if (!gv2[s]) continue;
        const int I = gI[s], J = gJ[s];
        const int r = 16 * I + lr, c = 16 * J + 4 * lq;
        float v[4];
        rt_tile(I, J, v);
        planes_put4<C>(Rp, 16 * GR, r - 16 * I0, c, v);
        if (I == J && I > 0) {
          const float z[4] = {0.f, 0.f, 0.f, 0.f};
          planes_put4<C>(Rp, 16 * GR, r - 16 * I0, c - 16, z);
        }
      }
      // the previous group's update: rows above this group
      {
#pragma unroll
        for (int s = 0; s < SR; ++s) {
          if (pv[s]) add_to_y(pI[s], pJ[s], acc[s]);
        }
      }
      __syncthreads();
#pragma unroll
      for (int s = 0; s < SR; ++s)
        if (gv2[s]) acc[s] = rty(Rp, 16 * GR, I0, gI[s], gJ[s]);
      __syncthreads();
#pragma unroll
      for (int s = 0; s < SR; ++s) {
        pv[s] = gv2[s];
        pI[s] = gI[s];
        pJ[s] = gJ[s];
      }
    }
#pragma unroll
    for (int s = 0; s < SR; ++s)
      if (pv[s]) add_to_y(pI[s], pJ[s], acc[s]);
    __syncthreads();
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
// NTH threads (256 or 512); with 512 the per-wave transpose buffers sit in
// the solve's scratch.
// kFwdOnly: the item never prepares for the backward pass (its code is left
// out of the forward kernels).  kOneBeta: one beta head per key head.
template <typename TIn, class P, int C, int DK, int NTH = 256, bool kFwdOnly = false, bool kOneBeta = false>
struct PrepItem {
  static constexpr int NB = C / 16;
  static constexpr int NKV = (C * DK / 8 + NTH - 1) / NTH;  // bound on 8-element log-alpha vectors per thread
  static constexpr int KS = DK / 32;
  using Split = typename P::Split;
  __device__ __forceinline__ bool bwd() const { return !kFwdOnly && a.bwd != 0; }
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
  int *const flags;                                    // [NB] block ranges, [kChunkWide], [kHasReset]
  float *const xb;                                     // this wave's transpose buffer [32 channels][kXbLd]
  unsigned char *const seg;                            // [C] document segment of each token (block route)
  const TIn *const la, *const bp, *const kbase, *const qbase;
  const size_t row_stride, la_row;                     // token strides of q / k and of log alpha
  void *const tKB, *const tQB, *const tKH, *const tL;

  // region0: floats before the union region
  __device__ __forceinline__ PrepItem(const ChunkArgs &a_, int c_, int hk_, int b_, float *smem_, int region0)
      : a(a_), c(c_), hk(hk_), b(b_), G(a_.G), gs(a_.gshift), T(a_.T), t0(c_ * C), tid(threadIdx.x),
        w(wave_id()), l(lane_id()), lr(lane_id() & 15), lq(lane_id() >> 4),
        lgG(__builtin_ctz(DK) - a_.gshift), Rb(kOneBeta ? 1 : a_.H_beta / a_.H_k), smem(smem_), lam(smem_),
        ureg(smem_ + region0), tmp(ureg + C * prep_ld(C)),
        bet(ureg + (NTH == 256 ? prep_union_floats(C, DK) : prep_union8_floats(C, DK))),
        flags(reinterpret_cast<int *>(bet + C)),
        xb((NTH == 256 ? reinterpret_cast<float *>(flags + 16) : tmp) + wave_id() * 32 * kXbLd),
        seg(reinterpret_cast<unsigned char *>(reinterpret_cast<float *>(flags + 16) + (NTH == 256 ? 4 * 32 * kXbLd : 0))),
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
        const int e = min(8 * (tid + NTH * j), C * G - 8);
        r.v[j].load(la + tok(e >> lgG) * la_row + (size_t)hk * G + (e & (G - 1)));
      }
    } else {
#pragma unroll
      for (int j = 0; j < NKV; ++j) {
        const int e = min(tid + NTH * j, C * G - 1);
        r.s[j] = la[tok(e >> lgG) * la_row + (size_t)hk * G + (e & (G - 1))];
      }
    }
  }

  // Lambda = in-chunk prefix sum of log alpha per decay group (Systolic
  // Linear Attention, Table 2), and the decay range flags: per 16-token block
  // and over the chunk.  With document resets (the same paper, Table 2,
  // kappa_c) seg[t] becomes the number of documents started at or before t in
  // the chunk and flags[kHasReset] is set.  Lambda does not restart at a
  // reset: every use of it is a difference within one document (pairs of
  // the same segment, the first segment's decay from the chunk start, the
  // last one's to the chunk end), which a restart leaves unchanged, and
  // without it Lambda stays monotone, so the pivoted factors stay bounded and
  // a block holding a reset needs no entry-by-entry pass.  Ends with a barrier.
  __device__ __forceinline__ void lambda(const LaRegs &r) {
    if (G >= 8) {
#pragma unroll
      for (int j = 0; j < NKV; ++j) {
        const int e = 8 * (tid + NTH * j);
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
        const int e = tid + NTH * j;
        if (e < C * G) lam[e] = (t0 + (e >> lgG) < T) ? static_cast<float>(r.s[j]) : 0.f;
      }
    }
    if (tid < 16) flags[tid] = 0;
    if (tid < C) seg[tid] = (a.reset && t0 + tid < T) ? (a.reset[(size_t)b * T + t0 + tid] != 0) : 0;
    __syncthreads();
    for (int g = tid; g < G; g += blockDim.x) prefix_column<C>(lam + g, G);
    __syncthreads();
    if (a.reset && tid == blockDim.x - 1) {            // reset marks -> segment numbers
      int n = 0;
      for (int t = 0; t < C; ++t) {
        if (seg[t]) {
          flags[kHasReset] = 1;
          ++n;
        }
        seg[t] = n;
      }
    }
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
  // exp(Lambda_C) per channel; -0 in every channel when a document starts in
  // the chunk (nothing is carried across the chunk, and the sign tells the
  // scan that kappa_c = 0 for the momentum buffer).  Reads flags[kHasReset],
  // so it runs after lambda().
  __device__ __forceinline__ void write_gm() const {
    if (tid < DK) gm_row()[tid] = flags[kHasReset] ? -0.f : __expf(lam[(C - 1) * G + (tid >> gs)]);
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
  // wave's LDS buffer into channel-row fragments.  Backward preparation: the
  // reverse scan's operands instead, tokens reversed within the chunk --
  // KB = J Khat (token rows), QB = (J Qbar)^T and KH = (J Kbar)^T.
  __device__ __forceinline__ void scan_operands(int I, int s, const float (&kbar)[8], const float (&qbar)[8],
                                                const float (&kh)[8]) const {
    if (bwd()) {
      IO::put_plain8(tKB, (NB - 1 - I) * KS + s, 16 * lq + 15 - lr, kh);
      put_channel_rows(tQB, I, s, qbar, true);
      put_channel_rows(tKH, I, s, kbar, true);
      return;
    }
    IO::put_plain8(tKB, I * KS + s, l, kbar);
    IO::put_plain8(tQB, I * KS + s, l, qbar);
    put_channel_rows(tKH, I, s, kh, false);
  }

  // A d_k x C channel-row tile from token-row values: lane (token lr,
  // channels 8 lq ..) writes, lane (channel 16 (l >> 5) + (l & 15), tokens
  // 8 g ..) reads back a fragment.  `rev`: token t goes to column C - 1 - t.
  __device__ __forceinline__ void put_channel_rows(void *tile, int I, int s, const float (&v)[8], bool rev) const {
#pragma unroll
    for (int e = 0; e < 8; ++e) xb[(8 * lq + e) * kXbLd + lr] = v[e];
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    const int chl = 16 * (l >> 5) + (l & 15), g = (l >> 4) & 1;
    float xt[8];
    const float4 u0 = *reinterpret_cast<const float4 *>(xb + chl * kXbLd + 8 * g);
    const float4 u1 = *reinterpret_cast<const float4 *>(xb + chl * kXbLd + 8 * g + 4);
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    if (!rev) {
      xt[0] = u0.x; xt[1] = u0.y; xt[2] = u0.z; xt[3] = u0.w; xt[4] = u1.x; xt[5] = u1.y; xt[6] = u1.z; xt[7] = u1.w;
      IO::put_plain8(tile, (2 * s + (l >> 5)) * (C / 32) + I / 2, 16 * (2 * (I & 1) + g) + (l & 15), xt);
    } else {
      // tokens 16 I + 8 g + e -> 16 Ir + 8 (1 - g) + 7 - e
      const int Ir = NB - 1 - I, gr = 1 - g;
      xt[0] = u1.w; xt[1] = u1.z; xt[2] = u1.y; xt[3] = u1.x; xt[4] = u0.w; xt[5] = u0.z; xt[6] = u0.y; xt[7] = u0.x;
      IO::put_plain8(tile, (2 * s + (l >> 5)) * (C / 32) + Ir / 2, 16 * (2 * (Ir & 1) + gr) + (l & 15), xt);
    }
  }

  // The 16 x 16 block (I, J) of L from an MFMA accumulator (lane: rows
  // 4 lq .. 4 lq + 3, column lr), through the wave's LDS buffer, as 32
  // fragments of 8 columns; on the diagonal block the entries above the
  // diagonal are zero.  Backward preparation: block (I, J) of L is block
  // (NB-1-J, NB-1-I) of J L^T J, entry (r, c) at (15 - c, 15 - r).
  __device__ __forceinline__ void store_L_block(int I, int J, const f32x4 &acc) const {
    const bool rev = bwd() != 0;
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const int r = 4 * lq + q4;
      const float v = (I > J || r >= lr) ? acc[q4] : 0.f;
      if (rev) {
        xb[(15 - lr) * kXbLd + 15 - r] = v;
      } else {
        xb[r * kXbLd + lr] = v;
      }
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    const int r = l & 15, h = (l >> 4) & 1;
    const float4 u0 = *reinterpret_cast<const float4 *>(xb + r * kXbLd + 8 * h);
    const float4 u1 = *reinterpret_cast<const float4 *>(xb + r * kXbLd + 8 * h + 4);
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    const int bi = rev ? NB - 1 - J : I, bj = rev ? NB - 1 - I : J;
    if (l < 32) {
      const float v[8] = {u0.x, u0.y, u0.z, u0.w, u1.x, u1.y, u1.z, u1.w};
      IO::put_plain8(tL, bi * (C / 32) + bj / 2, 16 * (2 * (bj & 1) + h) + r, v);
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
  static constexpr int NBET = kOneBeta ? (C + NTH - 1) / NTH : 1024 / NTH;   // beta values: C * Rb <= 1024
  __device__ __forceinline__ void load_betas(TIn (&bets)[NBET]) const {
#pragma unroll
    for (int j = 0; j < NBET; ++j) {
      const int e = min(tid + NTH * j, C * Rb - 1);
      bets[j] = bp[tok(e % C) * a.H_beta + hk * Rb + e / C];
    }
  }
  __device__ __forceinline__ void put_betas(const TIn (&bets)[NBET], int rb) const {
#pragma unroll
    for (int j = 0; j < NBET; ++j) {
      const int e = tid + NTH * j;
      if (e / C == rb && e < C * Rb) bet[e % C] = (t0 + e % C < T) ? static_cast<float>(bets[j]) : 0.f;
    }
  }

  // Per beta head: A = (I + G diag(beta))^{-1} from gsolve into asolve (row
  // stride C + 4 both), then diag(beta) A to the workspace: the upper half of
  // a 16 x 32 block that straddles the diagonal as zeros, blocks wholly above
  // it not at all.  bet0_ready: the first head's beta is already in LDS
  // (written before a barrier that precedes the call).
  // kApprox: the Neumann solves are compiled in (the exact solve's kernels
  // leave them out, which keeps their register allocation and schedule).
  template <bool kApprox = true>
  __device__ __forceinline__ void solve_store(float *gsolve, float *asolve, const TIn (&bets)[NBET],
                                              bool bet0_ready) const {
    // bf16 Neumann with one beta head per key head: the solve on split-bf16
    // planes, which leaves X^T in asolve's bytes and overwrites G
    const bool planes = kApprox && !P::kF32 && a.solve == 1 && Rb == 1 && !bwd();
    for (int rb = 0; rb < Rb; ++rb) {
      const int hb = hk * Rb + rb;
      __syncthreads();
      if (rb > 0 || !bet0_ready) {
        put_betas(bets, rb);
        __syncthreads();
      }
      if (a.solve == 0) {
        if (NTH == 512 || !bwd()) {
          solve_exact<C, NTH == 512, true>(gsolve, bet, asolve, tmp);
        } else {
          if constexpr (NTH != 512) solve_exact<C, false, false>(gsolve, bet, asolve, tmp);
        }
      } else if constexpr (kApprox) {
        if (a.solve == 1) {
          if constexpr (!P::kF32) {
            if (planes)
              solve_neumann_planes<C, NTH>(gsolve, bet, asolve, tmp, a.order, a.residual);
            else
              solve_neumann<C, NTH, Split>(gsolve, bet, asolve, tmp, a.order, a.residual);
          } else {
            solve_neumann<C, NTH, Split>(gsolve, bet, asolve, tmp, a.order, a.residual);
          }
        } else {
          solve_block_neumann<C>(gsolve, bet, asolve, tmp, a.order);
        }
      }
      __syncthreads();
      // diag(beta) A_c: the scan's chunk writes are E_c = diag(beta) A_c Y.
      // The exact solve has already scaled the rows, except for the
      // backward pass (four waves), which also stores A unscaled.
      const bool scaled = a.solve == 0 && (NTH == 512 || !bwd());
      void *tA = ws_tile(a, kWsA, a.H_beta, hb, b, c);
      for (int u = tid; u < C * C / 8; u += blockDim.x) {   // unit = fragment (row, col .. col + 7)
        const int blk = u >> 6, f = u & 63;
        if (2 * (blk % (C / 32)) > blk / (C / 32)) continue;   // block wholly above the diagonal: not written
        const int row = 16 * (blk / (C / 32)) + (f & 15), col = 32 * (blk % (C / 32)) + 8 * (f >> 4);
        const bool upper = col / 16 > row / 16;             // the half of a straddling block above the diagonal
        float x[8];
        if (bwd()) {
          // J (diag(beta) A)^T J: entry (row, col) = beta_r A[r][C-1-row], r = C-1-col
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int rr = C - 1 - col - e;
            x[e] = upper ? 0.f : bet[rr] * asolve[rr * (C + 4) + C - 1 - row];
          }
        } else if (planes) {
#pragma unroll
          for (int e = 0; e < 8; ++e)
            x[e] = upper ? 0.f : bet[row] * planes_get<C>(reinterpret_cast<const bf16 *>(asolve), C, col + e, row);
        } else {
          const float4 a0 = *reinterpret_cast<const float4 *>(asolve + row * (C + 4) + col);
          const float4 a1 = *reinterpret_cast<const float4 *>(asolve + row * (C + 4) + col + 4);
          const float bt = scaled ? 1.f : bet[row];
          const float y[8] = {bt * a0.x, bt * a0.y, bt * a0.z, bt * a0.w, bt * a1.x, bt * a1.y, bt * a1.z, bt * a1.w};
#pragma unroll
          for (int e = 0; e < 8; ++e) x[e] = upper ? 0.f : y[e];
        }
        IO::put_plain8(tA, blk, f, x);
      }
      if (bwd()) {
        // the gradient kernel's copies: A_c unscaled and (once) G_c, fp32 row-major
        float *au = a.au + (((size_t)b * a.H_beta + hb) * a.N_c + c) * (C * C);
        for (int u = tid; u < C * C / 4; u += blockDim.x) {
          const int row = u / (C / 4), col = 4 * (u % (C / 4));
          const float4 v = *reinterpret_cast<const float4 *>(asolve + row * (C + 4) + col);
          *reinterpret_cast<float4 *>(au + row * C + col) =
              make_float4(col <= row ? v.x : 0.f, col + 1 <= row ? v.y : 0.f, col + 2 <= row ? v.z : 0.f,
                          col + 3 <= row ? v.w : 0.f);
        }
        if (rb == 0) {
          float *gu = a.gu + (((size_t)b * a.H_k + hk) * a.N_c + c) * (C * C);
          for (int u = tid; u < C * C / 4; u += blockDim.x) {
            const int row = u / (C / 4), col = 4 * (u % (C / 4));
            const float4 v = *reinterpret_cast<const float4 *>(gsolve + row * (C + 4) + col);
            *reinterpret_cast<float4 *>(gu + row * C + col) =
                make_float4(col < row ? v.x : 0.f, col + 1 < row ? v.y : 0.f, col + 2 < row ? v.z : 0.f,
                            col + 3 < row ? v.w : 0.f);
          }
        }
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

// log alpha of one token for the lane's channels 32 s + 8 lq + e (s < KS,
// e < 8), in flight between issue() and get().
template <typename TIn, int KS, int kGate>
struct LaLane {
  static constexpr bool kVec = kGate != kGateGroupsFew;  // G >= 8: read as 8-element vectors
  Raw8<TIn> v[kVec ? KS : 1];
  TIn sc[4];
  // row: the token's G values for the key head
  __device__ __forceinline__ void issue(const TIn *row, int lq, int gs, int G) {
    if constexpr (kVec) {
#pragma unroll
      for (int s = 0; s < KS; ++s) v[s].load(row + min((32 * s + 8 * lq) >> gs, G - 8));
    } else {
#pragma unroll
      for (int g = 0; g < 4; ++g) sc[g] = row[min(g, G - 1)];
    }
  }
  // lt[s][e] = scale * log alpha; rising |= any value > 0
  __device__ __forceinline__ void get(float (&lt)[KS][8], float scale, int lq, int gs, int G, bool &rising) const {
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const int ch0 = 32 * s + 8 * lq;
      if constexpr (kGate == kGatePerChannel) {
        float f[8];
        v[s].to_float(f);
#pragma unroll
        for (int e = 0; e < 8; ++e) lt[s][e] = f[e] * scale;
      } else if constexpr (kGate == kGateGroupsVec) {
        float f[8];
        v[s].to_float(f);
        const int g0 = min(ch0 >> gs, G - 8);
        if (gs >= 3) {                                   // one group for the lane's eight channels
          const float u = pick(f, (ch0 >> gs) - g0) * scale;
#pragma unroll
          for (int e = 0; e < 8; ++e) lt[s][e] = u;
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) lt[s][e] = pick(f, ((ch0 + e) >> gs) - g0) * scale;
        }
      } else {
        // G < 8 < d_k / G: the lane's eight channels share one group
        const int g = ch0 >> gs;
        const float u = static_cast<float>(g == 0 ? sc[0] : g == 1 ? sc[1] : g == 2 ? sc[2] : sc[3]) * scale;
#pragma unroll
        for (int e = 0; e < 8; ++e) lt[s][e] = u;
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) rising |= lt[s][e] > 0.f;
    }
  }
};
// kMode: 0 the exact solve, forward only, no document resets; 1 the exact
// solve, forward or backward preparation (no resets: the backward pass
// takes the plain layer); 2 the Neumann solves (forward only, no resets);
// 3 the exact solve, forward with resets allowed; 4 as 0 with one beta head
// per key head; 5 as 2 with resets allowed.
template <typename TIn, class P, int DK, int kGate, int kMode>
__global__ __launch_bounds__(256, DK <= 128 ? 3 : 2) void prep_chunk_kernel(ChunkArgs a) {
  constexpr int C = 64;
  constexpr bool kApprox = kMode == 2 || kMode == 5;
  constexpr bool kResets = kMode == 3 || kMode == 5;
  using X = PrepItem<TIn, P, C, DK, 256, kMode != 1, kMode == 4>;
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
  LaLane<TIn, KS, kGate> lal;
  lal.issue(x.la + x.tok(tr) * x.la_row + (size_t)x.hk * G, lq, gs, G);
  Raw8<TIn> kt[KS], qt[KS];
  x.load_rows(kt, x.kbase, I);
  x.load_rows(qt, x.qbase, I);
  TIn bets[NBET];
  x.load_betas(bets);
  // a document starting at this token (Systolic Linear Attention, Table 2,
  // kappa_c): Lambda runs on across it, the pairs of different documents are
  // zero, only the first document sees the chunk-entry state and only the
  // last one carries to the chunk's end
  const bool resets = kResets && a.reset != nullptr;   // uniform
  const bool reset_here = resets && mt > 0.f && a.reset[x.tok(tr)] != 0;


  // ---- Lambda of the lane's token in log2 units (log2(e) Lambda): in-block
  // prefix, then block offsets
  constexpr float kLog2e = 1.4426950408889634f;
  const float scale = mt * kLog2e;                     // tokens past T: zero log decay
  float lt[KS][8];
  bool rising = false;                                 // a positive log alpha (Lambda not monotone)
  lal.get(lt, scale, lq, gs, G, rising);
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
  if (resets) {
    if (lq == 0) x.seg[tr] = reset_here ? 1 : 0;
    if (x.tid == 0) x.flags[kHasReset] = 0;
  }
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
  if (resets && x.tid == 255) {                        // reset marks -> document numbers within the chunk
    int n = 0;
    for (int t = 0; t < C; ++t) {
      n += x.seg[t];
      x.seg[t] = n;
    }
    x.flags[kHasReset] = n > 0;
  }
  __syncthreads();
  const bool wide = __builtin_amdgcn_readfirstlane(x.flags[kChunkWide]) != 0;
  if (wide) {
    if (x.tid == 0) x.gm_row()[0] = kWideMark;         // left to the block-pivot kernel
    return;
  }
  // exp(Lambda_C) per channel; -0 when a document starts in the chunk
  const bool has_reset = resets && x.flags[kHasReset] != 0;
  if (x.tid < DK) x.gm_row()[x.tid] = has_reset ? -0.f : gc[x.tid];
  const int seg_last = resets ? x.seg[C - 1] : 0;
  const bool sees_entry = !resets || x.seg[tr] == 0, carries = !resets || x.seg[tr] == seg_last;
  auto same_doc = [&](int r_, int c_) { return !resets || x.seg[r_] == x.seg[c_]; };
  auto load8 = [&](const float *p, float (&y)[8]) __attribute__((always_inline)) {
    const float4 u = *reinterpret_cast<const float4 *>(p);
    const float4 v = *reinterpret_cast<const float4 *>(p + 4);
    y[0] = u.x; y[1] = u.y; y[2] = u.z; y[3] = u.w; y[4] = v.x; y[5] = v.y; y[6] = v.z; y[7] = v.w;
  };
  // ---- row and column operands, scan operands, the diagonal pair.  The
  // forward pass forms the products transposed (column operand as the
  // MFMA's A), so a lane holds four consecutive columns of one row of G and
  // L, stored without a transpose; the backward pass's reversed layouts go
  // through the transpose buffers.
  using IO = typename X::IO;
  const bool fwd = !x.bwd();                           // uniform
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
      kbar[e] = sees_entry ? k * d : 0.f;
      qbar[e] = sees_entry ? q * d : 0.f;
      kh[e] = carries ? k * (ui * fc[e]) : 0.f;        // exp(Lambda_C - Lambda_t)
    }
    ak[s] = make_frag<Split>(yk);
    aq[s] = make_frag<Split>(yq);
    const Split bk = make_frag<Split>(yb);
    if (I < NB - 1) lds_put_frag(colop, I * KS + s, bk);
    if (fwd) {
      mma(dG, bk, ak[s]);
      mma(dL, bk, aq[s]);
    } else {
      mma(dG, ak[s], bk);
      mma(dL, aq[s], bk);
    }
    x.scan_operands(I, s, kbar, qbar, kh);
  }
  float *gsolve = x.smem;
  // forward: lane holds row 16 Ir + lr, columns 16 J + 4 lq ..
  auto put_pair = [&](int Ir, int J, const f32x4 &accG, const f32x4 &accL) __attribute__((always_inline)) {
    const int row = 16 * Ir + lr, c0 = 16 * J + 4 * lq;
    float g[4], lv[4];
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const bool same = same_doc(row, c0 + q4);
      g[q4] = (same && (Ir > J || lr > 4 * lq + q4)) ? accG[q4] : 0.f;
      lv[q4] = (same && (Ir > J || lr >= 4 * lq + q4)) ? accL[q4] : 0.f;
    }
    *reinterpret_cast<float4 *>(gsolve + row * (C + 4) + c0) = make_float4(g[0], g[1], g[2], g[3]);
    IO::put_half4(x.tL, Ir * (C / 32) + J / 2, 16 * (2 * (J & 1) + (lq >> 1)) + lr, lq & 1, lv);
  };
  if (fwd) {
    // the diagonal block's L now; its G row after the barrier (G overlays Lambda's rows)
    float lv[4];
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4)
      lv[q4] = (lr >= 4 * lq + q4 && same_doc(16 * I + lr, 16 * I + 4 * lq + q4)) ? dL[q4] : 0.f;
    IO::put_half4(x.tL, I * (C / 32) + I / 2, 16 * (2 * (I & 1) + (lq >> 1)) + lr, lq & 1, lv);
  } else {
    x.store_L_block(I, I, dL);
  }
  __syncthreads();                                     // column operands complete, Lambda rows dead
  if (fwd) {
    put_pair(I, I, dG, dL);
    for (int J = 0; J < I; ++J) {
      f32x4 accG = {0.f, 0.f, 0.f, 0.f}, accL = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        const Split bj = lds_get_frag<Split>(colop, J * KS + s);
        mma(accG, bj, ak[s]);
        mma(accL, bj, aq[s]);
      }
      put_pair(I, J, accG, accL);
    }
  } else {
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
  }
  x.zero_upper_L();
  x.template solve_store<kApprox>(gsolve, x.ureg, bets, true);
}

// Block-pivot route for one chunk: p = first token of the row block; every
// exponent on the causal side is <= 0, except on a diagonal block, where it
// is at most the block's decay range (<= kPivotRange unless the block is
// flagged and evaluated entry by entry).  Wave w owns blocks w (and 7 - w
// when C = 128).
template <typename TIn, class P, int C, int DK, int NTH, bool kFwdOnly = false>
__device__ __forceinline__ void prep_block_item(const ChunkArgs &a, int c, int hk, int b, float *smem) {
  using X = PrepItem<TIn, P, C, DK, NTH, kFwdOnly>;
  using Split = typename X::Split;
  constexpr int NB = X::NB, KS = X::KS;
  constexpr int NWV = NTH / 64;                        // waves
  constexpr int NR = NB >= NWV ? NB / NWV : 1;         // row blocks per wave (waves past NB build none)
  X x(a, c, hk, b, smem, prep_region0_floats(C, a.G));
  const int w = x.w, lr = x.lr, lq = x.lq, T = x.T, t0 = x.t0;
  auto own = [&](int r) { return (r & 1) ? NWV * r + NWV - 1 - w : NWV * r + w; };
  typename X::LaRegs lar;
  x.issue_la(lar);
  Raw8<TIn> kt[KS], qt[KS], kj[KS];
  x.load_rows(kt, x.kbase, own(0));
  x.load_rows(qt, x.qbase, own(0));
  x.load_rows(kj, x.kbase, 0);
  x.lambda(lar);
  x.write_gm();
  float *gmat = x.ureg;
  // Document segments (all 0 without resets): only segment 0 sees the
  // chunk-entry state (Kbar, Qbar rows), only the last one carries to the
  // chunk's end (Khat rows), and pairs of different segments are zero (a
  // select after the product; Lambda runs on across resets, so their factors
  // stay bounded).
  const bool resets = a.reset != nullptr;             // uniform: without resets no segment is read
  const int seg_last = resets ? x.seg[C - 1] : 0;
  auto same_doc = [&](int r_, int c_) { return !resets || x.seg[r_] == x.seg[c_]; };
  for (int r = 0; r < NR; ++r) {
    const int I = own(r);
    if (I >= NB) continue;                             // uniform per wave
    const int tr = 16 * I + lr, piv = 16 * I;
    const float mt = (t0 + tr < T) ? 1.f : 0.f;
    const bool sees_entry = !resets || x.seg[tr] == 0, carries = !resets || x.seg[tr] == seg_last;
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
        kbar[e] = sees_entry ? xk[e] * d : 0.f;
        qbar[e] = sees_entry ? xq[e] * d : 0.f;
        kh[e] = carries ? xk[e] * h : 0.f;
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
          if (row >= col && t0 + row < T && same_doc(row, col)) {
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
        const bool same = same_doc(row, col);
        gmat[row * (C + 4) + col] = ((I > J || row > col) && same) ? accG[q4] : 0.f;
        accL[q4] = same ? accL[q4] : 0.f;
      }
      x.store_L_block(I, J, accL);
    }
  }
  x.zero_upper_L();
  TIn bets[X::NBET];                                   // beta loaded here: short-lived registers
  x.load_betas(bets);
  x.solve_store(gmat, x.smem, bets, false);
}

// Block-pivot route at C = 128, d_k <= 128: eight waves, wave w owns row
// block w.  Lambda stays in registers as in the chunk-pivot route (log2
// units; in-block prefix P_t over a DPP row, block offsets through LDS).
// Off-diagonal pairs are factored at block boundaries,
//   exp(Lambda_t - Lambda_j) = exp(Lambda_t - Lambda_{16 I - 1})
//                              * prod_{J < K < I} exp(tot_K)
//                              * exp(Lambda_{16 J + 15} - Lambda_j),
// every factor <= 1 (tot_K: the block's summed log alpha).  The owner of
// block J builds the last factor's column operand once and shares it through
// LDS; a row operand walks down its row's pairs, multiplied by the block
// decay exp(tot_K) between pairs, so a pair costs no exponential and no
// global load.  The diagonal pair takes the same column operand with the row
// operand K_t exp(Lambda_t - Lambda_{16 I + 15}) (>= 1, at most
// exp(kPivotRange) unless the block is flagged and evaluated entry by
// entry).  Pairs are balanced: the owner of row I takes J = I - 3 .. I, and
// wave 7 - I the rest of the row (J <= I - 4).
//
// Products are formed transposed (column operand as the MFMA's A): a lane
// then holds four consecutive columns of one row of G and L, which go to
// LDS and to the workspace's fragments without a transpose.  For the same
// reason the fp16 K-hat^T fragments come from an MFMA with an identity
// operand (one nonzero product per output, exact) instead of an LDS
// transpose.  The backward pass never prepares C = 128 chunks.
// kMode: 0 the exact solve without document resets; 2 the Neumann solves
// without resets; 3 the exact solve with resets allowed; 5 the Neumann
// solves with resets allowed.
template <typename TIn, class P, int DK, int kGate, int kMode>
__global__ __launch_bounds__(512) void prep_block128_kernel(ChunkArgs a) {
  constexpr bool kResets = kMode == 3 || kMode == 5;
  constexpr int C = 128, NTH = 512;
  using X = PrepItem<TIn, P, C, DK, NTH, true>;        // C = 128: never the backward preparation
  using Split = typename X::Split;
  using IO = typename X::IO;
  constexpr int NB = X::NB, KS = X::KS, NBET = X::NBET;
  constexpr int R0 = C * (C + 4);
  constexpr float kLog2e = 1.4426950408889634f;
  static_assert(NB == 8 && DK <= 128, "eight row blocks, one per wave");
  extern __shared__ __align__(16) unsigned char smem_raw[];
  const X x(a, blockIdx.x, blockIdx.y, blockIdx.z, reinterpret_cast<float *>(smem_raw), R0);
  const int I = x.w, lr = x.lr, lq = x.lq, gs = x.gs, G = x.G, tid = x.tid;
  const int tr = 16 * I + lr;
  const float mt = (x.t0 + tr < x.T) ? 1.f : 0.f;
  // LDS.  Region 0 (later the solve's A): the column operands of blocks
  // 0 .. 6, the block decays exp(tot_K) and the block offsets.  The G region
  // holds the per-block factor tables until the pairs start.  The scratch
  // after G holds the block totals and first-token values until the tables
  // are built, then the transpose buffers.
  unsigned char *colop = reinterpret_cast<unsigned char *>(x.smem);
  float *dec = x.smem + (NB - 1) * KS * 512;           // [NB][DK] exp2(tot_K)
  float *offt = dec + NB * DK;                         // [NB + 1][DK] Lambda_{16 K - 1} (log2)
  float *f0t = x.ureg;                                 // [NB][DK] exp2(P_0)
  float *g0t = f0t + NB * DK;                          // [NB][DK] exp2(Lambda_{16 K})
  float *eit = g0t + NB * DK;                          // [NB][DK] exp2(P_0 - tot_K)
  float *hct = eit + NB * DK;                          // [NB][DK] exp2(Lambda_{C-1} - Lambda_{16 K + 15})
  float *stot = x.tmp;                                 // [NB][DK] block totals (log2)
  float *sp0 = stot + NB * DK;                         // [NB][DK] first-token values (log2)
  static_assert((NB - 1) * KS * 512 + NB * DK + (NB + 1) * DK <= R0, "region 0");
  static_assert(4 * NB * DK <= R0, "factor tables");

  // ---- all loads of the item, issued together
  LaLane<TIn, KS, kGate> lal;
  lal.issue(x.la + x.tok(tr) * x.la_row + (size_t)x.hk * G, lq, gs, G);
  const unsigned char rmark = (kResets && a.reset) ? a.reset[x.tok(tr)] : 0;
  Raw8<TIn> kt[KS], qt[KS];
  x.load_rows(kt, x.kbase, I);
  x.load_rows(qt, x.qbase, I);
  TIn bets[NBET];
  x.load_betas(bets);
  const bool reset_here = rmark != 0 && mt > 0.f;

  // ---- in-block prefix, block flag, block totals and first-token values
  float lt[KS][8];
  bool bad = false;                                    // a positive log alpha in the block
  lal.get(lt, mt * kLog2e, lq, gs, G, bad);
#pragma unroll
  for (int s = 0; s < KS; ++s) {
#pragma unroll
    for (int e = 0; e < 8; ++e) lt[s][e] = row_prefix16(lt[s][e]);
  }
#pragma unroll
  for (int s = 0; s < KS; ++s) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float p0 = dpp_row_bcast<0>(lt[s][e]);      // every lane takes part in the broadcast
      bad = bad | ((lr == 15) & !(p0 - lt[s][e] <= kPivotRange * kLog2e));
    }
  }
  const bool wide = __ballot(bad) != 0;                // uniform: the diagonal block entry by entry
  if (lr == 0 || lr == 15) {
    float *d0 = (lr == 0 ? sp0 : stot) + I * DK + 8 * lq;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      *reinterpret_cast<float4 *>(d0 + 32 * s) = make_float4(lt[s][0], lt[s][1], lt[s][2], lt[s][3]);
      *reinterpret_cast<float4 *>(d0 + 32 * s + 4) = make_float4(lt[s][4], lt[s][5], lt[s][6], lt[s][7]);
    }
  }
  if (lq == 0) x.seg[tr] = reset_here ? 1 : 0;
  if (tid == 0) x.flags[kHasReset] = 0;
  __syncthreads();
  // ---- per-block factor tables: thread (part, channel) takes blocks 2 part, 2 part + 1
  if (tid < 4 * DK) {
    const int ch = tid % DK, part = tid / DK;
    float tot[NB], all = 0.f, o = 0.f;
#pragma unroll
    for (int K = 0; K < NB; ++K) {
      tot[K] = stot[K * DK + ch];
      all += tot[K];
    }
#pragma unroll
    for (int K = 0; K < NB; ++K) {
      if (K / 2 == part) {
        const float p0 = sp0[K * DK + ch];
        f0t[K * DK + ch] = __builtin_amdgcn_exp2f(p0);
        g0t[K * DK + ch] = __builtin_amdgcn_exp2f(o + p0);
        eit[K * DK + ch] = __builtin_amdgcn_exp2f(p0 - tot[K]);
        hct[K * DK + ch] = __builtin_amdgcn_exp2f(all - o - tot[K]);
        dec[K * DK + ch] = __builtin_amdgcn_exp2f(tot[K]);
        offt[K * DK + ch] = o;
      }
      o += tot[K];
    }
    if (part == 3) offt[NB * DK + ch] = all;
  }
  if (kResets && a.reset && tid == NTH - 1) {          // reset marks -> document numbers
    int n = 0;
    for (int t = 0; t < C; ++t) {
      n += x.seg[t];
      x.seg[t] = n;
    }
    x.flags[kHasReset] = n > 0;
  }
  __syncthreads();
  // exp(Lambda_{C-1}) per channel; -0 when a document starts in the chunk
  if (tid < DK) x.gm_row()[tid] = x.flags[kHasReset] ? -0.f : __builtin_amdgcn_exp2f(offt[NB * DK + tid]);

  // Document segments (all 0 without resets): only segment 0 sees the
  // chunk-entry state, only the last one carries to the chunk's end, pairs
  // of different segments are zero (selects: no factor crosses a reset).
  const bool resets = kResets && a.reset != nullptr;
  const int seg_last = resets ? x.seg[C - 1] : 0;
  auto same_doc = [&](int r_, int c_) { return !resets || x.seg[r_] == x.seg[c_]; };
  const bool sees_entry = !resets || x.seg[tr] == 0, carries = !resets || x.seg[tr] == seg_last;
  auto load8 = [&](const float *p, float (&y)[8]) __attribute__((always_inline)) {
    const float4 u = *reinterpret_cast<const float4 *>(p);
    const float4 v = *reinterpret_cast<const float4 *>(p + 4);
    y[0] = u.x; y[1] = u.y; y[2] = u.z; y[3] = u.w; y[4] = v.x; y[5] = v.y; y[6] = v.z; y[7] = v.w;
  };
  // identity operands for the K-hat^T transpose: element (k, j) = [k == j + 16 h]
  FragH ident[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
#pragma unroll
    for (int e = 0; e < 8; ++e) ident[h].h[e] = (8 * lq + e == lr + 16 * h) ? f16(1.f) : f16(0.f);
  }

  // ---- operands of block I: scan operands, the shared column operand, the
  // row operands of the pair chain (fp32), the diagonal pair
  float yk[KS][8], yq[KS][8];
  f32x4 dG = {0.f, 0.f, 0.f, 0.f}, dL = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    const int ch0 = 32 * s + 8 * lq;
    float xk[8], xq[8], f0[8], g0[8], ei[8], hc[8];
    kt[s].to_float(xk);
    qt[s].to_float(xq);
    load8(f0t + I * DK + ch0, f0);
    load8(g0t + I * DK + ch0, g0);
    load8(eit + I * DK + ch0, ei);
    load8(hct + I * DK + ch0, hc);
    float ku[8], qu[8], kc[8], kbar[8], qbar[8], kh[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float p = lt[s][e], p0 = dpp_row_bcast<0>(p), p15 = dpp_row_bcast<15>(p);
      const float u = __builtin_amdgcn_exp2f(p - p0);  // exp(Lambda_t - Lambda_{16 I}) <= 1
      const float v = __builtin_amdgcn_exp2f(p15 - p); // exp(Lambda_{16 I + 15} - Lambda_t) <= 1
      const float k = xk[e] * mt, q = xq[e] * mt;       // tokens past T: zero rows
      ku[e] = k * u;
      qu[e] = q * u;
      yk[s][e] = ku[e] * f0[e];                        // exp(Lambda_t - Lambda_{16 I - 1})
      yq[s][e] = qu[e] * f0[e];
      kbar[e] = sees_entry ? ku[e] * g0[e] : 0.f;      // exp(Lambda_t)
      qbar[e] = sees_entry ? qu[e] * g0[e] : 0.f;
      kc[e] = k * v;                                   // column operand
      kh[e] = carries ? kc[e] * hc[e] : 0.f;           // exp(Lambda_{C-1} - Lambda_t)
    }
    const Split bc = make_frag<Split>(kc);
    if (I < NB - 1) lds_put_frag(colop, I * KS + s, bc);
    if (!wide) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        ku[e] *= ei[e];                                // exp(Lambda_t - Lambda_{16 I + 15})
        qu[e] *= ei[e];
      }
      mma(dG, bc, make_frag<Split>(ku));
      mma(dL, bc, make_frag<Split>(qu));
    }
    IO::put_plain8(x.tKB, I * KS + s, x.l, kbar);
    IO::put_plain8(x.tQB, I * KS + s, x.l, qbar);
    if constexpr (P::kF32) {
      x.put_channel_rows(x.tKH, I, s, kh, false);
    } else {
      const FragH fh = make_frag<FragH>(kh);
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        f32x4 t = {0.f, 0.f, 0.f, 0.f};
        mma(t, fh, ident[h]);                          // lane: channel 32 s + 16 h + lr, tokens 4 lq ..
        const float y[4] = {t[0], t[1], t[2], t[3]};
        IO::put_half4(x.tKH, (2 * s + h) * (C / 32) + I / 2, 16 * (2 * (I & 1) + (lq >> 1)) + lr, lq & 1, y);
      }
    }
    if (wide) {
      // Diagonal block entry by entry over this channel step: P of the
      // block's tokens through the wave's transpose buffer, the causal and
      // document masks before the exponential.  Lane: row lr, columns 4 lq ..
#pragma unroll
      for (int e = 0; e < 8; ++e) x.xb[(8 * lq + e) * kXbLd + lr] = lt[s][e];
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int cj = 4 * lq + q4, row = 16 * I + lr, col = 16 * I + cj;
        float sg = 0.f, sl = 0.f;
        if (lr >= cj && x.t0 + row < x.T && same_doc(row, col)) {
          const size_t rrow = x.tok(row) * x.row_stride + 32 * s, rcol = x.tok(col) * x.row_stride + 32 * s;
          for (int cl = 0; cl < 32; ++cl) {
            const float d = __builtin_amdgcn_exp2f(x.xb[cl * kXbLd + lr] - x.xb[cl * kXbLd + cj]);
            const float kcv = static_cast<float>(x.kbase[rcol + cl]);
            sg += static_cast<float>(x.kbase[rrow + cl]) * kcv * d;
            sl += static_cast<float>(x.qbase[rrow + cl]) * kcv * d;
          }
        }
        dG[q4] += sg;
        dL[q4] += sl;
      }
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    }
  }
  x.put_betas(bets, 0);                                // the solve's first beta head, read after later barriers
  // The helper's rows (wave I < 4 finishes row 7 - I), requested before the barrier
  const int Ih = NB - 1 - I;
  const bool helper = I < NB / 2;                      // uniform
  LaLane<TIn, KS, kGate> lah;
  if (helper) {
    lah.issue(x.la + x.tok(16 * Ih + lr) * x.la_row + (size_t)x.hk * G, lq, gs, G);
    x.load_rows(kt, x.kbase, Ih);
    x.load_rows(qt, x.qbase, Ih);
  }
  __syncthreads();                                     // column operands complete; factor tables dead

  // ---- pairs.  Lane: row 16 Ir + lr of G and L, columns 16 J + 4 lq ..
  float *gmat = x.ureg;
  auto put_pair = [&](int Ir, int J, const f32x4 &accG, const f32x4 &accL) __attribute__((always_inline)) {
    const int row = 16 * Ir + lr, c0 = 16 * J + 4 * lq;
    float g[4], lv[4];
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const bool keep = same_doc(row, c0 + q4);
      g[q4] = (keep && (Ir > J || lr > 4 * lq + q4)) ? accG[q4] : 0.f;
      lv[q4] = (keep && (Ir > J || lr >= 4 * lq + q4)) ? accL[q4] : 0.f;
    }
    *reinterpret_cast<float4 *>(gmat + row * (C + 4) + c0) = make_float4(g[0], g[1], g[2], g[3]);
    IO::put_half4(x.tL, Ir * (C / 32) + J / 2, 16 * (2 * (J & 1) + (lq >> 1)) + lr, lq & 1, lv);
  };
  put_pair(I, I, dG, dL);
  auto pair = [&](int Ir, int J) __attribute__((always_inline)) {
    f32x4 accG = {0.f, 0.f, 0.f, 0.f}, accL = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const Split bj = lds_get_frag<Split>(colop, J * KS + s);
      mma(accG, bj, make_frag<Split>(yk[s]));
      mma(accL, bj, make_frag<Split>(yq[s]));
    }
    put_pair(Ir, J, accG, accL);
  };
  auto decay = [&](int K) __attribute__((always_inline)) {   // pair (., K) -> (., K - 1)
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      float d[8];
      load8(dec + K * DK + 32 * s + 8 * lq, d);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        yk[s][e] *= d[e];
        yq[s][e] *= d[e];
      }
    }
  };
  const int jlo = I >= 3 ? I - 3 : 0;
  for (int J = I - 1; J >= jlo; --J) {
    pair(I, J);
    if (J > jlo) decay(J);
  }
  if (helper) {
    // row Ih from J = Ih - 4 down: row operand K_t exp(Lambda_t - Lambda_{16 (Ih - 3) - 1})
    const int jtop = Ih - 4, trh = 16 * Ih + lr;
    const float mh = (x.t0 + trh < x.T) ? 1.f : 0.f;
    bool unused = false;
    lah.get(lt, mh * kLog2e, lq, gs, G, unused);
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const int ch0 = 32 * s + 8 * lq;
      float oa[8], ob[8], xk[8], xq[8];
      load8(offt + Ih * DK + ch0, oa);
      load8(offt + (jtop + 1) * DK + ch0, ob);
      kt[s].to_float(xk);
      qt[s].to_float(xq);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float f = __builtin_amdgcn_exp2f(row_prefix16(lt[s][e]) + (oa[e] - ob[e]));
        yk[s][e] = xk[e] * mh * f;
        yq[s][e] = xq[e] * mh * f;
      }
    }
    for (int J = jtop; J >= 0; --J) {
      pair(Ih, J);
      if (J > 0) decay(J);
    }
  }
  x.zero_upper_L();
  x.template solve_store<kMode == 2 || kMode == 5>(gmat, x.smem, bets, true);
}

// Grid (N_c, H_k, B), one chunk per work group.  d_k <= 128: eight waves
// (C = 128: a 16-token row block per wave; two waves per SIMD hide each
// other's load, exponential and MFMA latencies); d_k = 256 keeps four, whose
// operand rows need the larger register file of a four-wave workgroup.
template <int DK>
constexpr int prep_block_threads() { return DK <= 128 ? 512 : 256; }
template <typename TIn, class P, int C, int DK>
__global__ __launch_bounds__(prep_block_threads<DK>()) void prep_block_kernel(ChunkArgs a) {
  extern __shared__ __align__(16) unsigned char smem_raw[];
  // C != 64 here: never the backward preparation
  prep_block_item<TIn, P, C, DK, prep_block_threads<DK>(), true>(a, blockIdx.x, blockIdx.y, blockIdx.z,
                                                            reinterpret_cast<float *>(smem_raw));
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
      prep_block_item<TIn, P, C, DK, 256>(a, c, hk, b, smem);
      __syncthreads();
    }
  }
}

#if !GDR_PREP_UNIT
bool prep_supported(int C, int d_k, int G) {
  if (!(C == 32 || C == 64 || C == 128)) return false;
  if (!(d_k == 64 || d_k == 128 || d_k == 256)) return false;
  // C = 64: the chunk-pivot kernel, and the 256-thread block-pivot kernel for
  // wide chunks; otherwise the block-pivot kernel, eight waves up to d_k = 128
  return (C == 64 || d_k > 128 ? prep_lds_bytes(C, d_k, G) : prep_block8_lds_bytes(C, d_k, G)) <= 160 * 1024;
}
#endif

template <class K>
static hipError_t set_lds(K kern, size_t /*lds*/) {
  return allow_full_lds(reinterpret_cast<const void *>(kern));
}

template <typename TIn, class P, int C, int DK>
static hipError_t launch_prep_t(const ChunkArgs &a, hipStream_t stream) {
  const size_t lds = prep_lds_bytes(C, DK, a.G);
  const dim3 grid(a.N_c, a.H_k, a.B);
  hipError_t e;
  if constexpr (C == 128 && DK <= 128) {
    if (a.bwd) return hipErrorInvalidValue;            // the backward pass prepares C = 64 chunks only
    const int md = a.solve != 0 ? (a.reset ? 5 : 2) : a.reset ? 3 : 0;
    auto pick = [&](auto g) {
      constexpr int kG = decltype(g)::value;
      if constexpr (P::kF32) {
        return a.solve != 0 ? prep_block128_kernel<TIn, P, DK, kG, 5> : prep_block128_kernel<TIn, P, DK, kG, 3>;
      } else {
        return md == 2   ? prep_block128_kernel<TIn, P, DK, kG, 2>
               : md == 5 ? prep_block128_kernel<TIn, P, DK, kG, 5>
               : md == 3 ? prep_block128_kernel<TIn, P, DK, kG, 3>
                         : prep_block128_kernel<TIn, P, DK, kG, 0>;
      }
    };
    auto block = a.G == DK  ? pick(std::integral_constant<int, kGatePerChannel>())
                 : a.G >= 8 ? pick(std::integral_constant<int, kGateGroupsVec>())
                            : pick(std::integral_constant<int, kGateGroupsFew>());
    const size_t lds_b = prep_block8_lds_bytes(C, DK, a.G);
    if ((e = set_lds(block, lds_b)) != hipSuccess) return e;
    hipLaunchKernelGGL(block, grid, dim3(512), lds_b, stream, a);
    return hipGetLastError();
  } else if constexpr (C != 64) {
    if (a.bwd) return hipErrorInvalidValue;            // the backward pass prepares C = 64 chunks only
    auto block = prep_block_kernel<TIn, P, C, DK>;
    constexpr int nth = prep_block_threads<DK>();
    const size_t lds_b = nth == 512 ? prep_block8_lds_bytes(C, DK, a.G) : lds;
    if ((e = set_lds(block, lds_b)) != hipSuccess) return e;
    hipLaunchKernelGGL(block, grid, dim3(nth), lds_b, stream, a);
    return hipGetLastError();
  } else {
  if (a.bwd && (a.solve != 0 || a.reset)) return hipErrorInvalidValue;   // backward: exact solve, plain layer
  // bf16 inputs get a variant per case; fp32 inputs (the checking mode) the
  // three general ones, which keeps the build short
  const int md = a.solve != 0 ? (a.reset ? 5 : 2) : a.bwd ? 1 : a.reset ? 3 : a.H_beta == a.H_k ? 4 : 0;
  auto pick = [&](auto g) {
    constexpr int kG = decltype(g)::value;
    if constexpr (P::kF32) {
      return a.solve != 0 ? prep_chunk_kernel<TIn, P, DK, kG, 5>
             : a.bwd      ? prep_chunk_kernel<TIn, P, DK, kG, 1>
                          : prep_chunk_kernel<TIn, P, DK, kG, 3>;
    } else {
      return md == 2   ? prep_chunk_kernel<TIn, P, DK, kG, 2>
             : md == 5 ? prep_chunk_kernel<TIn, P, DK, kG, 5>
             : md == 1 ? prep_chunk_kernel<TIn, P, DK, kG, 1>
             : md == 3 ? prep_chunk_kernel<TIn, P, DK, kG, 3>
             : md == 4 ? prep_chunk_kernel<TIn, P, DK, kG, 4>
                       : prep_chunk_kernel<TIn, P, DK, kG, 0>;
    }
  };
  auto chunk = a.G == DK  ? pick(std::integral_constant<int, kGatePerChannel>())
               : a.G >= 8 ? pick(std::integral_constant<int, kGateGroupsVec>())
                          : pick(std::integral_constant<int, kGateGroupsFew>());
  auto listed = prep_block_listed_kernel<TIn, P, C, DK>;
  const size_t chunk_lds = prep_chunk_lds_bytes(C, DK);
  if ((e = set_lds(chunk, chunk_lds)) != hipSuccess) return e;
  if ((e = set_lds(listed, lds)) != hipSuccess) return e;
  hipLaunchKernelGGL(chunk, grid, dim3(256), chunk_lds, stream, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  // wide-range chunks, if any: two work groups per CU (the LDS of the block
  // route allows two), at most 256 items each.  An odd group count: the
  // items of one chunk's key heads lie N_c apart, and N_c is often a power of
  // two, so a power-of-two count would hand a chunk with a document start in
  // it (every head of it marked) to N_c-divisible few groups in turn.
  const long n = (long)a.N_c * a.H_k * a.B;
  long groups = std::max(std::min(n, 511L), (n + 255) / 256);
  if (groups % 2 == 0) ++groups;
  hipLaunchKernelGGL(listed, dim3((unsigned)groups), dim3(256), lds, stream, a);
  return hipGetLastError();
  }
}

// kPart: which d_k a translation unit instantiates (0 every d_k, 1 only
// d_k = 128, 2 d_k in {64, 256}).
template <typename TIn, class P, int kPart>
static hipError_t launch_prep_dk(const ChunkArgs &a, hipStream_t s) {
  constexpr bool k128 = kPart != 2, kOther = kPart != 1;
  switch (a.C * 1000 + a.d_k) {
    case 32064: if constexpr (kOther) return launch_prep_t<TIn, P, 32, 64>(a, s); break;
    case 32128: if constexpr (k128) return launch_prep_t<TIn, P, 32, 128>(a, s); break;
    case 32256: if constexpr (kOther) return launch_prep_t<TIn, P, 32, 256>(a, s); break;
    case 64064: if constexpr (kOther) return launch_prep_t<TIn, P, 64, 64>(a, s); break;
    case 64128: if constexpr (k128) return launch_prep_t<TIn, P, 64, 128>(a, s); break;
    case 64256: if constexpr (kOther) return launch_prep_t<TIn, P, 64, 256>(a, s); break;
    case 128064: if constexpr (kOther) return launch_prep_t<TIn, P, 128, 64>(a, s); break;
    case 128128: if constexpr (k128) return launch_prep_t<TIn, P, 128, 128>(a, s); break;
    case 128256: if constexpr (kOther) return launch_prep_t<TIn, P, 128, 256>(a, s); break;
    default: break;
  }
  return hipErrorInvalidValue;
}

// The kernels are compiled in three translation units, so the prep build
// runs in parallel: this one (bf16 inputs with d_k = 128, and the
// dispatch), prep_f32.hip (fp32 inputs, GDR_PREP_UNIT 1) and
// prep_bf16x.hip (bf16 inputs with d_k 64 or 256, GDR_PREP_UNIT 2).
hipError_t launch_prep_f32(const ChunkArgs &a, hipStream_t stream);
hipError_t launch_prep_bf16x(const ChunkArgs &a, hipStream_t stream);
#if GDR_PREP_UNIT == 1
hipError_t launch_prep_f32(const ChunkArgs &a, hipStream_t stream) {
  return launch_prep_dk<float, PrecF32, 0>(a, stream);
}
#elif GDR_PREP_UNIT == 2
hipError_t launch_prep_bf16x(const ChunkArgs &a, hipStream_t stream) {
  return launch_prep_dk<bf16, PrecBF16, 2>(a, stream);
}
#else
hipError_t launch_prep(const ChunkArgs &a, bool in_bf16, hipStream_t stream) {
  if (!in_bf16) return launch_prep_f32(a, stream);
  if (a.d_k == 128) return launch_prep_dk<bf16, PrecBF16, 1>(a, stream);
  return launch_prep_bf16x(a, stream);
}
#endif

}  // namespace gdr
