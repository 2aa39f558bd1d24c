// Device helpers shared by the gfx950 kernels: MFMA wrappers and operand
// fragments.
//
// MFMA tiles are 16x16 with a 32-deep contraction block.  For one wave64:
//   A operand (16 x 32): lane l holds row l%16, contraction indices
//                        8*(l/16) .. 8*(l/16)+7
//   B operand (32 x 16): lane l holds column l%16, the same 8 indices
//   D (16 x 16, fp32):   lane l holds column l%16, rows 4*(l/16) .. +3
// Any consistent assignment of contraction indices gives the same product,
// so the fp32 path (v_mfma_f32_16x16x4_f32, four indices per instruction)
// reuses the layout: instruction s takes index 8*(l/16)+s from every lane,
// and eight instructions cover the block.
//
// Precision.  An operand is a fragment of one of three kinds:
//   Plain  - eight bf16 values (round-to-nearest-even of the fp32 value);
//   Split  - hi = bf16(x), lo = bf16(x - hi): ~16 significant bits;
//   F32    - eight fp32 values for the fp32 MFMA.
// A product of two Split fragments costs three bf16 MFMAs (lo*hi, hi*lo,
// hi*hi; lo*lo is below fp32 accumulation noise), Split x Plain two, and
// Plain x Plain one.  Which operands must be Split is a numerical decision
// made per product in the kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdr {

typedef __bf16 bf16;
typedef bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16;
typedef f16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }
// The wave index, as a scalar: branches on it are uniform per wave.
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

__device__ __forceinline__ bf16 to_bf16(float x) { return static_cast<bf16>(x); }

// Loads of one input element as fp32 (bf16 decodes exactly).
__device__ __forceinline__ float ldf(const float *p) { return *p; }
__device__ __forceinline__ float ldf(const bf16 *p) { return static_cast<float>(*p); }

// Eight consecutive inputs as fp32.
__device__ __forceinline__ void ld8(const float *p, float (&x)[8]) {
  const float4 a = *reinterpret_cast<const float4 *>(p);
  const float4 b = *reinterpret_cast<const float4 *>(p + 4);
  x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
  x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
}
__device__ __forceinline__ void ld8(const bf16 *p, float (&x)[8]) {
  const bf16x8 v = *reinterpret_cast<const bf16x8 *>(p);
#pragma unroll
  for (int e = 0; e < 8; ++e) x[e] = static_cast<float>(v[e]);
}

__device__ __forceinline__ void st(float *p, float x) { *p = x; }
__device__ __forceinline__ void st(bf16 *p, float x) { *p = to_bf16(x); }

// --------------------------------------------------------------- raw loads
// Eight consecutive input elements kept in registers until use.
template <typename T> struct Raw8;
template <> struct Raw8<bf16> {
  uint4 v;
  __device__ __forceinline__ void load(const bf16 *p) { v = *reinterpret_cast<const uint4 *>(p); }
  __device__ __forceinline__ void zero() { v = make_uint4(0, 0, 0, 0); }
  __device__ __forceinline__ void store(bf16 *p) const { *reinterpret_cast<uint4 *>(p) = v; }
  __device__ __forceinline__ void to_float(float (&x)[8]) const {
    const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = __uint_as_float(u[i] << 16);
      x[2 * i + 1] = __uint_as_float(u[i] & 0xffff0000u);
    }
  }
};
template <> struct Raw8<float> {
  float4 a, b;
  __device__ __forceinline__ void load(const float *p) {
    a = *reinterpret_cast<const float4 *>(p);
    b = *reinterpret_cast<const float4 *>(p + 4);
  }
  __device__ __forceinline__ void zero() { a = b = make_float4(0.f, 0.f, 0.f, 0.f); }
  __device__ __forceinline__ void store(float *p) const {
    *reinterpret_cast<float4 *>(p) = a;
    *reinterpret_cast<float4 *>(p + 4) = b;
  }
  __device__ __forceinline__ void to_float(float (&x)[8]) const {
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
    x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
  }
};

// Value of the lane N places lower in the same 16-lane DPP row, 0 for the
// first N lanes of the row.
template <int N>
__device__ __forceinline__ float dpp_row_shr(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x110 + N, 0xf, 0xf, true));
}
// Lane N of each DPP row (16 lanes) broadcast to the whole row.
template <int N>
__device__ __forceinline__ float dpp_row_bcast(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x150 + N, 0xf, 0xf, false));
}
// Inclusive prefix sum over the 16 lanes of each DPP row (lanes 16 r .. 16 r + 15).
__device__ __forceinline__ float row_prefix16(float v) {
  v += dpp_row_shr<1>(v);
  v += dpp_row_shr<2>(v);
  v += dpp_row_shr<4>(v);
  v += dpp_row_shr<8>(v);
  return v;
}

// In-place prefix sum over rows of one column of a row-major LDS matrix
// (the cumulative log-decay Lambda_t = sum_{s<=t} log alpha_s of Systolic
// Linear Attention, Table 2), 16 rows at a time so the reads of a block are
// in flight together.
template <int C>
__device__ __forceinline__ void prefix_column(float *col, int ld) {
  float acc = 0.f;
#pragma unroll
  for (int t0 = 0; t0 < C; t0 += 16) {
    float x[16];
#pragma unroll
    for (int t = 0; t < 16; ++t) x[t] = col[(t0 + t) * ld];
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      acc += x[t];
      col[(t0 + t) * ld] = acc;
    }
  }
}

// ----------------------------------------------------------------- fragments
struct FragS {            // split bf16 hi + lo
  bf16x8 h, l;
};
struct FragF {            // fp32
  float v[8];
};
struct FragH {            // plain fp16
  f16x8 h;
};
struct FragHS {           // split fp16 hi + lo
  f16x8 h, l;
};

template <class F> __device__ __forceinline__ F make_frag(const float (&x)[8]);

template <> __device__ __forceinline__ FragS make_frag<FragS>(const float (&x)[8]) {
  FragS f;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const bf16 h = to_bf16(x[e]);
    f.h[e] = h;
    f.l[e] = to_bf16(x[e] - static_cast<float>(h));
  }
  return f;
}
template <> __device__ __forceinline__ FragH make_frag<FragH>(const float (&x)[8]) {
  FragH f;
#pragma unroll
  for (int e = 0; e < 8; ++e) f.h[e] = static_cast<f16>(x[e]);
  return f;
}
template <> __device__ __forceinline__ FragHS make_frag<FragHS>(const float (&x)[8]) {
  FragHS f;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const f16 h = static_cast<f16>(x[e]);
    f.h[e] = h;
    f.l[e] = static_cast<f16>(x[e] - static_cast<float>(h));
  }
  return f;
}
template <> __device__ __forceinline__ FragF make_frag<FragF>(const float (&x)[8]) {
  FragF f;
#pragma unroll
  for (int e = 0; e < 8; ++e) f.v[e] = x[e];
  return f;
}

__device__ __forceinline__ f32x4 mfma_bf16(const bf16x8 &a, const bf16x8 &b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_f16(const f16x8 &a, const f16x8 &b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_f32(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ void mma(f32x4 &c, const FragS &a, const FragS &b) {
  c = mfma_bf16(a.l, b.h, c);
  c = mfma_bf16(a.h, b.l, c);
  c = mfma_bf16(a.h, b.h, c);
}
__device__ __forceinline__ void mma(f32x4 &c, const FragH &a, const FragH &b) {
  c = mfma_f16(a.h, b.h, c);
}
__device__ __forceinline__ void mma(f32x4 &c, const FragH &a, const FragHS &b) {
  c = mfma_f16(a.h, b.l, c);
  c = mfma_f16(a.h, b.h, c);
}
__device__ __forceinline__ void mma(f32x4 &c, const FragF &a, const FragF &b) {
#pragma unroll
  for (int s = 0; s < 8; ++s) c = mfma_f32(a.v[s], b.v[s], c);
}

// Precision policies.  Each kernel names, per operand, whether it needs the
// Split kind; the fp32 policy maps every kind to FragF.  Split bf16 pairs
// (bf16 range, about 16 significant bits) for the Gram of the prep kernels.
struct PrecBF16 {
  using Split = FragS;
  static constexpr bool kF32 = false;
};
struct PrecF32 {
  using Plain = FragF;
  using Split = FragF;
  static constexpr bool kF32 = true;
};
// fp16 operands for the state scan of bf16 inputs: the prepared chunk
// operands are single fp16 (11 significant bits, 2 bytes), the state and the
// chunk intermediates split fp16 pairs.
struct PrecF16 {
  using Plain = FragH;
  using Split = FragHS;
  static constexpr bool kF32 = false;
};

// LDS storage of an operand that is read back as B fragments: element (n, k)
// of an N x K operand (column n of the B matrix, contraction index k) lives at
// n * ld + k, so a fragment is eight consecutive values.  fp16 policy: hi and
// lo planes; fp32 policy: one fp32 plane (same bytes).
template <class P> struct OperandLds;

template <> struct OperandLds<PrecF16> {
  f16 *hi;
  f16 *lo;
  int ld;
  static constexpr int kBytesPerElem = 4;
  __device__ __forceinline__ void init(void *base, int n_rows, int ld_) {
    hi = reinterpret_cast<f16 *>(base);
    lo = hi + n_rows * ld_;
    ld = ld_;
  }
  __device__ __forceinline__ void put4(int n, int k, const f32x4 &x) {
    typedef f16 f16x4 __attribute__((ext_vector_type(4)));
    f16x4 h, l;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      h[r] = static_cast<f16>(x[r]);
      l[r] = static_cast<f16>(x[r] - static_cast<float>(h[r]));
    }
    *reinterpret_cast<f16x4 *>(hi + n * ld + k) = h;
    *reinterpret_cast<f16x4 *>(lo + n * ld + k) = l;
  }
  __device__ __forceinline__ FragHS get(int n, int k) const {
    FragHS f;
    f.h = *reinterpret_cast<const f16x8 *>(hi + n * ld + k);
    f.l = *reinterpret_cast<const f16x8 *>(lo + n * ld + k);
    return f;
  }
  // the hi plane only: the operand rounded once to fp16
  __device__ __forceinline__ FragH get_hi(int n, int k) const {
    FragH f;
    f.h = *reinterpret_cast<const f16x8 *>(hi + n * ld + k);
    return f;
  }
};

template <> struct OperandLds<PrecF32> {
  float *v;
  int ld;
  static constexpr int kBytesPerElem = 4;
  __device__ __forceinline__ void init(void *base, int /*n_rows*/, int ld_) {
    v = reinterpret_cast<float *>(base);
    ld = ld_;
  }
  // four consecutive k for one n (D-layout rows of one column)
  __device__ __forceinline__ void put4(int n, int k, const f32x4 &x) {
    *reinterpret_cast<f32x4 *>(v + n * ld + k) = x;
  }
  __device__ __forceinline__ FragF get_hi(int n, int k) const { return get(n, k); }   // fp32: the operand itself
  __device__ __forceinline__ FragF get(int n, int k) const {
    FragF f;
    const float4 a = *reinterpret_cast<const float4 *>(v + n * ld + k);
    const float4 b = *reinterpret_cast<const float4 *>(v + n * ld + k + 4);
    f.v[0] = a.x; f.v[1] = a.y; f.v[2] = a.z; f.v[3] = a.w;
    f.v[4] = b.x; f.v[5] = b.y; f.v[6] = b.z; f.v[7] = b.w;
    return f;
  }
};

// LDS storage of the state operand S^T (B fragments, same addressing as
// OperandLds): one fp16 plane for the fp16 policy -- the state itself stays
// in fp32 accumulators, only the operand copy of each chunk is rounded once
// -- and the fp32 plane for the fp32 policy.
template <class P> struct StateLds;
template <> struct StateLds<PrecF16> {
  f16 *v;
  int ld;
  __device__ __forceinline__ void init(void *base, int /*n_rows*/, int ld_) {
    v = reinterpret_cast<f16 *>(base);
    ld = ld_;
  }
  __device__ __forceinline__ void put4(int n, int k, const f32x4 &x) {
    typedef f16 f16x4 __attribute__((ext_vector_type(4)));
    f16x4 h;
#pragma unroll
    for (int r = 0; r < 4; ++r) h[r] = static_cast<f16>(x[r]);
    *reinterpret_cast<f16x4 *>(v + n * ld + k) = h;
  }
  __device__ __forceinline__ FragH get(int n, int k) const {
    FragH f;
    f.h = *reinterpret_cast<const f16x8 *>(v + n * ld + k);
    return f;
  }
};
template <> struct StateLds<PrecF32> : OperandLds<PrecF32> {};

// ------------------------------------------------------------ workspace tiles
// Fragment-major tiles: an R x K tile (R a multiple of 16, K of 32) is stored
// as (R/16) x (K/32) blocks in row-block-major order; block (i, j) holds its
// 16 x 32 elements as 64 fragments of eight consecutive columns, fragment
// f = 16 q + r being row 16 i + r, columns 32 j + 8 q .. + 7: exactly the
// operand lane f of a 16x16x32 MFMA reads, so a wave loads a block as one
// contiguous run.  fp16 tiles: 1 KiB blocks, fragment f at byte 16 f; fp32
// tiles: 2 KiB blocks, fragment f at byte 32 f.
template <class P> struct TileIO;

// Tiles are written with non-temporal stores.  The scan reads them from HBM
// right after prep: with ordinary stores, prep leaves the L2 full of dirty
// workspace lines, and the scan's start competes with their write-back
// (measured: the scan runs 4 % faster on the per-channel workload and 12 %
// on the scalar-gate one).
// fp16 tiles (operands prepared from bf16 inputs): plain only, 1 KiB blocks.
template <> struct TileIO<PrecF16> {
  __device__ static unsigned char *at(void *t, int blk, int f) {
    return static_cast<unsigned char *>(t) + blk * 1024 + f * 16;
  }
  __device__ static void put_plain8(void *t, int blk, int f, const float (&x)[8]) {
    f16x8 h;
#pragma unroll
    for (int e = 0; e < 8; ++e) h[e] = static_cast<f16>(x[e]);
    __builtin_nontemporal_store(h, reinterpret_cast<f16x8 *>(at(t, blk, f)));
  }
  // half h (elements 4 h .. 4 h + 3) of a fragment
  __device__ static void put_half4(void *t, int blk, int f, int h, const float (&x)[4]) {
    typedef f16 f16x4 __attribute__((ext_vector_type(4)));
    f16x4 v;
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = static_cast<f16>(x[e]);
    __builtin_nontemporal_store(v, reinterpret_cast<f16x4 *>(at(t, blk, f) + 8 * h));
  }
  __device__ static FragH get_plain(const void *t, int blk, int f) {
    FragH v;
    v.h = *reinterpret_cast<const f16x8 *>(at(const_cast<void *>(t), blk, f));
    return v;
  }
};

template <> struct TileIO<PrecF32> {
  __device__ static float *at(void *t, int blk, int f) {
    return reinterpret_cast<float *>(static_cast<unsigned char *>(t) + blk * 2048 + f * 32);
  }
  __device__ static void put_plain8(void *t, int blk, int f, const float (&x)[8]) {
    float *p = at(t, blk, f);
    __builtin_nontemporal_store(f32x4{x[0], x[1], x[2], x[3]}, reinterpret_cast<f32x4 *>(p));
    __builtin_nontemporal_store(f32x4{x[4], x[5], x[6], x[7]}, reinterpret_cast<f32x4 *>(p + 4));
  }
  __device__ static void put_half4(void *t, int blk, int f, int h, const float (&x)[4]) {
    __builtin_nontemporal_store(f32x4{x[0], x[1], x[2], x[3]}, reinterpret_cast<f32x4 *>(at(t, blk, f) + 4 * h));
  }
  __device__ static FragF get_plain(const void *t, int blk, int f) {
    const float *p = at(const_cast<void *>(t), blk, f);
    const float4 a = *reinterpret_cast<const float4 *>(p);
    const float4 b = *reinterpret_cast<const float4 *>(p + 4);
    FragF v;
    v.v[0] = a.x; v.v[1] = a.y; v.v[2] = a.z; v.v[3] = a.w;
    v.v[4] = b.x; v.v[5] = b.y; v.v[6] = b.z; v.v[7] = b.w;
    return v;
  }
};

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

// Lower-triangular chunk operands (diag(beta) A_c and L_c, and the reversed
// transposes the backward pass uses): of their 16 x 32 operand blocks (I, s)
// (row block I, contraction step s) only those with s <= I / 2 are nonzero.
// Their number, and the position of block (I, s) among them in row-major
// order.
__host__ __device__ constexpr int tri_blocks(int nb) { return (nb / 2) * (nb / 2 + 1); }
__device__ __forceinline__ int tri_index(int I, int s) {
  const int m = I >> 1;
  return ((I & 1) ? (m + 1) * (m + 1) : m * (m + 1)) + s;
}

}  // namespace gdr
