// Output epilogue of the Systolic Linear Attention layer (section 2.3, the
// token-level recurrence box): each value head's readout is normalised on
// its own and gated by the sigmoid of its output-gate slice,
//   y = sigmoid(z) (.) o / sqrt(mean(o^2) + eps) (.) w,
// the mean over the d_v entries of one (batch, token, value head) row, w an
// optional per-channel scale.  When d_v is 32, 64, 128 or 256, a lane holds
// four consecutive elements of a row (one 16-byte fp32 or 8-byte bf16 access
// each for o, z and y, o read once) and d_v / 4 lanes share a row, several
// rows to a wave; the sum of squares is reduced over those lanes.  Other
// widths take one wave per row.  y may alias o: a lane rewrites only
// elements it has already read.
#include "common.hpp"
#include "kernels.hpp"

namespace gdr {

constexpr int kNormRowsPerGroup = 4;

template <typename TO, typename TZ>
__global__ __launch_bounds__(64 * kNormRowsPerGroup) void gated_rmsnorm_kernel(const TO *o, const TZ *z,
                                                                                const float *w, float eps, TO *y,
                                                                                long long rows, int d_v) {
  const long long row = (long long)blockIdx.x * kNormRowsPerGroup + (threadIdx.x >> 6);
  if (row >= rows) return;
  const int l = lane_id();
  const TO *orow = o + row * d_v;
  const TZ *zrow = z + row * d_v;
  TO *yrow = y + row * d_v;
  float ss = 0.f;
  for (int i = l; i < d_v; i += kWave) {
    const float x = ldf(orow + i);
    ss += x * x;
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) ss += __shfl_xor(ss, m);
  const float inv = 1.f / sqrtf(ss / (float)d_v + eps);
  for (int i = l; i < d_v; i += kWave) {
    const float x = ldf(orow + i);
    const float gate = 1.f / (1.f + __expf(-ldf(zrow + i)));
    st(yrow + i, gate * (x * inv) * (w ? w[i] : 1.f));
  }
}

// Four consecutive elements as fp32 and back.
__device__ __forceinline__ void ld4(const float *p, float (&x)[4]) {
  const float4 v = *reinterpret_cast<const float4 *>(p);
  x[0] = v.x; x[1] = v.y; x[2] = v.z; x[3] = v.w;
}
__device__ __forceinline__ void ld4(const bf16 *p, float (&x)[4]) {
  const uint2 v = *reinterpret_cast<const uint2 *>(p);
  x[0] = __uint_as_float(v.x << 16); x[1] = __uint_as_float(v.x & 0xffff0000u);
  x[2] = __uint_as_float(v.y << 16); x[3] = __uint_as_float(v.y & 0xffff0000u);
}
__device__ __forceinline__ void st4(float *p, const float (&x)[4]) {
  *reinterpret_cast<float4 *>(p) = make_float4(x[0], x[1], x[2], x[3]);
}
__device__ __forceinline__ void st4(bf16 *p, const float (&x)[4]) {
  typedef bf16 bf16x4 __attribute__((ext_vector_type(4)));
  bf16x4 v;
#pragma unroll
  for (int e = 0; e < 4; ++e) v[e] = to_bf16(x[e]);
  *reinterpret_cast<bf16x4 *>(p) = v;
}

// LPR = d_v / 4 lanes per row (8 .. 64), 64 / LPR rows per wave, four waves
template <typename TO, typename TZ, int LPR>
__global__ __launch_bounds__(256) void gated_rmsnorm4_kernel(const TO *o, const TZ *z, const float *w, float eps, TO *y,
                                                             long long rows) {
  constexpr int DV = 4 * LPR, RPW = 64 / LPR;
  const int l = lane_id();
  const long long row = ((long long)blockIdx.x * 4 + (threadIdx.x >> 6)) * RPW + l / LPR;
  const bool ok = row < rows;
  const long long r = ok ? row : rows - 1;            // every lane joins the reduction
  const int c = 4 * (l % LPR);
  float x[4], g[4];
  ld4(o + r * DV + c, x);
  ld4(z + r * DV + c, g);
  float ss = x[0] * x[0] + x[1] * x[1] + x[2] * x[2] + x[3] * x[3];
#pragma unroll
  for (int m = LPR / 2; m >= 1; m >>= 1) ss += __shfl_xor(ss, m);
  const float inv = 1.f / sqrtf(ss / (float)DV + eps);
  float sc[4] = {1.f, 1.f, 1.f, 1.f};
  if (w) {                                              // the weight is only 4-byte aligned
#pragma unroll
    for (int e = 0; e < 4; ++e) sc[e] = w[c + e];
  }
  float out[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) out[e] = (1.f / (1.f + __expf(-g[e]))) * (x[e] * inv) * sc[e];
  if (ok) st4(y + r * DV + c, out);
}

hipError_t launch_gated_rmsnorm(const void *o, const void *z, const float *weight, float eps, void *y,
                                long long rows, int d_v, bool o_bf16, bool z_bf16, hipStream_t stream) {
  if (d_v == 32 || d_v == 64 || d_v == 128 || d_v == 256) {
    const long long per_group = 4LL * (64 / (d_v / 4));   // rows per work group
    const dim3 g4((unsigned)((rows + per_group - 1) / per_group)), b4(256);
#define GDR_NORM4(TO, TZ, LPR)                                                                                       \
  hipLaunchKernelGGL((gated_rmsnorm4_kernel<TO, TZ, LPR>), g4, b4, 0, stream, static_cast<const TO *>(o),           \
                     static_cast<const TZ *>(z), weight, eps, static_cast<TO *>(y), rows)
#define GDR_NORM4_DV(TO, TZ)                         \
  switch (d_v) {                                     \
    case 32: GDR_NORM4(TO, TZ, 8); break;            \
    case 64: GDR_NORM4(TO, TZ, 16); break;           \
    case 128: GDR_NORM4(TO, TZ, 32); break;          \
    default: GDR_NORM4(TO, TZ, 64); break;           \
  }
    if (o_bf16) {
      if (z_bf16) GDR_NORM4_DV(bf16, bf16) else GDR_NORM4_DV(bf16, float)
    } else {
      if (z_bf16) GDR_NORM4_DV(float, bf16) else GDR_NORM4_DV(float, float)
    }
#undef GDR_NORM4_DV
#undef GDR_NORM4
    return hipGetLastError();
  }
  const dim3 grid((unsigned)((rows + kNormRowsPerGroup - 1) / kNormRowsPerGroup)), block(64 * kNormRowsPerGroup);
#define GDR_NORM(TO, TZ)                                                                                     \
  hipLaunchKernelGGL((gated_rmsnorm_kernel<TO, TZ>), grid, block, 0, stream, static_cast<const TO *>(o),     \
                     static_cast<const TZ *>(z), weight, eps, static_cast<TO *>(y), rows, d_v)
  if (o_bf16) {
    if (z_bf16) GDR_NORM(bf16, bf16); else GDR_NORM(bf16, float);
  } else {
    if (z_bf16) GDR_NORM(float, bf16); else GDR_NORM(float, float);
  }
#undef GDR_NORM
  return hipGetLastError();
}

}  // namespace gdr
