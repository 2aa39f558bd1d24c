// Output epilogue of the Systolic Linear Attention layer (section 2.3, the
// token-level recurrence box): each value head's readout is normalised on
// its own and gated by the sigmoid of its output-gate slice,
//   y = sigmoid(z) (.) o / sqrt(mean(o^2) + eps) (.) w,
// the mean over the d_v entries of one (batch, token, value head) row, w an
// optional per-channel scale.  One wave per row: the sum of squares is
// reduced across the wave, then every lane scales its own elements.  y may
// alias o: a lane rewrites only elements it has already read.
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

hipError_t launch_gated_rmsnorm(const void *o, const void *z, const float *weight, float eps, void *y,
                                long long rows, int d_v, bool o_bf16, bool z_bf16, hipStream_t stream) {
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
