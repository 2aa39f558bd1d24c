// Chunk size 16 on the 32-deep MFMA tiles: every 16-token chunk becomes a
// 32-token chunk whose second half is identity tokens (zero q, k, v, beta and
// log alpha: no decay, no erase, no write), and the C = 32 path runs on the
// padded sequence.  The state after each padded chunk equals the state after
// the 16-token chunk, and within a padded chunk the in-chunk matrices are
// those of the 16 real tokens bordered by zeros (G, L and beta vanish on the
// padding), so the exact solve, both Neumann forms and chunk-boundary
// momentum (Systolic Linear Attention, Table 2) act per 16 real tokens, as
// at C = 16.
//
// Real token t sits at padded position 32 (t / 16) + t % 16.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.hpp"

namespace gdr {

// pad: dst [B][Tp][units] from src [B][T][units], zero rows on the padding;
// unpad: dst [B][T][units] from src [B][Tp][units].
template <typename U>
__global__ __launch_bounds__(256) void pad_rows_kernel(U *dst, const U *src, int B, int T, int Tp, long long units,
                                                       int unpad) {
  const long long rows = (long long)B * (unpad ? T : Tp);
  const long long n = rows * units;
  for (long long i = blockIdx.x * 256LL + threadIdx.x; i < n; i += (long long)gridDim.x * 256) {
    const long long row = i / units, u = i - row * units;
    const long long b = row / (unpad ? T : Tp);
    const int t = (int)(row - b * (unpad ? T : Tp));
    if (unpad) {
      const int tp = 32 * (t / 16) + t % 16;
      dst[i] = src[(b * Tp + tp) * units + u];
    } else {
      const int real = 16 * (t / 32) + t % 32;
      const bool ok = (t % 32) < 16 && real < T;
      U z{};
      dst[i] = ok ? src[(b * T + real) * units + u] : z;
    }
  }
}

template <typename U>
static hipError_t launch_u(void *dst, const void *src, size_t row_bytes, int B, int T, int Tp, bool unpad,
                           hipStream_t s) {
  const long long units = (long long)(row_bytes / sizeof(U));
  const long long n = (long long)B * (unpad ? T : Tp) * units;
  if (n == 0) return hipSuccess;
  const long long blocks = (n + 255) / 256;
  const unsigned grid = (unsigned)(blocks < (1LL << 20) ? blocks : (1LL << 20));
  hipLaunchKernelGGL(pad_rows_kernel<U>, dim3(grid), dim3(256), 0, s, static_cast<U *>(dst),
                     static_cast<const U *>(src), B, T, Tp, units, unpad ? 1 : 0);
  return hipGetLastError();
}

hipError_t launch_pad_rows(void *dst, const void *src, size_t row_bytes, int B, int T, int Tp, bool unpad,
                           hipStream_t s) {
  const uintptr_t al = reinterpret_cast<uintptr_t>(dst) | reinterpret_cast<uintptr_t>(src) | row_bytes;
  if (al % 16 == 0) return launch_u<uint4>(dst, src, row_bytes, B, T, Tp, unpad, s);
  if (al % 4 == 0) return launch_u<uint32_t>(dst, src, row_bytes, B, T, Tp, unpad, s);
  if (al % 2 == 0) return launch_u<uint16_t>(dst, src, row_bytes, B, T, Tp, unpad, s);
  return launch_u<uint8_t>(dst, src, row_bytes, B, T, Tp, unpad, s);
}

}  // namespace gdr
