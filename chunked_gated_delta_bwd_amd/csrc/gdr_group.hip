// Grouped heads: q and k carry Hk heads, each read by G = H / Hk consecutive value
// heads, so the gradient of a key head's q (or k) row is the sum of what its G value
// heads contribute (FlashQLA GDN overview, section 4: its benchmarks name key and value
// head counts apart, hk and hv, and its tests cover GQA).  The gradient kernels
// write those contributions per value head, [tokens][H][K]; this kernel sums each
// group into the [tokens][Hk][K] output.
//
// Plain streaming work, bound by HBM: every lane owns eight consecutive channels of
// one (token, key head) row, reads its G source rows (contiguous, K apart) with one
// 16-byte (bf16) or two 16-byte (fp32) loads each, adds in fp32 in head order and
// stores once in the output dtype.
#include <hip/hip_runtime.h>

#include "gdr_device.h"
#include "gdr_internal.h"

namespace gdr {

template <typename TIO>
__global__ __launch_bounds__(256) void k_group_sum(const void* __restrict__ src, void* __restrict__ dst,
                                                    int64_t n8, int Hk, int K, int G) {
  const int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (i >= n8) return;
  const int64_t e = i * 8;                       // first output element of this lane
  const int64_t row = e / K;                     // (token, key head) row: token row / Hk, head row % Hk
  const int c = int(e - row * K);
  const int64_t t = row / Hk;
  const int j = int(row - t * Hk);
  const int64_t s0 = (t * int64_t(Hk) * G + int64_t(j) * G) * K + c;   // value head j G of token t
  float acc[8], x[8];
  IO<TIO>::load8(src, s0, acc);
  for (int h = 1; h < G; ++h) {
    IO<TIO>::load8(src, s0 + int64_t(h) * K, x);
#pragma unroll
    for (int m = 0; m < 8; ++m) acc[m] += x[m];
  }
  IO<TIO>::store8(dst, e, acc);
}

int launch_group_sum(const Params& p, const void* src, void* dst, void* stream) {
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  const int64_t n8 = int64_t(p.T) * p.Hk * p.K / 8;
  if (n8 == 0) return 0;
  const dim3 grid(unsigned((n8 + 255) / 256));
  if (p.dtype == GDR_BF16) k_group_sum<bf16><<<grid, 256, 0, s>>>(src, dst, n8, p.Hk, p.K, p.G);
  else k_group_sum<float><<<grid, 256, 0, s>>>(src, dst, n8, p.Hk, p.K, p.G);
  return static_cast<int>(hipGetLastError());
}

}  // namespace gdr
