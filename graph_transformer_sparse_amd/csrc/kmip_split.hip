// Split-precision rows for the fp32 entry points.
//
// Page "k-Maximum Inner Product Attention for Graph Transformers and the
// Expressive Power of GraphGPS", Tables 15 and 16: k-MIP attention is timed
// there with fp32 inputs and arithmetic.  The matrix cores of gfx950 take
// bf16 (8 significant bits), so an fp32 inner product is rebuilt from bf16
// terms: x = hi + lo + r with hi = bf16(x), lo = bf16(x - hi) (x - hi is exact
// in fp32), |lo| <= 2^-9 |x| and |r| <= 2^-18 |x|.  Then
//
//   q.k = q_hi.k_hi + q_hi.k_lo + q_lo.k_hi + (dropped terms, ~3 * 2^-18 relative),
//
// and the three kept products are one inner product of rows three times as
// long: q3 = [q_hi | q_hi | q_lo], k3 = [k_hi | k_lo | k_hi].  Every bf16
// product is exact in the fp32 MFMA accumulator, so the scan's score error is
// about (3 * 2^-18 + 3d * 2^-24) * sum_c |q_c k_c| at most (dropped terms, then
// fp32 accumulation of 3d products): near fp32 rounding, where one bf16
// rounding of q and k would cost ~2^-8.
//
// The split is a streaming pass (4 bytes read, 6 written per element and
// tensor).  One thread handles 8 consecutive elements of one row.
#include "kmip_internal.h"

namespace kmip {
namespace {

// fp32 -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t bf16_rne(float x) {
  const uint32_t u = __float_as_uint(x);
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// blockIdx.y = 0: q rows -> [hi | hi | lo]; 1: k rows -> [hi | lo | hi].
template <int D>
__global__ __launch_bounds__(256) void split_rows_kernel(const float* __restrict__ q,
                                                         const float* __restrict__ k,
                                                         int64_t rows, uint16_t* __restrict__ q3,
                                                         uint16_t* __restrict__ k3) {
  constexpr int G = D / 8;                         // 8-element groups per row
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= rows * G) return;
  const bool is_k = blockIdx.y != 0;
  const int64_t r = t / G;
  const int c = (int)(t % G) * 8;
  const float4* src = reinterpret_cast<const float4*>((is_k ? k : q) + r * D + c);
  const float4 a = src[0], b = src[1];
  const float x[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
  uint32_t hw[4], lw[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    uint32_t h2[2], l2[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const float v = x[2 * e + u];
      h2[u] = bf16_rne(v);
      l2[u] = bf16_rne(v - __uint_as_float(h2[u] << 16));
    }
    hw[e] = h2[0] | (h2[1] << 16);
    lw[e] = l2[0] | (l2[1] << 16);
  }
  const uint4 hi = make_uint4(hw[0], hw[1], hw[2], hw[3]);
  const uint4 lo = make_uint4(lw[0], lw[1], lw[2], lw[3]);
  uint16_t* dst = (is_k ? k3 : q3) + r * (3 * D) + c;
  *reinterpret_cast<uint4*>(dst) = hi;
  *reinterpret_cast<uint4*>(dst + D) = is_k ? lo : hi;
  *reinterpret_cast<uint4*>(dst + 2 * D) = is_k ? hi : lo;
}

}  // namespace

hipError_t launch_split_rows(const float* q, const float* k, int64_t rows, int d, uint16_t* q3,
                             uint16_t* k3, hipStream_t s) {
  const dim3 grid((unsigned)ceil_div(rows * (d / 8), 256), 2);
  if (d == 32)
    hipLaunchKernelGGL(split_rows_kernel<32>, grid, dim3(256), 0, s, q, k, rows, q3, k3);
  else if (d == 64)
    hipLaunchKernelGGL(split_rows_kernel<64>, grid, dim3(256), 0, s, q, k, rows, q3, k3);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace kmip
