// Softmax over the selected scores, gather of the selected rows and the
// weighted sums: the forward output and the query side of the backward.
//
// Page "k-Maximum Inner Product Attention for Graph Transformers and the
// Expressive Power of GraphGPS", Abstract: after the top-k selection the
// output of a query is the softmax-weighted sum of the value rows of its
// selected keys.  The backward follows from that definition with the
// selection held fixed (gradients flow through the selected entries only).
//
// These kernels are bandwidth bound (a handful of flops per gathered byte).
// A query row (node, head) is handled by 16 lanes; each lane owns d/16
// consecutive columns, so one gathered bf16 row is a single 64- or 128-byte
// coalesced segment.  Index and score rows are read once per row group and
// broadcast with 16-lane shuffles.
#include "kmip_internal.h"

namespace kmip {
namespace {

constexpr int ROWS_PER_BLOCK = 16;          // 256 threads, 16 lanes per row
constexpr int MAXK = 64;

template <int EPL>
struct Cols;                                 // EPL bf16 values of one row
template <>
struct Cols<2> {
  static __device__ __forceinline__ void load(const uint16_t* p, float* x) {
    const uint32_t w = *reinterpret_cast<const uint32_t*>(p);
    x[0] = __uint_as_float(w << 16);
    x[1] = __uint_as_float(w & 0xffff0000u);
  }
};
template <>
struct Cols<4> {
  static __device__ __forceinline__ void load(const uint16_t* p, float* x) {
    const uint2 w = *reinterpret_cast<const uint2*>(p);
    x[0] = __uint_as_float(w.x << 16);
    x[1] = __uint_as_float(w.x & 0xffff0000u);
    x[2] = __uint_as_float(w.y << 16);
    x[3] = __uint_as_float(w.y & 0xffff0000u);
  }
};

template <int EPL>
__device__ __forceinline__ void load_cols_f32(const float* p, float* x) {
  if constexpr (EPL == 2) {
    const float2 t = *reinterpret_cast<const float2*>(p);
    x[0] = t.x;
    x[1] = t.y;
  } else {
    const float4 t = *reinterpret_cast<const float4*>(p);
    x[0] = t.x;
    x[1] = t.y;
    x[2] = t.z;
    x[3] = t.w;
  }
}

template <int EPL>
__device__ __forceinline__ void store_cols(float* p, const float* x) {
  if constexpr (EPL == 2) {
    *reinterpret_cast<float2*>(p) = make_float2(x[0], x[1]);
  } else {
    *reinterpret_cast<float4*>(p) = make_float4(x[0], x[1], x[2], x[3]);
  }
}

__device__ __forceinline__ float sum16(float x) {
#pragma unroll
  for (int o = 8; o >= 1; o >>= 1) x += __shfl_xor(x, o, 16);
  return x;
}

// out[row] = sum_t softmax(score[row])_t * V[idx[row][t]]
template <int D>
__global__ __launch_bounds__(256) void gather_av_kernel(
    const uint16_t* __restrict__ V, int64_t NH, int H, int topk,
    const int32_t* __restrict__ idx, const float* __restrict__ score,
    float* __restrict__ out) {
  constexpr int EPL = D / 16;
  const int l16 = threadIdx.x & 15;
  const int64_t row = (int64_t)blockIdx.x * ROWS_PER_BLOCK + (threadIdx.x >> 4);
  if (row >= NH) return;                    // whole 16-lane groups leave together
  const int h = (int)(row % H);
  const int32_t* ir = idx + row * topk;
  const float* sr = score + row * topk;

  // Lane l16 holds entries l16, l16+16, ... of the row.
  int jv[MAXK / 16];
  float sv[MAXK / 16];
#pragma unroll
  for (int c = 0; c < MAXK / 16; ++c) {
    const int t = c * 16 + l16;
    jv[c] = t < topk ? ir[t] : -1;
    sv[c] = t < topk ? sr[t] : 0.f;
  }
  const float m = __shfl(sv[0], 0, 16);     // best score: entries are sorted
  float acc[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) acc[e] = 0.f;
  float z = 0.f;
#pragma unroll
  for (int c = 0; c < MAXK / 16; ++c) {
    if (c * 16 >= topk) break;
    const int tn = topk - c * 16 < 16 ? topk - c * 16 : 16;

    for (int u = 0; u < tn; ++u) {
      const int j = __shfl(jv[c], u, 16);
      if (j >= 0) {
        const float w = __expf(__shfl(sv[c], u, 16) - m);
        float x[EPL];
        Cols<EPL>::load(V + ((int64_t)j * H + h) * D + l16 * EPL, x);
        z += w;
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[e] = fmaf(w, x[e], acc[e]);
      }
    }
  }
  const float inv = 1.f / z;
#pragma unroll
  for (int e = 0; e < EPL; ++e) acc[e] *= inv;
  store_cols<EPL>(out + row * D + l16 * EPL, acc);
}

// Query side of the backward.  p = softmax(score), dp_t = dO . v_t,
// D = sum p dp, ds_t = p_t (dp_t - D), dq = sum ds_t k_t.  Writes dq and
// pairs[row*topk + t] = (p_t, ds_t) (zeros on unused slots).
//
// dp_t - D cancels when one weight dominates (p_0 -> 1), so the weights are
// normalised and dp, D, ds and dq are carried in fp64: the products of fp32
// dO and bf16 v are exact in fp64, and an fp32 p_0 alone would already carry
// an absolute error of ~6e-8.  The exponentials stay fp32 (each w_t is
// relatively accurate, which keeps p_0 = 1/Z accurate in fp64).
__device__ __forceinline__ double sum16d(double x) {
#pragma unroll
  for (int o = 8; o >= 1; o >>= 1) x += __shfl_xor(x, o, 16);
  return x;
}

template <int D>
__global__ __launch_bounds__(256) void bwd_query_kernel(
    const uint16_t* __restrict__ Kt, const uint16_t* __restrict__ V, int64_t NH, int H,
    int topk, const int32_t* __restrict__ idx, const float* __restrict__ score,
    const float* __restrict__ dout, float* __restrict__ dq, float2* __restrict__ pairs) {
  constexpr int EPL = D / 16;
  const int l16 = threadIdx.x & 15;
  const int64_t row = (int64_t)blockIdx.x * ROWS_PER_BLOCK + (threadIdx.x >> 4);
  if (row >= NH) return;
  const int h = (int)(row % H);
  const int32_t* ir = idx + row * topk;
  const float* sr = score + row * topk;

  int jv[MAXK / 16];
  float sv[MAXK / 16];
#pragma unroll
  for (int c = 0; c < MAXK / 16; ++c) {
    const int t = c * 16 + l16;
    jv[c] = t < topk ? ir[t] : -1;
    sv[c] = t < topk ? sr[t] : 0.f;
  }
  float g[EPL];
  load_cols_f32<EPL>(dout + row * D + l16 * EPL, g);
  const float m = __shfl(sv[0], 0, 16);

  // Pass 1: weights w_t and dp_t; lane (t % 16) keeps entry t.
  double wv[MAXK / 16], dpv[MAXK / 16];
  double z = 0.0, dsum = 0.0;
#pragma unroll
  for (int c = 0; c < MAXK / 16; ++c) {
    wv[c] = 0.0;
    dpv[c] = 0.0;
    if (c * 16 < topk) {
      const int tn = topk - c * 16 < 16 ? topk - c * 16 : 16;
      for (int u = 0; u < tn; ++u) {
        const int j = __shfl(jv[c], u, 16);
        double dp = 0.0, w = 0.0;
        if (j >= 0) {                      // uniform across the 16 lanes
          float x[EPL];
          Cols<EPL>::load(V + ((int64_t)j * H + h) * D + l16 * EPL, x);
          double part = 0.0;
#pragma unroll
          for (int e = 0; e < EPL; ++e) part = fma((double)g[e], (double)x[e], part);
          dp = sum16d(part);
          w = (double)__expf(__shfl(sv[c], u, 16) - m);
        }
        z += w;
        dsum = fma(w, dp, dsum);
        if (l16 == u) {
          wv[c] = w;
          dpv[c] = dp;
        }
      }
    }
  }
  const double inv = 1.0 / z;
  const double Dm = dsum * inv;

  // Pass 2: ds_t and dq = sum ds_t k_t.
  double acc[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) acc[e] = 0.0;
#pragma unroll
  for (int c = 0; c < MAXK / 16; ++c) {
    if (c * 16 < topk) {
      const int t = c * 16 + l16;
      const double p = wv[c] * inv;
      const double ds = p * (dpv[c] - Dm);
      if (t < topk) pairs[row * topk + t] = make_float2((float)p, (float)ds);
      const int tn = topk - c * 16 < 16 ? topk - c * 16 : 16;
      for (int u = 0; u < tn; ++u) {
        const int j = __shfl(jv[c], u, 16);
        const double dsu = __shfl(ds, u, 16);
        if (j >= 0) {
          float x[EPL];
          Cols<EPL>::load(Kt + ((int64_t)j * H + h) * D + l16 * EPL, x);
#pragma unroll
          for (int e = 0; e < EPL; ++e) acc[e] = fma(dsu, (double)x[e], acc[e]);
        }
      }
    }
  }
  float r[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) r[e] = (float)acc[e];
  store_cols<EPL>(dq + row * D + l16 * EPL, r);
}

}  // namespace

hipError_t launch_gather_av(const uint16_t* v, int64_t N, int H, int d, int topk,
                            const int32_t* topk_idx, const float* topk_score, float* out,
                            hipStream_t s) {
  const int64_t NH = N * H;
  const unsigned blocks = (unsigned)ceil_div(NH, ROWS_PER_BLOCK);
  if (d == 32)
    hipLaunchKernelGGL(gather_av_kernel<32>, dim3(blocks), dim3(256), 0, s, v, NH, H, topk,
                       topk_idx, topk_score, out);
  else if (d == 64)
    hipLaunchKernelGGL(gather_av_kernel<64>, dim3(blocks), dim3(256), 0, s, v, NH, H, topk,
                       topk_idx, topk_score, out);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_bwd_query(const uint16_t* k, const uint16_t* v, int64_t N, int H, int d,
                            int topk, const int32_t* topk_idx, const float* topk_score,
                            const float* dout, float* dq, float2* pairs, hipStream_t s) {
  const int64_t NH = N * H;
  const unsigned blocks = (unsigned)ceil_div(NH, ROWS_PER_BLOCK);
  if (d == 32)
    hipLaunchKernelGGL(bwd_query_kernel<32>, dim3(blocks), dim3(256), 0, s, k, v, NH, H, topk,
                       topk_idx, topk_score, dout, dq, pairs);
  else if (d == 64)
    hipLaunchKernelGGL(bwd_query_kernel<64>, dim3(blocks), dim3(256), 0, s, k, v, NH, H, topk,
                       topk_idx, topk_score, dout, dq, pairs);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace kmip
