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
// consecutive columns, so one gathered row is a single coalesced segment
// (64 or 128 bytes in bf16, 128 or 256 in fp32).  Index and score rows are
// read once per row group and broadcast with 16-lane shuffles.
#include "kmip_cols.h"
#include "kmip_internal.h"

namespace kmip {
namespace {

constexpr int ROWS_PER_BLOCK = 16;          // 256 threads, 16 lanes per row
constexpr int MAXK = 64;

// out[row] = sum_t softmax(score[row])_t * V[idx[row][t]] (bf16 V rows).
template <int D, typename T>
__global__ __launch_bounds__(256) void gather_av_kernel(
    const T* __restrict__ V, int64_t NH, int H, int topk,
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
  const int64_t self = row / H;
  float acc[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) acc[e] = 0.f;
  float z = 0.f;
#pragma unroll
  for (int c = 0; c < MAXK / 16; ++c) {
    if (c * 16 >= topk) break;
    // The chunk's 16 rows are requested together; unused slots read the
    // query's own row with weight 0 (adding 0 leaves the sums unchanged).
    const float wl = jv[c] >= 0 ? __expf(sv[c] - m) : 0.f;   // this lane's entry
    float x[16][EPL];
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int j = __shfl(jv[c], u, 16);
      load_cols<EPL>(V + ((j >= 0 ? (int64_t)j : self) * H + h) * D + l16 * EPL, x[u]);
    }
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const float w = __shfl(wl, u, 16);
      z += w;
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[e] = fmaf(w, x[u][e], acc[e]);
    }
  }
  const float inv = 1.f / z;
#pragma unroll
  for (int e = 0; e < EPL; ++e) acc[e] *= inv;
  store_cols<EPL>(out + row * D + l16 * EPL, acc);
}

// fp32 entry point: the scan selects on split-precision scores (error up to
// ~2^-16 |q||k|), and the softmax weights would inherit that error, which the
// backward's p (dp - D) can amplify where dp is close to D.  This variant
// recomputes each selected score in fp32 from the fp32 rows, s_t = q . k_t
// (lane partials of d/16 products, then a 16-lane tree), overwrites the saved
// score with it and weighs V with it.  The shift m is the best split score,
// within 2 eps of the best recomputed one, so exp stays bounded.  Selection
// and order are the scan's.
template <int D>
__global__ __launch_bounds__(256) void gather_rescore_av_kernel(
    const float* __restrict__ Q, const float* __restrict__ K, const float* __restrict__ V,
    int64_t NH, int H, int topk, const int32_t* __restrict__ idx, float* __restrict__ score,
    float* __restrict__ out) {
  constexpr int EPL = D / 16;
  const int l16 = threadIdx.x & 15;
  const int64_t row = (int64_t)blockIdx.x * ROWS_PER_BLOCK + (threadIdx.x >> 4);
  if (row >= NH) return;
  const int h = (int)(row % H);
  const int32_t* ir = idx + row * topk;
  float* sr = score + row * topk;

  int jv[MAXK / 16];
  float sv[MAXK / 16];
#pragma unroll
  for (int c = 0; c < MAXK / 16; ++c) {
    const int t = c * 16 + l16;
    jv[c] = t < topk ? ir[t] : -1;
    sv[c] = t < topk ? sr[t] : 0.f;
  }
  float qx[EPL];
  load_cols<EPL>(Q + row * D + l16 * EPL, qx);
  const float m = __shfl(sv[0], 0, 16);
  float acc[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) acc[e] = 0.f;
  float z = 0.f;
#pragma unroll
  for (int c = 0; c < MAXK / 16; ++c) {
    if (c * 16 >= topk) break;
    const int tn = topk - c * 16 < 16 ? topk - c * 16 : 16;
    float snew = sv[c];
    for (int u = 0; u < tn; ++u) {
      const int j = __shfl(jv[c], u, 16);
      if (j >= 0) {                         // uniform across the 16 lanes
        const int64_t base = ((int64_t)j * H + h) * D + l16 * EPL;
        float kx[EPL], vx[EPL];
        load_cols<EPL>(K + base, kx);
        load_cols<EPL>(V + base, vx);
        float part = 0.f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) part = fmaf(qx[e], kx[e], part);
#pragma unroll
        for (int o = 8; o >= 1; o >>= 1) part += __shfl_xor(part, o, 16);
        const float w = __expf(part - m);
        z += w;
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[e] = fmaf(w, vx[e], acc[e]);
        if (l16 == u) snew = part;
      }
    }
    const int t = c * 16 + l16;
    if (t < topk && jv[c] >= 0) sr[t] = snew;
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
// dO and bf16 or fp32 v are exact in fp64, and an fp32 p_0 alone would
// already carry an absolute error of ~6e-8.  The exponentials stay fp32 (each w_t is
// relatively accurate, which keeps p_0 = 1/Z accurate in fp64).
__device__ __forceinline__ double sum16d(double x) {
#pragma unroll
  for (int o = 8; o >= 1; o >>= 1) x += __shfl_xor(x, o, 16);
  return x;
}

// CPL consecutive row elements as fp32 (bf16 bit patterns or fp32), and
// the same elements copied as stored.
template <int CPL>
__device__ __forceinline__ void load_span(const uint16_t* p, float* x) {
#pragma unroll
  for (int h = 0; h < CPL / 8; ++h) {
    const uint4 w = *reinterpret_cast<const uint4*>(p + 8 * h);
    const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[8 * h + 2 * i] = __uint_as_float(u[i] << 16);
      x[8 * h + 2 * i + 1] = __uint_as_float(u[i] & 0xffff0000u);
    }
  }
}
template <int CPL>
__device__ __forceinline__ void load_span(const float* p, float* x) {
#pragma unroll
  for (int h = 0; h < CPL / 4; ++h) {
    const float4 w = *reinterpret_cast<const float4*>(p + 4 * h);
    x[4 * h] = w.x;
    x[4 * h + 1] = w.y;
    x[4 * h + 2] = w.z;
    x[4 * h + 3] = w.w;
  }
}
template <int CPL>
__device__ __forceinline__ void store_span(uint16_t* p, const float* x) {
#pragma unroll
  for (int h = 0; h < CPL / 8; ++h) {
    uint32_t u[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      u[i] = (__float_as_uint(x[8 * h + 2 * i]) >> 16) |
             (__float_as_uint(x[8 * h + 2 * i + 1]) & 0xffff0000u);
    *reinterpret_cast<uint4*>(p + 8 * h) = make_uint4(u[0], u[1], u[2], u[3]);
  }
}
template <int CPL>
__device__ __forceinline__ void store_span(float* p, const float* x) {
#pragma unroll
  for (int h = 0; h < CPL / 4; ++h)
    *reinterpret_cast<float4*>(p + 4 * h) = make_float4(x[4 * h], x[4 * h + 1], x[4 * h + 2],
                                                        x[4 * h + 3]);
}

// A query row is handled by 16 lanes.  Pass 1 takes the row's keys 16 at a
// time in four steps of four: in step p, lane l works on slot p*4 + (l & 3)
// and on the column quarter l >> 2, so the four lanes of a key read its K
// and V rows as one coalesced segment, each forming fp64 partial dot
// products over d/4 columns; two butterfly steps add the quarters, and lane
// l keeps the sums of step l >> 2, which are those of slot l.  Pass 2 gives
// each lane d/16 columns of dq = sum_t ds_t k_t; the ds_t and the first
// chunk's K rows reach it through LDS (later chunks' K rows are read again).
template <int D, typename T, int KMAX>
__global__ __launch_bounds__(256) void bwd_query_kernel(
    const T* __restrict__ Q, const T* __restrict__ Kt, const T* __restrict__ V, int64_t NH,
    int H, int topk, const int32_t* __restrict__ idx, const float* __restrict__ dout,
    float* __restrict__ dq, float2* __restrict__ pairs) {
  constexpr int EPL = D / 16;        // pass 2: columns per lane
  constexpr int CPL = D / 4;         // pass 1: columns per lane (one quarter)
  // First chunk's K rows, [group][slot][D] (+ padding so that the four
  // groups of a wave start on different banks), ds and key of every slot.
  constexpr int KROW = 16 * D + 64 / (int)sizeof(T);
  __shared__ T klds[ROWS_PER_BLOCK * KROW];
  __shared__ double dsl[ROWS_PER_BLOCK][KMAX];
  __shared__ int32_t jl[ROWS_PER_BLOCK][KMAX];
  const int l16 = threadIdx.x & 15, grp = threadIdx.x >> 4;
  const int64_t row = (int64_t)blockIdx.x * ROWS_PER_BLOCK + grp;
  if (row >= NH) return;                // whole 16-lane groups; no block barriers below
  const int h = (int)(row % H);
  const int64_t self = row / H;
  const int32_t* ir = idx + row * topk;
  const int qt = l16 >> 2, ks = l16 & 3;
  T* kg = klds + grp * KROW;

  // This lane's quarter of q and dO, widened once.
  float qf[CPL], gf[CPL];
  load_span<CPL>(Q + row * D + qt * CPL, qf);
  load_span<CPL>(dout + row * D + qt * CPL, gf);
  double qd[CPL], gd[CPL];
#pragma unroll
  for (int e = 0; e < CPL; ++e) {
    qd[e] = (double)qf[e];
    gd[e] = (double)gf[e];
  }

  // Pass 1.  The scores are recomputed here in fp64 from the input rows
  // (exact products), not taken from the forward's fp32 scores: where the
  // gradient is a cancelling sum of small softmax terms, the fp32
  // accumulation error of the scores (a few ulps) would be amplified.
  // dp_t - D is evaluated as (dp_t - dp_0) - sum_u p_u (dp_u - dp_0), with
  // entry 0 the best score (the largest weight): the same value, without the
  // cancellation that loses the small terms of sum_u p_u dp_u when the
  // softmax is nearly one-hot.  Unused slots read the query's own row and
  // count zero.
  double wv[KMAX / 16], dpv[KMAX / 16];
  double zl = 0.0, dl = 0.0;    // this lane's share of Z and sum w (dp - dp_0)
  double dp0 = 0.0, m = 0.0;    // entry 0's dp and score (the forward's best)
#pragma unroll
  for (int c = 0; c < KMAX / 16; ++c) {
    wv[c] = 0.0;
    dpv[c] = 0.0;
    if (c * 16 < topk) {
      double sc = 0.0, dp = 0.0;
      int32_t jmine = -1;
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const int t = c * 16 + p * 4 + ks;
        const int32_t jraw = ir[t < topk ? t : topk - 1];
        const int32_t j = t < topk ? jraw : -1;
        const int64_t jr = ((j >= 0 ? (int64_t)j : self) * H + h) * D + qt * CPL;
        float kx[CPL], vx[CPL];
        load_span<CPL>(Kt + jr, kx);
        load_span<CPL>(V + jr, vx);
        if (c == 0) store_span<CPL>(kg + (p * 4 + ks) * D + qt * CPL, kx);
        double s = 0.0, g = 0.0;
#pragma unroll
        for (int e = 0; e < CPL; ++e) {
          s = fma(qd[e], (double)kx[e], s);
          g = fma(gd[e], (double)vx[e], g);
        }
        s += __shfl_xor(s, 4, 16);
        g += __shfl_xor(g, 4, 16);
        s += __shfl_xor(s, 8, 16);
        g += __shfl_xor(g, 8, 16);
        if (p == qt) {                  // slot p*4 + ks == c*16 + l16
          sc = s;
          dp = g;
          jmine = j;
        }
      }
      jl[grp][c * 16 + l16] = jmine;
      if (c == 0) {
        dp0 = __shfl(dp, 0, 16);
        m = __shfl(sc, 0, 16);
      }
      const bool live = jmine >= 0;
      // fp64 exp: weights far below the best (e^-87 and less) stay normal
      // numbers instead of underflowing in fp32.
      const double w = live ? exp(sc - m) : 0.0;
      wv[c] = w;
      dpv[c] = live ? dp - dp0 : 0.0;
      zl += w;
      dl = fma(w, dpv[c], dl);
    }
  }
  const double inv = 1.0 / sum16d(zl);
  const double Dm = sum16d(dl) * inv;

  // Pass 2: ds_t, then dq = sum ds_t k_t over this lane's columns.
#pragma unroll
  for (int c = 0; c < KMAX / 16; ++c) {
    if (c * 16 < topk) {
      const int t = c * 16 + l16;
      const double p = wv[c] * inv;
      const double ds = p * (dpv[c] - Dm);
      if (t < topk) pairs[row * topk + t] = make_float2((float)p, (float)ds);
      dsl[grp][t] = ds;                    // 0 on unused slots
    }
  }
  __builtin_amdgcn_wave_barrier();
  double acc[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) acc[e] = 0.0;
#pragma unroll
  for (int c = 0; c < KMAX / 16; ++c) {
    if (c * 16 < topk) {
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        const double dsu = dsl[grp][c * 16 + u];
        float x[EPL];
        if (c == 0) {
          load_cols<EPL>(kg + u * D + l16 * EPL, x);
        } else {
          const int32_t j = jl[grp][c * 16 + u];
          load_cols<EPL>(Kt + ((j >= 0 ? (int64_t)j : self) * H + h) * D + l16 * EPL, x);
        }
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[e] = fma(dsu, (double)x[e], acc[e]);
      }
    }
  }
  float r[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) r[e] = (float)acc[e];
  store_cols<EPL>(dq + row * D + l16 * EPL, r);
}

template <int D, typename T>
void launch_gather_t(const T* v, int64_t NH, int H, int topk, const int32_t* idx,
                     const float* score, float* out, hipStream_t s) {
  const unsigned blocks = (unsigned)ceil_div(NH, ROWS_PER_BLOCK);
  hipLaunchKernelGGL((gather_av_kernel<D, T>), dim3(blocks), dim3(256), 0, s, v, NH, H, topk,
                     idx, score, out);
}

template <int D, typename T>
void launch_bwd_query_t(const T* q, const T* k, const T* v, int64_t NH, int H, int topk,
                        const int32_t* idx, const float* dout, float* dq, float2* pairs,
                        hipStream_t s) {
  // Per-row LDS sized by the list length: 20 KB per workgroup at k <= 16
  // (seven share a CU) instead of 30 KB (five).
  const unsigned blocks = (unsigned)ceil_div(NH, ROWS_PER_BLOCK);
  if (topk <= 16)
    hipLaunchKernelGGL((bwd_query_kernel<D, T, 16>), dim3(blocks), dim3(256), 0, s, q, k, v, NH,
                       H, topk, idx, dout, dq, pairs);
  else
    hipLaunchKernelGGL((bwd_query_kernel<D, T, MAXK>), dim3(blocks), dim3(256), 0, s, q, k, v,
                       NH, H, topk, idx, dout, dq, pairs);
}

}  // namespace

hipError_t launch_gather_rescore_av(const float* q, const float* k, const float* v, int64_t N,
                                    int H, int d, int topk, const int32_t* topk_idx,
                                    float* topk_score, float* out, hipStream_t s) {
  const int64_t NH = N * H;
  const unsigned blocks = (unsigned)ceil_div(NH, ROWS_PER_BLOCK);
  if (d == 32)
    hipLaunchKernelGGL(gather_rescore_av_kernel<32>, dim3(blocks), dim3(256), 0, s, q, k, v, NH,
                       H, topk, topk_idx, topk_score, out);
  else if (d == 64)
    hipLaunchKernelGGL(gather_rescore_av_kernel<64>, dim3(blocks), dim3(256), 0, s, q, k, v, NH,
                       H, topk, topk_idx, topk_score, out);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_gather_av(const uint16_t* v, int64_t N, int H, int d, int topk,
                            const int32_t* topk_idx, const float* topk_score, float* out,
                            hipStream_t s) {
  const int64_t NH = N * H;
  if (d == 32) launch_gather_t<32>(v, NH, H, topk, topk_idx, topk_score, out, s);
  else if (d == 64) launch_gather_t<64>(v, NH, H, topk, topk_idx, topk_score, out, s);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_bwd_query(const void* q, const void* k, const void* v, bool f32, int64_t N,
                            int H, int d, int topk, const int32_t* topk_idx, const float* dout,
                            float* dq, float2* pairs, hipStream_t s) {
  const int64_t NH = N * H;
  const uint16_t *qb = static_cast<const uint16_t*>(q), *kb = static_cast<const uint16_t*>(k),
                 *vb = static_cast<const uint16_t*>(v);
  const float *qf = static_cast<const float*>(q), *kf = static_cast<const float*>(k),
              *vf = static_cast<const float*>(v);
  if (d == 32 && !f32)
    launch_bwd_query_t<32>(qb, kb, vb, NH, H, topk, topk_idx, dout, dq, pairs, s);
  else if (d == 32)
    launch_bwd_query_t<32>(qf, kf, vf, NH, H, topk, topk_idx, dout, dq, pairs, s);
  else if (d == 64 && !f32)
    launch_bwd_query_t<64>(qb, kb, vb, NH, H, topk, topk_idx, dout, dq, pairs, s);
  else if (d == 64)
    launch_bwd_query_t<64>(qf, kf, vf, NH, H, topk, topk_idx, dout, dq, pairs, s);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace kmip
