// Per-lane column loads and stores of the bandwidth-bound kernels: a row of
// D elements is spread over 16 lanes, each owning EPL = D / 16 consecutive
// columns, so one row is a single coalesced segment.  Rows are bf16 bit
// patterns or fp32; values are widened to fp32 (bf16 -> fp32 is exact).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kmip {

template <int EPL>
__device__ __forceinline__ void load_cols(const uint16_t* p, float* x) {
  static_assert(EPL == 2 || EPL == 4, "d / 16 columns per lane");
  if constexpr (EPL == 2) {
    const uint32_t w = *reinterpret_cast<const uint32_t*>(p);
    x[0] = __uint_as_float(w << 16);
    x[1] = __uint_as_float(w & 0xffff0000u);
  } else {
    const uint2 w = *reinterpret_cast<const uint2*>(p);
    x[0] = __uint_as_float(w.x << 16);
    x[1] = __uint_as_float(w.x & 0xffff0000u);
    x[2] = __uint_as_float(w.y << 16);
    x[3] = __uint_as_float(w.y & 0xffff0000u);
  }
}

template <int EPL>
__device__ __forceinline__ void load_cols(const float* p, float* x) {
  static_assert(EPL == 2 || EPL == 4, "d / 16 columns per lane");
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

}  // namespace kmip
