// Host side of the score scan: the ragged tile plan for batched graphs, the
// query order for one graph, and the dispatch to the per-dimension scan
// kernels (kmip_scan_kernels.h, instantiated in kmip_scan_d*.hip).
#include "kmip_internal.h"

namespace kmip {
namespace {

// ------------------------------------------------------------------ tile plan
constexpr int PLAN_THREADS = 1024;

// One block: tile_start[b] = sum over earlier graphs of ceil(n_b / tile_rows).
__global__ __launch_bounds__(PLAN_THREADS) void tile_count_scan_kernel(
    const int32_t* __restrict__ offsets, int B, int tile_rows, int32_t* __restrict__ tile_start) {
  __shared__ int32_t buf[PLAN_THREADS];
  int32_t carry = 0;
  for (int base = 0; base < B; base += PLAN_THREADS) {
    const int b = base + (int)threadIdx.x;
    int32_t c = 0;
    if (b < B) {
      const int32_t nb = offsets[b + 1] - offsets[b];
      c = nb > 0 ? (nb + tile_rows - 1) / tile_rows : 0;
    }
    buf[threadIdx.x] = c;
    __syncthreads();
    for (int o = 1; o < PLAN_THREADS; o <<= 1) {       // inclusive Hillis-Steele scan
      const int32_t add = threadIdx.x >= (unsigned)o ? buf[threadIdx.x - o] : 0;
      __syncthreads();
      buf[threadIdx.x] += add;
      __syncthreads();
    }
    if (b < B) tile_start[b] = carry + buf[threadIdx.x] - c;
    carry += buf[PLAN_THREADS - 1];
    __syncthreads();
  }
  if (threadIdx.x == 0) tile_start[B] = carry;
}

__global__ void tile_fill_kernel(const int32_t* __restrict__ offsets, int B, int tile_rows,
                                 const int32_t* __restrict__ tile_start, int64_t max_tiles,
                                 int2* __restrict__ tiles) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= max_tiles) return;
  const int32_t total = tile_start[B];
  if (t >= total) {
    tiles[t] = make_int2(-1, 0);
    return;
  }
  int lo = 0, hi = B - 1;               // last graph whose first tile is <= t
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (tile_start[mid] <= t) lo = mid; else hi = mid - 1;
  }
  tiles[t] = make_int2(lo, offsets[lo] + (int)(t - tile_start[lo]) * tile_rows);
}

// ------------------------------------------------------------ query order
// Queries of one head are grouped by a 14-bit sign-random-projection code of
// q (Rademacher directions fixed by the constants below), so that the 32
// queries of a wavefront tend to point the same way and share their few
// high-scoring keys: the selection pass then meets far fewer 32-key blocks
// holding a candidate for any of its queries.  The order only changes which
// queries share a wavefront; every query's result is independent of it.
constexpr int LSH_BITS = 14;
constexpr int LSH_BINS = 1 << LSH_BITS;
// Each (head, code) count is split over LSH_COPIES counters picked by the
// node id, which keeps atomic contention low when many queries share a code.
constexpr int LSH_COPIES = 4;
__constant__ uint32_t kLshSigns[LSH_BITS][2] = {
    {0x9e3779b9u, 0x7f4a7c15u}, {0xf39cc060u, 0x5ced1d6bu}, {0xbf58476du, 0x1ce4e5b9u},
    {0x94d049bbu, 0x133111ebu}, {0x2545f491u, 0x4f6cdd1du}, {0xd6e8feb8u, 0x6658e9a5u},
    {0x85ebca6bu, 0xc2b2ae35u}, {0x27d4eb2fu, 0x165667b1u}, {0xa0761d64u, 0xe7037ed1u},
    {0x8ebc6af0u, 0x589965ccu}, {0x1d8e4e27u, 0xc5ed3a8bu}, {0x6a09e667u, 0xbb67ae85u},
    {0x3c6ef372u, 0xa54ff53au}, {0x510e527fu, 0x9b05688cu}};

__global__ void fill_zero_kernel(int32_t* __restrict__ p, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0;
}

// codes[h*N + i] and per-(head, code) counts.
template <int D>
__global__ void lsh_code_kernel(const uint16_t* __restrict__ Q, int64_t N, int H,
                                uint16_t* __restrict__ codes, int32_t* __restrict__ counts) {
  const int64_t r = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;   // r = i*H + h
  if (r >= N * H) return;
  const int64_t i = r / H;
  const int h = (int)(r % H);
  // The code uses the first min(D, 64) elements (for split rows: the high
  // parts).
  constexpr int DH = D < 64 ? D : 64;
  float x[DH];
  const uint4* src = reinterpret_cast<const uint4*>(Q + r * D);
#pragma unroll
  for (int c = 0; c < DH / 8; ++c) {
    const uint4 w = src[c];
    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x[8 * c + 2 * e] = __uint_as_float(ws[e] << 16);
      x[8 * c + 2 * e + 1] = __uint_as_float(ws[e] & 0xffff0000u);
    }
  }
  uint32_t code = 0;
#pragma unroll
  for (int b = 0; b < LSH_BITS; ++b) {
    float acc = 0.f;
#pragma unroll
    for (int c = 0; c < (D < 64 ? D : 64); ++c) {
      const bool neg = (kLshSigns[b][c >> 5] >> (c & 31)) & 1u;
      acc += neg ? -x[c] : x[c];
    }
    code |= (acc > 0.f ? 1u : 0u) << b;
  }
  codes[h * N + i] = (uint16_t)code;
  atomicAdd(&counts[((int64_t)h * LSH_BINS + code) * LSH_COPIES + (i & (LSH_COPIES - 1))], 1);
}

// perm[h*N + pos] = i, positions handed out per (head, code) from the
// scanned counts.  The order inside a code group is immaterial.
__global__ void lsh_place_kernel(const uint16_t* __restrict__ codes, int64_t N, int H,
                                 int32_t* __restrict__ cursor, int32_t* __restrict__ perm) {
  const int64_t r = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;   // r = h*N + i
  if (r >= N * H) return;
  const int h = (int)(r / N);
  const int64_t i = r % N;
  const int pos = atomicAdd(
      &cursor[((int64_t)h * LSH_BINS + codes[r]) * LSH_COPIES + (i & (LSH_COPIES - 1))], 1);
  perm[pos] = (int32_t)i;
}

}  // namespace

int scan_list_len(int topk) {
  static const int lens[] = {5, 8, 15, 16, 32, 45, 48, 64};
  for (int L : lens)
    if (topk <= L) return L;
  return -1;
}

hipError_t launch_tile_plan(const int32_t* offsets, int num_graphs, int64_t max_tiles,
                            int tile_rows, int32_t* tile_start, int2* tiles, hipStream_t s) {
  hipLaunchKernelGGL(tile_count_scan_kernel, dim3(1), dim3(PLAN_THREADS), 0, s, offsets,
                     num_graphs, tile_rows, tile_start);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const unsigned blocks = (unsigned)ceil_div(max_tiles, 256);
  hipLaunchKernelGGL(tile_fill_kernel, dim3(blocks), dim3(256), 0, s, offsets, num_graphs,
                     tile_rows, tile_start, max_tiles, tiles);
  return hipGetLastError();
}

size_t query_order_bytes(int64_t N, int H) {
  const int64_t nb = (int64_t)H * LSH_BINS * LSH_COPIES;
  return align256((size_t)N * H * 4) + align256((size_t)N * H * 2) + 2 * align256((size_t)nb * 4) +
         align256((size_t)scan_aux_elems(nb) * 4);
}

hipError_t launch_query_order(const uint16_t* q, int64_t N, int H, int d, void* ws,
                              int32_t** perm_out, hipStream_t s) {
  const int64_t nb = (int64_t)H * LSH_BINS * LSH_COPIES;
  char* p = static_cast<char*>(ws);
  int32_t* perm = reinterpret_cast<int32_t*>(p); p += align256((size_t)N * H * 4);
  uint16_t* codes = reinterpret_cast<uint16_t*>(p); p += align256((size_t)N * H * 2);
  int32_t* counts = reinterpret_cast<int32_t*>(p); p += align256((size_t)nb * 4);
  int32_t* cursor = reinterpret_cast<int32_t*>(p); p += align256((size_t)nb * 4);
  int32_t* aux = reinterpret_cast<int32_t*>(p);
  const unsigned rows = (unsigned)ceil_div(N * H, 256);
  hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)ceil_div(nb, 256)), dim3(256), 0, s,
                     counts, nb);
  switch (d) {
    case 32: hipLaunchKernelGGL(lsh_code_kernel<32>, dim3(rows), dim3(256), 0, s, q, N, H,
                                codes, counts); break;
    case 64: hipLaunchKernelGGL(lsh_code_kernel<64>, dim3(rows), dim3(256), 0, s, q, N, H,
                                codes, counts); break;
    case 96: hipLaunchKernelGGL(lsh_code_kernel<96>, dim3(rows), dim3(256), 0, s, q, N, H,
                                codes, counts); break;
    case 192: hipLaunchKernelGGL(lsh_code_kernel<192>, dim3(rows), dim3(256), 0, s, q, N, H,
                                 codes, counts); break;
    default: return hipErrorInvalidValue;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // Exclusive scan over (head, code, copy): head h's positions start at h*N.
  e = launch_exclusive_scan(counts, cursor, nb, aux, s);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(lsh_place_kernel, dim3(rows), dim3(256), 0, s, codes, N, H, cursor, perm);
  *perm_out = perm;
  return hipGetLastError();
}

hipError_t launch_score_topk(const ScanArgs& args, int d, hipStream_t s) {
  const int kp = scan_list_len(args.topk);
  switch (d) {
    case 32: return launch_scan_d32(kp, args, s);
    case 64: return launch_scan_d64(kp, args, s);
    case 96: return launch_scan_d96(kp, args, s);
    case 192: return launch_scan_d192(kp, args, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace kmip
