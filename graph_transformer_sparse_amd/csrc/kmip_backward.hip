// Key side of the k-MIP backward: dk_j = sum_i ds_ij q_i and
// dv_j = sum_i p_ij dO_i over every query i that selected key j.
//
// Page "k-Maximum Inner Product Attention for Graph Transformers and the
// Expressive Power of GraphGPS", Abstract: the attention pattern is the
// sparse set of selected (query, key) pairs; its gradient reaches a key only
// through the pairs that selected it.
//
// The forward leaves the selection as rows of k keys per query.  The key
// side needs the transpose, so:
//  1. a stable LSD radix sort (8-bit digits) orders the pairs (row*k + slot)
//     by the key h*N + j (padding slots get the sentinel H*N); within a key
//     the pairs stay in ascending pair id, i.e. ascending query.  The first
//     pass derives the keys from topk_idx and the pair ids from positions;
//     every pass carries the pair's (p, ds), so the reduction reads them in
//     sorted order instead of gathering 8 bytes per pair;
//  2. key segment pointers come from a binary search of the sorted keys;
//  3. fixed-length slices of the sorted pairs are reduced by 16-lane groups
//     (no atomics).  Runs that cover a whole key segment are written
//     directly; runs cut by a slice boundary go to per-slice partials, which
//     a fix-up pass adds in slice order.  Keys selected by no query get exact
//     zeros.  Every sum has a fixed order, so results are bitwise repeatable.
#include "kmip_cols.h"
#include "kmip_internal.h"

namespace kmip {
namespace {

// Sort key of pair pid (row-major [N][H][k] slots of topk_idx).
__device__ __forceinline__ uint32_t pair_key(const int32_t* __restrict__ idx, int64_t pid,
                                             int64_t N, int H, int topk) {
  const int h = (int)((pid / topk) % H);
  const int32_t j = idx[pid];
  return j < 0 ? (uint32_t)(N * H) : (uint32_t)(h * N + j);
}

// ------------------------------------------------------------ device scan
__device__ __forceinline__ int32_t wave_incl_scan(int32_t x, int lane) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int32_t y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  return x;
}

// Exclusive scan of the values of one block (256 threads); returns the
// thread's exclusive prefix and the block total through *total.
__device__ __forceinline__ int32_t block_excl_scan(int32_t x, int32_t* sh, int32_t* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int32_t incl = wave_incl_scan(x, lane);
  if (lane == 63) sh[wave] = incl;
  __syncthreads();
  int32_t base = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < SCAN_THREADS / 64; ++w) {
    const int32_t v = sh[w];
    base += w < wave ? v : 0;
    tot += v;
  }
  __syncthreads();
  *total = tot;
  return base + incl - x;
}

__global__ __launch_bounds__(SCAN_THREADS) void scan_reduce_kernel(
    const int32_t* __restrict__ in, int64_t n, int32_t* __restrict__ aux) {
  __shared__ int32_t sh[SCAN_THREADS / 64];
  const int64_t base = (int64_t)blockIdx.x * SCAN_TILE_ELEMS + (int64_t)threadIdx.x * SCAN_ITEMS;
  int32_t s = 0;
#pragma unroll
  for (int i = 0; i < SCAN_ITEMS; ++i) s += (base + i < n) ? in[base + i] : 0;
  int32_t tot;
  block_excl_scan(s, sh, &tot);
  if (threadIdx.x == 0) aux[blockIdx.x] = tot;
}

// One block: exclusive scan of aux[0..m) in place.
__global__ __launch_bounds__(SCAN_THREADS) void scan_aux_kernel(int32_t* __restrict__ aux,
                                                                int64_t m) {
  __shared__ int32_t sh[SCAN_THREADS / 64];
  int32_t carry = 0;
  for (int64_t b = 0; b < m; b += SCAN_THREADS) {
    const int64_t i = b + threadIdx.x;
    const int32_t x = i < m ? aux[i] : 0;
    int32_t tot;
    const int32_t ex = block_excl_scan(x, sh, &tot);
    if (i < m) aux[i] = carry + ex;
    carry += tot;
  }
}

// One block scans up to SCAN_SINGLE_TILES tiles in order, carrying the sum.
// in and out may be the same array (each element is read before it is
// written, by the same thread), so neither is declared __restrict__.
constexpr int SCAN_SINGLE_TILES = 4;
__global__ __launch_bounds__(SCAN_THREADS) void scan_single_kernel(
    const int32_t* in, int32_t* out, int64_t n) {
  __shared__ int32_t sh[SCAN_THREADS / 64];
  int32_t carry = 0;
  for (int64_t tile = 0; tile < n; tile += SCAN_TILE_ELEMS) {
    const int64_t base = tile + (int64_t)threadIdx.x * SCAN_ITEMS;
    int32_t v[SCAN_ITEMS];
    int32_t s = 0;
#pragma unroll
    for (int i = 0; i < SCAN_ITEMS; ++i) {
      v[i] = (base + i < n) ? in[base + i] : 0;
      s += v[i];
    }
    int32_t tot;
    int32_t run = block_excl_scan(s, sh, &tot) + carry;
#pragma unroll
    for (int i = 0; i < SCAN_ITEMS; ++i) {
      if (base + i < n) out[base + i] = run;
      run += v[i];
    }
    carry += tot;
  }
}

// in and out may be the same array (see scan_single_kernel).
__global__ __launch_bounds__(SCAN_THREADS) void scan_down_kernel(
    const int32_t* in, int32_t* out, int64_t n, const int32_t* __restrict__ aux) {
  __shared__ int32_t sh[SCAN_THREADS / 64];
  const int64_t base = (int64_t)blockIdx.x * SCAN_TILE_ELEMS + (int64_t)threadIdx.x * SCAN_ITEMS;
  int32_t v[SCAN_ITEMS];
  int32_t s = 0;
#pragma unroll
  for (int i = 0; i < SCAN_ITEMS; ++i) {
    v[i] = (base + i < n) ? in[base + i] : 0;
    s += v[i];
  }
  int32_t tot;
  int32_t run = block_excl_scan(s, sh, &tot) + aux[blockIdx.x];
#pragma unroll
  for (int i = 0; i < SCAN_ITEMS; ++i) {
    if (base + i < n) out[base + i] = run;
    run += v[i];
  }
}

// ------------------------------------------------------------ radix sort
// Digit histogram of one tile.  First pass (keys == nullptr): the keys are
// derived from topk_idx.
__global__ __launch_bounds__(SORT_THREADS) void radix_hist_kernel(
    const uint32_t* __restrict__ keys, const int32_t* __restrict__ idx, int64_t N, int H,
    int topk, int64_t P, int shift, int32_t* __restrict__ hist, int64_t nblk) {
  __shared__ int32_t cnt[SORT_BINS];
  cnt[threadIdx.x] = 0;
  __syncthreads();
  const int64_t base = (int64_t)blockIdx.x * SORT_TILE;
#pragma unroll
  for (int i = 0; i < SORT_ITEMS; ++i) {
    const int64_t e = base + i * SORT_THREADS + threadIdx.x;
    if (e < P) {
      const uint32_t k = keys ? keys[e] : pair_key(idx, e, N, H, topk);
      atomicAdd(&cnt[(k >> shift) & (SORT_BINS - 1)], 1);
    }
  }
  __syncthreads();
  hist[(int64_t)threadIdx.x * nblk + blockIdx.x] = cnt[threadIdx.x];
}

// Stable scatter.  Wave w of the block ranks the elements
// [tile + w*1024, +1024) in order, 64 at a time: equal digits inside a
// 64-element chunk are found with 8 ballots, and a per-wave running count
// per digit carries the rank across chunks.  Waves are then offset by the
// counts of the earlier waves, the tile is reordered by digit in LDS, and
// each digit's run is written at the block's offset from the scanned
// histogram.
// First pass (keys_in == nullptr): keys come from topk_idx and pair ids are
// the positions.
__global__ __launch_bounds__(SORT_THREADS) void radix_scatter_kernel(
    const uint32_t* __restrict__ keys_in, const uint32_t* __restrict__ vals_in,
    const float2* __restrict__ pay_in, const int32_t* __restrict__ idx, int64_t N, int H,
    int topk, int64_t P, int shift, const int32_t* __restrict__ hist_scan, int64_t nblk,
    uint32_t* __restrict__ keys_out, uint32_t* __restrict__ vals_out,
    float2* __restrict__ pay_out) {
  constexpr int NW = SORT_THREADS / 64;
  constexpr int PER_WAVE = SORT_TILE / NW;
  constexpr int CHUNKS = PER_WAVE / 64;
  static_assert(SORT_THREADS == SCAN_THREADS && SORT_BINS == SORT_THREADS,
                "one digit per thread; block_excl_scan covers the block");
  __shared__ int32_t wcnt[NW][SORT_BINS];
  __shared__ int32_t gbase[SORT_BINS];
  __shared__ int32_t dstart[SORT_BINS];
  __shared__ int32_t sh[SORT_THREADS / 64];
  __shared__ uint32_t lk[SORT_TILE];
  __shared__ uint32_t lv[SORT_TILE];
  __shared__ float2 lpay[SORT_TILE];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int w = 0; w < NW; ++w) wcnt[w][threadIdx.x] = 0;
  gbase[threadIdx.x] = hist_scan[(int64_t)threadIdx.x * nblk + blockIdx.x];
  __syncthreads();

  const uint64_t lt = (1ull << lane) - 1ull;
  const int64_t wbase = (int64_t)blockIdx.x * SORT_TILE + (int64_t)wave * PER_WAVE;
  const bool first = keys_in == nullptr;
  uint32_t k[CHUNKS], v[CHUNKS];
  float2 pl[CHUNKS];
  int32_t rank[CHUNKS];
#pragma unroll
  for (int c = 0; c < CHUNKS; ++c) {
    const int64_t e = wbase + c * 64 + lane;
    const bool valid = e < P;
    k[c] = !valid ? 0u : first ? pair_key(idx, e, N, H, topk) : keys_in[e];
    v[c] = !valid ? 0u : first ? (uint32_t)e : vals_in[e];
    pl[c] = valid ? pay_in[e] : make_float2(0.f, 0.f);
    const int dg = (int)((k[c] >> shift) & (SORT_BINS - 1));
    uint64_t peers = __ballot(valid);
#pragma unroll
    for (int b = 0; b < SORT_BITS; ++b) {
      const int bit = (dg >> b) & 1;
      const uint64_t bal = __ballot(bit);
      peers &= bit ? bal : ~bal;
    }
    const int32_t before = wcnt[wave][dg];
    rank[c] = before + __popcll(peers & lt);
    const bool leader = valid && (lane == 63 || (peers >> (lane + 1)) == 0ull);
    if (leader) wcnt[wave][dg] = before + __popcll(peers);
  }
  __syncthreads();
  int32_t dtot = 0;
  {   // exclusive prefix over waves, one digit per thread
    const int d = threadIdx.x;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const int32_t c = wcnt[w][d];
      wcnt[w][d] = dtot;
      dtot += c;
    }
  }
  // Block-local start of every digit's run, then the tile is staged in LDS
  // in digit order so that the global writes go out as contiguous runs.
  int32_t tile_total;
  dstart[threadIdx.x] = block_excl_scan(dtot, sh, &tile_total);
  __syncthreads();
#pragma unroll
  for (int c = 0; c < CHUNKS; ++c) {
    const int64_t e = wbase + c * 64 + lane;
    if (e < P) {
      const int dg = (int)((k[c] >> shift) & (SORT_BINS - 1));
      const int lp = dstart[dg] + wcnt[wave][dg] + rank[c];
      lk[lp] = k[c];
      lv[lp] = v[c];
      lpay[lp] = pl[c];
    }
  }
  __syncthreads();
  for (int i = threadIdx.x; i < tile_total; i += SORT_THREADS) {
    const uint32_t kk = lk[i];
    const int dg = (int)((kk >> shift) & (SORT_BINS - 1));
    const int64_t pos = (int64_t)gbase[dg] + (i - dstart[dg]);
    keys_out[pos] = kk;
    vals_out[pos] = lv[i];
    pay_out[pos] = lpay[i];
  }
}

// ------------------------------------------------------------ segmented reduce
constexpr int SEG_GROUPS = 16;     // 16-lane groups per 256-thread block

// partials layout: [slice][slot 0|1][dk | dv][D], fp64.  Sums are carried in
// fp64 (hub keys add thousands of terms of mixed sign) and rounded to fp32
// once, when the key's total is written.  Q rows are bf16 (QT = uint16_t) or
// fp32.
template <int D, typename QT>
__global__ __launch_bounds__(256) void segreduce_kernel(
    const QT* __restrict__ Q, const float* __restrict__ dout,
    const float2* __restrict__ spay, const uint32_t* __restrict__ skeys,
    const uint32_t* __restrict__ svals, const int32_t* __restrict__ key_ptr, int64_t N, int H,
    int topk, int64_t nslices, double* __restrict__ partials, float* __restrict__ dk,
    float* __restrict__ dv) {
  constexpr int EPL = D / 16;
  const int l16 = threadIdx.x & 15;
  const int64_t slice = (int64_t)blockIdx.x * SEG_GROUPS + (threadIdx.x >> 4);
  if (slice >= nslices) return;
  const int64_t HN = N * H;
  const int64_t valid_end = key_ptr[HN];
  const int64_t s0 = slice * SEG_SLICE;
  if (s0 >= valid_end) return;
  const int64_t s1 = s0 + SEG_SLICE < valid_end ? s0 + SEG_SLICE : valid_end;

  double ak[EPL], av[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) ak[e] = av[e] = 0.0;
  uint32_t cur = skeys[s0];
  int64_t run0 = s0;

  auto flush = [&](uint32_t key, int64_t ra, int64_t rb) __attribute__((always_inline)) {
    const int64_t sa = key_ptr[key], sb = key_ptr[key + 1];
    if (ra == sa && rb == sb) {
      const int64_t j = key % N, h = key / N;
      const int64_t orow = j * H + h;
      float fk[EPL], fv[EPL];
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        fk[e] = (float)ak[e];
        fv[e] = (float)av[e];
      }
      store_cols<EPL>(dk + orow * D + l16 * EPL, fk);
      store_cols<EPL>(dv + orow * D + l16 * EPL, fv);
      return;
    }
    const int slot = (ra == s0) ? 0 : 1;
    double* dst = partials + ((slice * 2 + slot) * 2) * D + l16 * EPL;
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      dst[e] = ak[e];
      dst[D + e] = av[e];
    }
  };

  // The slice's keys, pair ids and (p, ds) are read once, coalesced: lane l
  // of the group holds pairs s0 + 16 i + l.  The loop then takes them by
  // shuffles and requests the q and dO rows of four pairs at a time.
  constexpr int PER_LANE = SEG_SLICE / 16;
  const int n = (int)(s1 - s0);
  uint32_t mk[PER_LANE], mv[PER_LANE];
  float mpx[PER_LANE], mpy[PER_LANE];
#pragma unroll
  for (int i = 0; i < PER_LANE; ++i) {
    const int u = i * 16 + l16;
    const bool ok = u < n;
    mk[i] = ok ? skeys[s0 + u] : 0u;
    mv[i] = ok ? svals[s0 + u] : 0u;
    const float2 pr = ok ? spay[s0 + u] : make_float2(0.f, 0.f);
    mpx[i] = pr.x;
    mpy[i] = pr.y;
  }
#pragma unroll
  for (int g4 = 0; g4 < SEG_SLICE; g4 += 4) {
    if (g4 >= n) break;
    uint32_t key[4];
    float px[4], py[4], qx[4][EPL], gx[4][EPL];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int ip = g4 + u, i = ip / 16, src = ip % 16;
      key[u] = __shfl(mk[i], src, 16);
      const uint32_t pid = __shfl(mv[i], src, 16);
      px[u] = __shfl(mpx[i], src, 16);
      py[u] = __shfl(mpy[i], src, 16);
      if (ip < n) {
        const int64_t row = pid / (uint32_t)topk;
        load_cols<EPL>(Q + row * D + l16 * EPL, qx[u]);
        load_cols<EPL>(dout + row * D + l16 * EPL, gx[u]);
      }
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int ip = g4 + u;
      if (ip >= n) break;
      const int64_t t = s0 + ip;
      if (key[u] != cur) {
        flush(cur, run0, t);
#pragma unroll
        for (int e = 0; e < EPL; ++e) ak[e] = av[e] = 0.0;
        cur = key[u];
        run0 = t;
      }
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        ak[e] = fma((double)py[u], (double)qx[u][e], ak[e]);
        av[e] = fma((double)px[u], (double)gx[u][e], av[e]);
      }
    }
  }
  flush(cur, run0, s1);
}

// One 16-lane group per key: zeros for unselected keys, and the in-order sum
// of slice partials for keys whose segment crosses a slice boundary.
template <int D>
__global__ __launch_bounds__(256) void segfix_kernel(const int32_t* __restrict__ key_ptr,
                                                     int64_t N, int H,
                                                     const double* __restrict__ partials,
                                                     float* __restrict__ dk,
                                                     float* __restrict__ dv) {
  constexpr int EPL = D / 16;
  const int l16 = threadIdx.x & 15;
  const int64_t key = (int64_t)blockIdx.x * SEG_GROUPS + (threadIdx.x >> 4);
  const int64_t HN = N * H;
  if (key >= HN) return;
  const int64_t a = key_ptr[key], b = key_ptr[key + 1];
  const int64_t orow = (key % N) * H + key / N;
  double ak[EPL], av[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) ak[e] = av[e] = 0.0;
  if (a < b) {
    const int64_t sa = a / SEG_SLICE, sb = (b - 1) / SEG_SLICE;
    if (sa == sb) return;                       // written by segreduce_kernel
    for (int64_t s = sa; s <= sb; ++s) {
      const int slot = (s == sa && a != sa * SEG_SLICE) ? 1 : 0;
      const double* src = partials + ((s * 2 + slot) * 2) * D + l16 * EPL;
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        ak[e] += src[e];
        av[e] += src[D + e];
      }
    }
  }
  float fk[EPL], fv[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) {
    fk[e] = (float)ak[e];
    fv[e] = (float)av[e];
  }
  store_cols<EPL>(dk + orow * D + l16 * EPL, fk);
  store_cols<EPL>(dv + orow * D + l16 * EPL, fv);
}

// key_ptr[key] = first position of the sorted keys that is >= key, for
// key in [0, H*N + 1]: the segment of key is [key_ptr[key], key_ptr[key+1]).
__global__ void key_ptr_kernel(const uint32_t* __restrict__ skeys, int64_t P, int64_t nkeys,
                               int32_t* __restrict__ key_ptr) {
  const int64_t key = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (key >= nkeys) return;
  int64_t lo = 0, hi = P;
  while (lo < hi) {
    const int64_t mid = (lo + hi) >> 1;
    if ((int64_t)skeys[mid] < key) lo = mid + 1; else hi = mid;
  }
  key_ptr[key] = (int32_t)lo;
}

int sort_passes(int64_t max_key) {
  int bits = 0;
  while ((max_key >> bits) != 0) ++bits;
  return bits == 0 ? 1 : (bits + SORT_BITS - 1) / SORT_BITS;
}

}  // namespace

int64_t scan_aux_elems(int64_t n) { return ceil_div(n, SCAN_TILE_ELEMS) + 1; }

hipError_t launch_exclusive_scan(const int32_t* in, int32_t* out, int64_t n, int32_t* aux,
                                 hipStream_t s) {
  const int64_t nb = ceil_div(n, SCAN_TILE_ELEMS);
  if (nb <= SCAN_SINGLE_TILES) {                 // small arrays: one launch
    hipLaunchKernelGGL(scan_single_kernel, dim3(1), dim3(SCAN_THREADS), 0, s, in, out, n);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(scan_reduce_kernel, dim3((unsigned)nb), dim3(SCAN_THREADS), 0, s, in, n,
                     aux);
  hipLaunchKernelGGL(scan_aux_kernel, dim3(1), dim3(SCAN_THREADS), 0, s, aux, nb);
  hipLaunchKernelGGL(scan_down_kernel, dim3((unsigned)nb), dim3(SCAN_THREADS), 0, s, in, out,
                     n, aux);
  return hipGetLastError();
}

size_t sort_scratch_bytes(int64_t P, int64_t HN) {
  const int64_t nblk = ceil_div(P, SORT_TILE);
  const int64_t hist_n = (int64_t)SORT_BINS * nblk;
  const int64_t aux_n = scan_aux_elems(hist_n);
  size_t b = 0;
  b += 4 * align256((size_t)P * 4);            // keys[2], vals[2]
  b += align256((size_t)P * sizeof(float2));   // pay[1]
  b += align256((size_t)hist_n * 4);
  b += align256((size_t)aux_n * 4);
  b += align256((size_t)(HN + 2) * 4);         // key_ptr
  return b;
}

void sort_scratch_carve(void* base, float2* pairs, int64_t P, int64_t HN, SortScratch* sc) {
  const int64_t nblk = ceil_div(P, SORT_TILE);
  const int64_t hist_n = (int64_t)SORT_BINS * nblk;
  const int64_t aux_n = scan_aux_elems(hist_n);
  char* p = static_cast<char*>(base);
  sc->keys[0] = reinterpret_cast<uint32_t*>(p); p += align256((size_t)P * 4);
  sc->keys[1] = reinterpret_cast<uint32_t*>(p); p += align256((size_t)P * 4);
  sc->vals[0] = reinterpret_cast<uint32_t*>(p); p += align256((size_t)P * 4);
  sc->vals[1] = reinterpret_cast<uint32_t*>(p); p += align256((size_t)P * 4);
  sc->pay[0] = pairs;
  sc->pay[1] = reinterpret_cast<float2*>(p); p += align256((size_t)P * sizeof(float2));
  sc->hist = reinterpret_cast<int32_t*>(p); p += align256((size_t)hist_n * 4);
  sc->scan_aux = reinterpret_cast<int32_t*>(p); p += align256((size_t)aux_n * 4);
  sc->key_ptr = reinterpret_cast<int32_t*>(p);
  sc->final_buf = 0;
}

hipError_t launch_selection_transpose(const int32_t* topk_idx, int64_t N, int H, int topk,
                                      SortScratch* sc, hipStream_t s) {
  const int64_t P = N * H * topk;
  const int64_t HN = N * H;
  const int64_t nblk = ceil_div(P, SORT_TILE);
  const int passes = sort_passes(HN);
  hipError_t e = hipSuccess;
  int cur = 0;
  for (int ps = 0; ps < passes; ++ps) {
    const int shift = ps * SORT_BITS;
    // Pass 0 reads topk_idx and the caller's pairs (pay[0]); later passes
    // ping-pong between the buffer pairs.
    const uint32_t* kin = ps == 0 ? nullptr : sc->keys[cur];
    const uint32_t* vin = ps == 0 ? nullptr : sc->vals[cur];
    hipLaunchKernelGGL(radix_hist_kernel, dim3((unsigned)nblk), dim3(SORT_THREADS), 0, s, kin,
                       topk_idx, N, H, topk, P, shift, sc->hist, nblk);
    e = launch_exclusive_scan(sc->hist, sc->hist, (int64_t)SORT_BINS * nblk, sc->scan_aux, s);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(radix_scatter_kernel, dim3((unsigned)nblk), dim3(SORT_THREADS), 0, s,
                       kin, vin, sc->pay[cur], topk_idx, N, H, topk, P, shift, sc->hist, nblk,
                       sc->keys[cur ^ 1], sc->vals[cur ^ 1], sc->pay[cur ^ 1]);
    cur ^= 1;
  }
  sc->final_buf = cur;
  hipLaunchKernelGGL(key_ptr_kernel, dim3((unsigned)ceil_div(HN + 2, 256)), dim3(256), 0, s,
                     sc->keys[cur], P, HN + 2, sc->key_ptr);
  return hipGetLastError();
}

size_t segreduce_scratch_bytes(int64_t P, int d) {
  const int64_t nslices = ceil_div(P, SEG_SLICE);
  return align256((size_t)nslices * 2 * 2 * d * sizeof(double));
}

namespace {
template <int D, typename QT>
void launch_keys_t(const QT* q, const float* dout, int64_t N, int H, int topk,
                   const SortScratch* sc, double* partials, float* dk, float* dv,
                   hipStream_t s) {
  const int64_t P = N * H * topk;
  const int64_t HN = N * H;
  const int64_t nslices = ceil_div(P, SEG_SLICE);
  const unsigned b1 = (unsigned)ceil_div(nslices, SEG_GROUPS);
  const unsigned b2 = (unsigned)ceil_div(HN, SEG_GROUPS);
  hipLaunchKernelGGL((segreduce_kernel<D, QT>), dim3(b1), dim3(256), 0, s, q, dout,
                     sc->pay[sc->final_buf], sc->keys[sc->final_buf], sc->vals[sc->final_buf],
                     sc->key_ptr, N, H, topk, nslices, partials, dk, dv);
  hipLaunchKernelGGL(segfix_kernel<D>, dim3(b2), dim3(256), 0, s, sc->key_ptr, N, H, partials,
                     dk, dv);
}
}  // namespace

hipError_t launch_bwd_keys(const void* q, bool q_f32, const float* dout, int64_t N, int H,
                           int d, int topk, const SortScratch* sc, double* partials, float* dk,
                           float* dv, hipStream_t s) {
  const uint16_t* qb = static_cast<const uint16_t*>(q);
  const float* qf = static_cast<const float*>(q);
  if (d == 32 && !q_f32) launch_keys_t<32>(qb, dout, N, H, topk, sc, partials, dk, dv, s);
  else if (d == 32) launch_keys_t<32>(qf, dout, N, H, topk, sc, partials, dk, dv, s);
  else if (d == 64 && !q_f32) launch_keys_t<64>(qb, dout, N, H, topk, sc, partials, dk, dv, s);
  else if (d == 64) launch_keys_t<64>(qf, dout, N, H, topk, sc, partials, dk, dv, s);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace kmip
