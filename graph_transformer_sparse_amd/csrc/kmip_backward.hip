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
//  1. a stable LSD radix sort orders the pairs (row*k + slot) by the key
//     h*N + j (padding slots get the sentinel H*N); within a key the pairs
//     stay in ascending pair id, i.e. ascending query.  Digits are up to 11
//     bits wide, so keys of up to 22 bits (N*H < 4M) take two passes.  The
//     first pass derives the keys from topk_idx and the pair ids from
//     positions; every pass carries the pair's (p, ds), so the reduction
//     reads them in sorted order instead of gathering 8 bytes per pair;
//  2. key segment pointers come from a search of the sorted keys, confined
//     to the range of the key's top digit;
//  3. fixed-length slices of the sorted pairs are reduced by 16-lane groups
//     (no atomics).  Runs that cover a whole key segment are written
//     directly; runs cut by a slice boundary go to per-slice partials, which
//     a fix-up pass adds in slice order.  Keys selected by no query get exact
//     zeros.  Every sum has a fixed order, so results are bitwise repeatable.
#include <algorithm>

#include "kmip_cols.h"
#include "kmip_internal.h"

namespace kmip {
namespace {

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
template <int NT = SCAN_THREADS>
__device__ __forceinline__ int32_t block_excl_scan(int32_t x, int32_t* sh, int32_t* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int32_t incl = wave_incl_scan(x, lane);
  if (lane == 63) sh[wave] = incl;
  __syncthreads();
  int32_t base = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) {
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
// Each pass is a stable counting sort on one digit of the key:
//  - radix_hist_kernel counts the digits of each tile of SORT_TILE pairs
//    into one contiguous row of hist ([tile][bin]);
//  - col_reduce / col_scan / col_down turn the rows into output offsets:
//    tile r's run of digit b starts at (pairs of smaller digits) + (digit b
//    in tiles before r);
//  - radix_scatter_kernel ranks the tile's pairs by digit (stable) and
//    writes every digit's run at its offset.

// First pass: the key of pair pid (pair ids < 2^31), from its entry j of
// topk_idx.
__device__ __forceinline__ uint32_t pair_key_of(int32_t j, uint32_t pid, uint32_t N, uint32_t H,
                                                uint32_t topk) {
  const uint32_t h = (pid / topk) % H;
  return j < 0 ? N * H : h * N + (uint32_t)j;
}

__global__ __launch_bounds__(SORT_THREADS) void radix_hist_kernel(
    const uint32_t* __restrict__ keys, const int32_t* __restrict__ idx, uint32_t N, uint32_t H,
    uint32_t topk, uint32_t P, int shift, int bits, int32_t* __restrict__ hist) {
  __shared__ int32_t cnt[SORT_MAX_BINS];
  const int nb = 1 << bits;
  const uint32_t mask = (uint32_t)nb - 1u;
  for (int b = threadIdx.x; b < nb; b += SORT_THREADS) cnt[b] = 0;
  const uint32_t base = blockIdx.x * (uint32_t)SORT_TILE;
  // Loads are unconditional (positions past P read the last pair and are
  // dropped below), so all of them are in flight together.
  uint32_t k[SORT_ITEMS];
  if (keys != nullptr) {
#pragma unroll
    for (int i = 0; i < SORT_ITEMS; ++i) {
      const uint32_t e = base + i * SORT_THREADS + threadIdx.x;
      k[i] = keys[e < P ? e : P - 1];
    }
  } else {
    int32_t j[SORT_ITEMS];
#pragma unroll
    for (int i = 0; i < SORT_ITEMS; ++i) {
      const uint32_t e = base + i * SORT_THREADS + threadIdx.x;
      j[i] = idx[e < P ? e : P - 1];
    }
#pragma unroll
    for (int i = 0; i < SORT_ITEMS; ++i) {
      const uint32_t e = base + i * SORT_THREADS + threadIdx.x;
      k[i] = pair_key_of(j[i], e < P ? e : P - 1, N, H, topk);
    }
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < SORT_ITEMS; ++i)
    if (base + i * SORT_THREADS + threadIdx.x < P) atomicAdd(&cnt[(k[i] >> shift) & mask], 1);
  __syncthreads();
  int32_t* row = hist + (int64_t)blockIdx.x * nb;
  for (int b = threadIdx.x; b < nb; b += SORT_THREADS) row[b] = cnt[b];
}

// colsum[g][bin] = sum of hist[r][bin] over the rg tiles r of group g.
__global__ __launch_bounds__(256) void col_reduce_kernel(const int32_t* __restrict__ hist,
                                                         int nblk, int nb, int rg,
                                                         int32_t* __restrict__ colsum) {
  const int bin = blockIdx.y * 256 + threadIdx.x;
  if (bin >= nb) return;
  const int r0 = blockIdx.x * rg;
  const int r1 = r0 + rg < nblk ? r0 + rg : nblk;
  int32_t s[4] = {0, 0, 0, 0};
  int r = r0;
  for (; r + 4 <= r1; r += 4) {
#pragma unroll
    for (int u = 0; u < 4; ++u) s[u] += hist[(int64_t)(r + u) * nb + bin];
  }
  for (; r < r1; ++r) s[0] += hist[(int64_t)r * nb + bin];
  colsum[(int64_t)blockIdx.x * nb + bin] = (s[0] + s[1]) + (s[2] + s[3]);
}

// Per bin (one thread each): colsum[g][bin] becomes the exclusive prefix of
// the column over the groups, bintot[bin] its total.  The column (at most
// COL_MAX_GROUPS values) is read with independent loads, all in flight
// together (groups past ng re-read the last one and are masked).
constexpr int COL_MAX_GROUPS = 64;
__global__ __launch_bounds__(256) void col_scan_kernel(int32_t* __restrict__ colsum, int ng,
                                                       int nb, int32_t* __restrict__ bintot) {
  const int bin = blockIdx.x * 256 + threadIdx.x;
  if (bin >= nb) return;
  int32_t c[COL_MAX_GROUPS];
  const int32_t* col = colsum + bin;
#pragma unroll
  for (int g = 0; g < COL_MAX_GROUPS; ++g) {
    c[g] = *col;
    col += g + 1 < ng ? nb : 0;
  }
  int32_t* out = colsum + bin;
  int32_t run = 0;
#pragma unroll
  for (int g = 0; g < COL_MAX_GROUPS; ++g) {
    if (g < ng) {
      *out = run;
      out += nb;
      run += c[g];
    }
  }
  bintot[bin] = run;
}

// hist[r][bin] becomes the output offset of tile r's run of digit bin: the
// start of the digit in the pass output (an exclusive scan of the bin totals,
// done by every workgroup for itself: at most 2048 values), plus the column
// prefix of the tile's group, plus the digit's counts in the group's earlier
// tiles.  The workgroups of group 0 also write binbase[bin] = the digit's
// start, binbase[nb] = P.
__global__ __launch_bounds__(256) void col_down_kernel(int32_t* __restrict__ hist, int nblk,
                                                       int nb, int rg,
                                                       const int32_t* __restrict__ colsum,
                                                       const int32_t* __restrict__ bintot,
                                                       int32_t* __restrict__ binbase) {
  __shared__ int32_t sh[256 / 64];
  __shared__ int32_t starts[SORT_MAX_BINS];
  // bins [t*bpt, t*bpt + bpt) per thread
  const int bpt = nb > 256 ? nb / 256 : 1;
  const int b0 = threadIdx.x * bpt;
  int32_t mine = 0;
  for (int i = 0; i < bpt; ++i)
    if (b0 + i < nb) mine += bintot[b0 + i];
  int32_t total;
  int32_t st = block_excl_scan(mine, sh, &total);
  for (int i = 0; i < bpt; ++i) {
    if (b0 + i < nb) {
      starts[b0 + i] = st;
      st += bintot[b0 + i];
    }
  }
  __syncthreads();
  const int bin = blockIdx.y * 256 + threadIdx.x;
  if (bin >= nb) return;
  if (blockIdx.x == 0) {
    binbase[bin] = starts[bin];
    if (bin == 0) binbase[nb] = total;
  }
  const int r0 = blockIdx.x * rg;
  const int r1 = r0 + rg < nblk ? r0 + rg : nblk;
  int32_t run = starts[bin] + colsum[(int64_t)blockIdx.x * nb + bin];
  int r = r0;
  for (; r + 4 <= r1; r += 4) {
    int32_t c[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) c[u] = hist[(int64_t)(r + u) * nb + bin];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      hist[(int64_t)(r + u) * nb + bin] = run;
      run += c[u];
    }
  }
  for (; r < r1; ++r) {
    const int32_t c = hist[(int64_t)r * nb + bin];
    hist[(int64_t)r * nb + bin] = run;
    run += c;
  }
}

// Stable scatter of one tile (SORT_TILE pairs, SCATTER_THREADS threads).
// Wave w ranks the pairs [tile + w*512, +512) in order, 64 at a time: equal
// digits inside a 64-pair chunk are found with one ballot per digit bit, and
// a per-wave running count per digit carries the rank across chunks.  The
// counts are then turned into tile positions (digits in order, waves in
// order within a digit), the tile is staged in LDS in that order, and each
// digit's run is written at its offset: consecutive lanes write consecutive
// addresses.  Keys and pair ids are staged and written first, then p, then
// ds, through the same LDS space.
// First pass (keys_in == nullptr): keys come from topk_idx and pair ids are
// the positions.
constexpr int SCATTER_THREADS = 512;
__global__ __launch_bounds__(SCATTER_THREADS) void radix_scatter_kernel(
    const uint32_t* __restrict__ keys_in, const uint32_t* __restrict__ vals_in,
    const float2* __restrict__ pay_in, const int32_t* __restrict__ idx, uint32_t N, uint32_t H,
    uint32_t topk, uint32_t P, int shift, int bits, const int32_t* __restrict__ offs,
    uint32_t* __restrict__ keys_out, uint32_t* __restrict__ vals_out,
    float2* __restrict__ pay_out) {
  constexpr int NT = SCATTER_THREADS;
  constexpr int NW = NT / 64;
  constexpr int PER_WAVE = SORT_TILE / NW;
  constexpr int CHUNKS = PER_WAVE / 64;
  __shared__ uint16_t wcnt[NW][SORT_MAX_BINS];
  __shared__ int32_t gm[SORT_MAX_BINS];   // output offset of the digit minus its tile start
  __shared__ uint32_t lk[SORT_TILE];
  __shared__ uint32_t lv[SORT_TILE];      // pair ids, then p, then ds
  __shared__ int32_t sh[NW];
  float* lf = reinterpret_cast<float*>(lv);
  float* po = reinterpret_cast<float*>(pay_out);
  // Workgroups are dealt to the 8 XCDs in turn (the grid is a multiple of 8);
  // XCD x takes the x-th eighth of the tiles.  Consecutive tiles write
  // adjacent pieces of every digit's run, so a cache line of the output is
  // then filled inside one XCD's L2 rather than written back in parts by
  // several.
  const uint32_t tile = (blockIdx.x % 8) * (gridDim.x / 8) + blockIdx.x / 8;
  if (tile >= (P + SORT_TILE - 1) / SORT_TILE) return;
  const int nb = 1 << bits;
  const uint32_t mask = (uint32_t)nb - 1u;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int b = threadIdx.x; b < nb; b += NT) {
#pragma unroll
    for (int w = 0; w < NW; ++w) wcnt[w][b] = 0;
    gm[b] = offs[(int64_t)tile * nb + b];
  }
  const uint32_t wbase = tile * (uint32_t)SORT_TILE + (uint32_t)wave * PER_WAVE;
  // Loads are unconditional (positions past P read the last pair and are
  // dropped below), so all of them are in flight together.
  uint32_t k[CHUNKS], v[CHUNKS];
  float2 pl[CHUNKS];
  if (keys_in != nullptr) {
#pragma unroll
    for (int c = 0; c < CHUNKS; ++c) {
      const uint32_t e = wbase + c * 64 + lane;
      const uint32_t ec = e < P ? e : P - 1;
      k[c] = keys_in[ec];
      v[c] = vals_in[ec];
      pl[c] = pay_in[ec];
    }
  } else {
    int32_t j[CHUNKS];
#pragma unroll
    for (int c = 0; c < CHUNKS; ++c) {
      const uint32_t e = wbase + c * 64 + lane;
      v[c] = e < P ? e : P - 1;
      j[c] = idx[v[c]];
      pl[c] = pay_in[v[c]];
    }
#pragma unroll
    for (int c = 0; c < CHUNKS; ++c) k[c] = pair_key_of(j[c], v[c], N, H, topk);
  }
  __syncthreads();

  const uint64_t lt = (1ull << lane) - 1ull;
  int32_t lp[CHUNKS];
#pragma unroll
  for (int c = 0; c < CHUNKS; ++c) {
    const bool valid = wbase + c * 64 + lane < P;
    const int dg = (int)((k[c] >> shift) & mask);
    uint64_t peers = __ballot(valid);
    for (int b = 0; b < bits; ++b) {
      const int bit = (dg >> b) & 1;
      const uint64_t bal = __ballot(bit);
      peers &= bit ? bal : ~bal;
    }
    const int32_t before = wcnt[wave][dg];
    lp[c] = before + __popcll(peers & lt);
    const bool leader = valid && (lane == 63 || (peers >> (lane + 1)) == 0ull);
    if (leader) wcnt[wave][dg] = (uint16_t)(before + __popcll(peers));
  }
  __syncthreads();

  // Tile start of every digit (thread t owns digits [t*bpt, t*bpt + bpt)),
  // then each wave's start within the digit.
  const int bpt = nb > NT ? nb / NT : 1;
  const int d0 = threadIdx.x * bpt;
  int32_t mine = 0;
  for (int i = 0; i < bpt; ++i) {
    const int b = d0 + i;
    if (b < nb) {
#pragma unroll
      for (int w = 0; w < NW; ++w) mine += wcnt[w][b];
    }
  }
  int32_t tile_total;
  int32_t start = block_excl_scan<NT>(mine, sh, &tile_total);
  for (int i = 0; i < bpt; ++i) {
    const int b = d0 + i;
    if (b < nb) {
      gm[b] -= start;
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        const int32_t c = wcnt[w][b];
        wcnt[w][b] = (uint16_t)start;
        start += c;
      }
    }
  }
  __syncthreads();

#pragma unroll
  for (int c = 0; c < CHUNKS; ++c) {
    if (wbase + c * 64 + lane < P) {
      const int dg = (int)((k[c] >> shift) & mask);
      lp[c] += wcnt[wave][dg];
      lk[lp[c]] = k[c];
      lv[lp[c]] = v[c];
    }
  }
  __syncthreads();
  for (int i = threadIdx.x; i < tile_total; i += NT) {
    const uint32_t kk = lk[i];
    const int64_t pos = (int64_t)gm[(kk >> shift) & mask] + i;
    keys_out[pos] = kk;
    vals_out[pos] = lv[i];
  }
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    __syncthreads();
#pragma unroll
    for (int c = 0; c < CHUNKS; ++c)
      if (wbase + c * 64 + lane < P) lf[lp[c]] = half == 0 ? pl[c].x : pl[c].y;
    __syncthreads();
    for (int i = threadIdx.x; i < tile_total; i += NT) {
      const int64_t pos = (int64_t)gm[(lk[i] >> shift) & mask] + i;
      po[2 * pos + half] = lf[i];
    }
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
  // Workgroups are dealt to the 8 XCDs in turn; XCD x takes the x-th eighth
  // of the slices, a contiguous range of keys (at most a few heads), so the
  // q and dO rows it gathers come from fewer queries.
  const int64_t per_xcd = gridDim.x / 8;
  const int64_t lblock = (int64_t)(blockIdx.x % 8) * per_xcd + blockIdx.x / 8;
  const int64_t slice = lblock * SEG_GROUPS + (threadIdx.x >> 4);
  if (slice >= nslices) return;
  const int64_t HN = N * H;
  const int64_t valid_end = key_ptr[HN];
  const int64_t s0 = slice * SEG_SLICE;
  if (s0 >= valid_end) return;
  const int64_t s1 = s0 + SEG_SLICE < valid_end ? s0 + SEG_SLICE : valid_end;
  const int n = (int)(s1 - s0);
  // The keys just before and after the slice tell whether its first run
  // starts a segment and whether its last run ends one.
  const uint32_t kprev = skeys[s0 > 0 ? s0 - 1 : 0];
  const uint32_t knext = skeys[s1 < valid_end ? s1 : s1 - 1];

  double ak[EPL], av[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) ak[e] = av[e] = 0.0;

  // Run [ra, rb) of key: a whole segment is written out; a run cut by the
  // slice boundary goes to the slice's partials (slot 0: the run that starts
  // the slice; slot 1: a later run, which then ends the slice).
  auto flush = [&](uint32_t key, int64_t ra, int64_t rb) __attribute__((always_inline)) {
    const bool starts = ra > s0 || s0 == 0 || kprev != key;
    const bool ends = rb < s1 || s1 == valid_end || knext != key;
    if (starts && ends) {
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
  // of the group holds pairs s0 + 16 i + l (positions past the slice repeat
  // its last pair, so every load is unconditional and all are in flight
  // together).  The loop then takes them by shuffles and requests the q and
  // dO rows of SEG_BATCH pairs at a time.
  constexpr int PER_LANE = SEG_SLICE / 16;
  constexpr int SEG_BATCH = 8;
  uint32_t mk[PER_LANE], mv[PER_LANE];
  float mpx[PER_LANE], mpy[PER_LANE];
#pragma unroll
  for (int i = 0; i < PER_LANE; ++i) {
    const int u = i * 16 + l16;
    const int64_t t = s0 + (u < n ? u : n - 1);
    mk[i] = skeys[t];
    mv[i] = svals[t];
    const float2 pr = spay[t];
    mpx[i] = pr.x;
    mpy[i] = pr.y;
  }
  uint32_t cur = __shfl(mk[0], 0, 16);
  int64_t run0 = s0;
#pragma unroll
  for (int g = 0; g < SEG_SLICE; g += SEG_BATCH) {
    if (g >= n) break;
    uint32_t key[SEG_BATCH];
    float px[SEG_BATCH], py[SEG_BATCH], qx[SEG_BATCH][EPL], gx[SEG_BATCH][EPL];
#pragma unroll
    for (int u = 0; u < SEG_BATCH; ++u) {
      const int ip = g + u, i = ip / 16, src = ip % 16;
      key[u] = __shfl(mk[i], src, 16);
      const uint32_t pid = __shfl(mv[i], src, 16);
      px[u] = __shfl(mpx[i], src, 16);
      py[u] = __shfl(mpy[i], src, 16);
      const int64_t row = pid / (uint32_t)topk;
      load_cols<EPL>(Q + row * D + l16 * EPL, qx[u]);
      load_cols<EPL>(dout + row * D + l16 * EPL, gx[u]);
    }
#pragma unroll
    for (int u = 0; u < SEG_BATCH; ++u) {
      const int ip = g + u;
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

// One 16-lane group per SEGFIX_KEYS consecutive keys: zeros for unselected
// keys, and the in-order sum of slice partials for keys whose segment
// crosses a slice boundary (keys inside one slice were written by
// segreduce_kernel).  The group reads the keys' segment pointers with one
// load and takes them by shuffles.
constexpr int SEGFIX_KEYS = 8;
template <int D>
__global__ __launch_bounds__(256) void segfix_kernel(const int32_t* __restrict__ key_ptr,
                                                     int64_t N, int H,
                                                     const double* __restrict__ partials,
                                                     float* __restrict__ dk,
                                                     float* __restrict__ dv) {
  constexpr int EPL = D / 16;
  const int l16 = threadIdx.x & 15;
  const int64_t HN = N * H;
  const int64_t key0 = ((int64_t)blockIdx.x * SEG_GROUPS + (threadIdx.x >> 4)) * SEGFIX_KEYS;
  if (key0 >= HN) return;
  // key_ptr has H*N + 2 entries; lanes past the end re-read the last one
  const int64_t pk = key0 + l16 <= HN + 1 ? key0 + l16 : HN + 1;
  const int32_t kp = key_ptr[pk];
#pragma unroll
  for (int i = 0; i < SEGFIX_KEYS; ++i) {
    const int64_t key = key0 + i;
    if (key >= HN) break;
    const int64_t a = __shfl(kp, i, 16), b = __shfl(kp, i + 1, 16);
    const int64_t sa = a / SEG_SLICE, sb = (b - 1) / SEG_SLICE;
    if (a < b && sa == sb) continue;          // written by segreduce_kernel
    const int64_t orow = (key % N) * H + key / N;
    double ak[EPL], av[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) ak[e] = av[e] = 0.0;
    if (a < b) {
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
}

// key_ptr[key] = first position of the sorted keys that is >= key, for key
// in [0, H*N + 1]: the segment of key is [key_ptr[key], key_ptr[key + 1]).
// The last pass sorted on the top digit, so the search is confined to the
// range of the key's top digit, binbase[top] .. binbase[top + 1].
__global__ void key_ptr_kernel(const uint32_t* __restrict__ skeys, uint32_t nkeys, int shift,
                               int nb, const int32_t* __restrict__ binbase,
                               int32_t* __restrict__ key_ptr) {
  const uint32_t key = blockIdx.x * blockDim.x + threadIdx.x;
  if (key >= nkeys) return;
  const uint32_t top = key >> shift;
  uint32_t lo, hi;
  if (top >= (uint32_t)nb) {
    lo = hi = (uint32_t)binbase[nb];
  } else {
    lo = (uint32_t)binbase[top];
    hi = (uint32_t)binbase[top + 1];
  }
  while (lo < hi) {
    const uint32_t mid = lo + ((hi - lo) >> 1);
    if (skeys[mid] < key) lo = mid + 1; else hi = mid;
  }
  key_ptr[key] = (int32_t)lo;
}

// Digit plan: the keys (sentinel H*N included) span `bits` bits, sorted low
// digit first in passes of at most SORT_MAX_BITS bits, widths as equal as
// possible (the first pass is the widest).
struct SortPlan {
  int passes;
  int shift[3], bits[3];
  int tiles, row_group, groups;
};

SortPlan sort_plan(int64_t P, int64_t max_key) {
  int bits = 1;
  while ((max_key >> bits) != 0) ++bits;
  SortPlan p{};
  p.passes = (bits + SORT_MAX_BITS - 1) / SORT_MAX_BITS;
  int sh = 0;
  for (int i = 0; i < p.passes; ++i) {
    const int left = p.passes - i;
    const int b = (bits - sh + left - 1) / left;
    p.shift[i] = sh;
    p.bits[i] = b;
    sh += b;
  }
  p.tiles = (int)ceil_div(P, SORT_TILE);
  // at most COL_MAX_GROUPS row groups: col_scan_kernel holds a column in registers
  p.row_group = (int)std::max<int64_t>(16, ceil_div(p.tiles, COL_MAX_GROUPS));
  p.groups = (int)ceil_div(p.tiles, p.row_group);
  return p;
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
  const SortPlan pl = sort_plan(P, HN);
  const int64_t bins = (int64_t)1 << pl.bits[0];
  size_t b = 0;
  b += 4 * align256((size_t)P * 4);            // keys[2], vals[2]
  b += align256((size_t)P * sizeof(float2));   // pay[1]
  b += align256((size_t)pl.tiles * bins * 4);  // hist
  b += align256((size_t)pl.groups * bins * 4); // colsum
  b += align256((size_t)(bins + 1) * 4);       // binbase
  b += align256((size_t)bins * 4);             // bintot
  b += align256((size_t)(HN + 2) * 4);         // key_ptr
  return b;
}

void sort_scratch_carve(void* base, float2* pairs, int64_t P, int64_t HN, SortScratch* sc) {
  const SortPlan pl = sort_plan(P, HN);
  const int64_t bins = (int64_t)1 << pl.bits[0];
  char* p = static_cast<char*>(base);
  sc->keys[0] = reinterpret_cast<uint32_t*>(p); p += align256((size_t)P * 4);
  sc->keys[1] = reinterpret_cast<uint32_t*>(p); p += align256((size_t)P * 4);
  sc->vals[0] = reinterpret_cast<uint32_t*>(p); p += align256((size_t)P * 4);
  sc->vals[1] = reinterpret_cast<uint32_t*>(p); p += align256((size_t)P * 4);
  sc->pay[0] = pairs;
  sc->pay[1] = reinterpret_cast<float2*>(p); p += align256((size_t)P * sizeof(float2));
  sc->hist = reinterpret_cast<int32_t*>(p); p += align256((size_t)pl.tiles * bins * 4);
  sc->colsum = reinterpret_cast<int32_t*>(p); p += align256((size_t)pl.groups * bins * 4);
  sc->binbase = reinterpret_cast<int32_t*>(p); p += align256((size_t)(bins + 1) * 4);
  sc->bintot = reinterpret_cast<int32_t*>(p); p += align256((size_t)bins * 4);
  sc->key_ptr = reinterpret_cast<int32_t*>(p);
  sc->final_buf = 0;
}

hipError_t launch_selection_transpose(const int32_t* topk_idx, int64_t N, int H, int topk,
                                      SortScratch* sc, hipStream_t s) {
  const int64_t P = N * H * topk;
  const int64_t HN = N * H;
  const SortPlan pl = sort_plan(P, HN);
  const uint32_t n32 = (uint32_t)N, h32 = (uint32_t)H, k32 = (uint32_t)topk, p32 = (uint32_t)P;
  int cur = 0;
  for (int ps = 0; ps < pl.passes; ++ps) {
    const int shift = pl.shift[ps], bits = pl.bits[ps], nb = 1 << bits;
    const dim3 cols((unsigned)pl.groups, (unsigned)ceil_div(nb, 256));
    // Pass 0 reads topk_idx and the caller's pairs (pay[0]); later passes
    // ping-pong between the buffer pairs.
    const uint32_t* kin = ps == 0 ? nullptr : sc->keys[cur];
    const uint32_t* vin = ps == 0 ? nullptr : sc->vals[cur];
    hipLaunchKernelGGL(radix_hist_kernel, dim3((unsigned)pl.tiles), dim3(SORT_THREADS), 0, s,
                       kin, topk_idx, n32, h32, k32, p32, shift, bits, sc->hist);
    hipLaunchKernelGGL(col_reduce_kernel, cols, dim3(256), 0, s, sc->hist, pl.tiles, nb,
                       pl.row_group, sc->colsum);
    hipLaunchKernelGGL(col_scan_kernel, dim3((unsigned)ceil_div(nb, 256)), dim3(256), 0, s,
                       sc->colsum, pl.groups, nb, sc->bintot);
    hipLaunchKernelGGL(col_down_kernel, cols, dim3(256), 0, s, sc->hist, pl.tiles, nb,
                       pl.row_group, sc->colsum, sc->bintot, sc->binbase);
    hipLaunchKernelGGL(radix_scatter_kernel, dim3((unsigned)(8 * ceil_div(pl.tiles, 8))),
                       dim3(SCATTER_THREADS), 0, s,
                       kin, vin, sc->pay[cur], topk_idx, n32, h32, k32, p32, shift, bits,
                       sc->hist, sc->keys[cur ^ 1], sc->vals[cur ^ 1], sc->pay[cur ^ 1]);
    cur ^= 1;
  }
  sc->final_buf = cur;
  const int last = pl.passes - 1;
  hipLaunchKernelGGL(key_ptr_kernel, dim3((unsigned)ceil_div(HN + 2, 256)), dim3(256), 0, s,
                     sc->keys[cur], (uint32_t)(HN + 2), pl.shift[last], 1 << pl.bits[last],
                     sc->binbase, sc->key_ptr);
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
  const unsigned b1 = (unsigned)(8 * ceil_div(ceil_div(nslices, SEG_GROUPS), 8));
  const unsigned b2 = (unsigned)ceil_div(HN, SEG_GROUPS * SEGFIX_KEYS);
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
