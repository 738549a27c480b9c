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
// Queries of one head are grouped by their nearest pivot: npiv query rows of
// the head, at evenly spaced node ids (about one per 96 nodes, so a group
// fills about three wavefronts; a multiple of 32, at least 32), and a query's
// group is the pivot with the largest inner product (the lowest pivot index
// on ties).  The 32 queries of a wavefront then tend to point the same way
// and share their few high-scoring keys, so the selection pass meets far
// fewer 32-key blocks holding a candidate for any of its queries.  The order
// only changes which queries share a wavefront; every query's result is
// independent of it.
//
// The groups themselves are placed in the order of a pivot rank: pivots are
// sorted by their nearest anchor (ORDER_ANCHORS pivots at even spacing, the
// lowest anchor index on ties), stably by pivot index.  Pivots that point the
// same way share an anchor, so the groups of one cluster of similar queries
// sit next to each other in the order, and a window of nearby positions holds
// most of a query's similar nodes (the threshold window in the scan uses
// this).
constexpr int ORDER_PIVOTS = 1024;                // pivots staged in LDS at a time
constexpr int ORDER_ANCHORS = 64;
constexpr int ORDER_MAX_PIVOTS = 16384;           // codes are 16-bit
int order_pivots(int64_t N) {
  const int64_t p = (N / 96) & ~int64_t(31);
  return (int)(p < 32 ? 32 : p > ORDER_MAX_PIVOTS ? ORDER_MAX_PIVOTS : p);
}
constexpr int ORDER_WAVES = 8;                    // wavefronts per workgroup
constexpr int ORDER_QB = 2;                       // blocks of 32 queries per wavefront
// Each (head, pivot) count is split over ORDER_COPIES counters picked by the
// node id, which keeps atomic contention low when many queries share a pivot.

__global__ void fill_zero_kernel(int32_t* __restrict__ p, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0;
}

// Node id of pivot p of a head: evenly spaced, clamped to the last node.
__device__ __forceinline__ int64_t pivot_node(int p, int64_t N, int npiv) {
  const int64_t stride = N / npiv > 0 ? N / npiv : 1;
  const int64_t r = (int64_t)p * stride;
  return r < N ? r : N - 1;
}

// anchor[h*npiv + p] = the anchor (pivot a * (npiv / ORDER_ANCHORS)) with the
// largest inner product with pivot p, over the first DP elements of the rows
// (fp32 sums of exact bf16 products, in element order).  One thread per pivot.
template <int D, int DP>
__global__ __launch_bounds__(256) void pivot_anchor_kernel(const uint16_t* __restrict__ Q,
                                                           int64_t N, int H, int npiv,
                                                           uint8_t* __restrict__ anchor) {
  __shared__ float av[ORDER_ANCHORS][DP];
  const int h = blockIdx.y;
  const int nanch = npiv < ORDER_ANCHORS ? npiv : ORDER_ANCHORS;
  const int astep = npiv / nanch;
  for (int t = threadIdx.x; t < nanch * DP; t += blockDim.x) {
    const int a = t / DP, c = t % DP;
    const int64_t row = pivot_node(a * astep, N, npiv);
    av[a][c] = __uint_as_float((uint32_t)Q[(row * H + h) * D + c] << 16);
  }
  __syncthreads();
  const int p = blockIdx.x * blockDim.x + threadIdx.x;
  if (p >= npiv) return;
  const uint16_t* qp = Q + (pivot_node(p, N, npiv) * H + h) * D;
  float x[DP];
#pragma unroll
  for (int c = 0; c < DP; ++c) x[c] = __uint_as_float((uint32_t)qp[c] << 16);
  float best = -__builtin_inff();
  int ba = 0;
  for (int a = 0; a < nanch; ++a) {
    float sc = 0.f;
#pragma unroll
    for (int c = 0; c < DP; ++c) sc = fmaf(x[c], av[a][c], sc);
    if (sc > best) {
      best = sc;
      ba = a;
    }
  }
  anchor[(int64_t)h * npiv + p] = (uint8_t)ba;
}

// prank[h*npiv + p] = position of pivot p when the head's pivots are sorted by
// (anchor, pivot index).  One wavefront per head: the anchors are counted
// (LDS atomics), scanned, and then the pivots are numbered 64 at a time in
// index order, a pivot's place among equal anchors of its 64 coming from six
// ballots.
__global__ __launch_bounds__(64) void pivot_rank_kernel(const uint8_t* __restrict__ anchor,
                                                        int npiv, int32_t* __restrict__ prank) {
  __shared__ int32_t cnt[ORDER_ANCHORS];
  __shared__ int32_t next[ORDER_ANCHORS];
  static_assert(ORDER_ANCHORS == 64, "one anchor per lane");
  const int h = blockIdx.x, lane = threadIdx.x;
  const uint8_t* an = anchor + (int64_t)h * npiv;
  cnt[lane] = 0;
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_wave_barrier();
  for (int p = lane; p < npiv; p += 64) atomicAdd(&cnt[an[p]], 1);
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "workgroup");
  __builtin_amdgcn_wave_barrier();
  int32_t x = cnt[lane], incl = x;                // exclusive scan over the 64 anchors
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int32_t y = __shfl_up(incl, o, 64);
    if (lane >= o) incl += y;
  }
  next[lane] = incl - x;
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "workgroup");
  __builtin_amdgcn_wave_barrier();
  const uint64_t lt = (1ull << lane) - 1ull;
  for (int base = 0; base < npiv; base += 64) {
    const int p = base + lane;
    const bool valid = p < npiv;
    const int g = valid ? an[p] : 0;
    uint64_t peers = __ballot(valid);
#pragma unroll
    for (int bit = 0; bit < 6; ++bit) {
      const uint64_t bal = __ballot((g >> bit) & 1);
      peers &= ((g >> bit) & 1) ? bal : ~bal;
    }
    const int32_t first = next[g];
    if (valid) prank[(int64_t)h * npiv + p] = first + __popcll(peers & lt);
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "workgroup");
    __builtin_amdgcn_wave_barrier();
    const bool leader = valid && (peers >> lane) == 1ull;   // last lane of its anchor
    if (leader) next[g] = first + __popcll(peers);
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "workgroup");
    __builtin_amdgcn_wave_barrier();
  }
}

// codes[h*N + i] = rank of the nearest pivot of query i of head h, and
// per-(head, pivot rank) counts.  Rows hold D bf16 elements; the inner products use the first DP
// (for split-precision rows, the high parts).  The workgroup stages the
// head's pivots in LDS, ORDER_PIVOTS at a time, in MFMA operand order
// (block j*NM + m: pivots [32j, 32j + 32) of the batch, elements
// [16m, 16m + 16)); each wavefront scores its ORDER_QB blocks of 32 queries
// against all of them with 32x32x16 MFMAs, keys' role taken by the pivots.
// npiv is a multiple of 32.
template <int D, int DP>
__global__ __launch_bounds__(ORDER_WAVES * 64) void pivot_code_kernel(
    const uint16_t* __restrict__ Q, int64_t N, int H, int npiv,
    const int32_t* __restrict__ prank, uint16_t* __restrict__ codes,
    int32_t* __restrict__ counts) {
  constexpr int NM = DP / 16;
  constexpr int PER_THREAD = ORDER_PIVOTS * DP / 8 / (ORDER_WAVES * 64);
  static_assert(PER_THREAD * ORDER_WAVES * 64 * 8 == ORDER_PIVOTS * DP, "fill covers a batch");
  __shared__ __attribute__((aligned(16))) unsigned char piv[ORDER_PIVOTS * DP * 2];
  const int h = blockIdx.y;
  const int lane = threadIdx.x & 63, lrow = lane & 31, lhalf = lane >> 5;
  const int64_t i0 = ((int64_t)blockIdx.x * ORDER_WAVES + (threadIdx.x >> 6)) * (32 * ORDER_QB);
  const bool active = i0 < N;                     // uniform per wavefront
  bf16x8_t qb[ORDER_QB][NM];
#pragma unroll
  for (int b = 0; b < ORDER_QB; ++b) {
    const int64_t i = i0 + 32 * b + lrow;
    const uint16_t* qp = Q + ((i < N ? i : N - 1) * H + h) * D + 8 * lhalf;
#pragma unroll
    for (int m = 0; m < NM; ++m) qb[b][m] = *reinterpret_cast<const bf16x8_t*>(qp + 16 * m);
  }
  // Per lane and query block: the best of its pivots.  acc[r] of block j is
  // pivot base + 32j + 4*lhalf + 8*(r/4) + r%4, increasing in r, j and the
  // batch, so strict compares keep the lowest index among equal scores.  The
  // loop keeps the best block's index and scores (sv); the position inside
  // it is found once at the end.
  float best[ORDER_QB], sv[ORDER_QB][16];
  int bblk[ORDER_QB];
#pragma unroll
  for (int b = 0; b < ORDER_QB; ++b) {
    best[b] = -__builtin_inff();
    bblk[b] = 0;
#pragma unroll
    for (int r = 0; r < 16; ++r) sv[b][r] = best[b];
  }
  for (int base = 0; base < npiv; base += ORDER_PIVOTS) {
    const int nb = npiv - base < ORDER_PIVOTS ? npiv - base : ORDER_PIVOTS;
    if (base > 0) __syncthreads();                // the previous batch has been read
    // All of a thread's pieces are requested before any is stored.
    const int pieces = nb * DP / 8;               // 16-byte operand pieces
    uint4 pv[PER_THREAD];
#pragma unroll
    for (int u = 0; u < PER_THREAD; ++u) {
      const int tu = threadIdx.x + u * ORDER_WAVES * 64;
      const int t = tu < pieces ? tu : pieces - 1;   // loads stay in range; stores are skipped
      const int blk = t >> 6, l = t & 63;
      const int64_t row = pivot_node(base + (blk / NM) * 32 + (l & 31), N, npiv);
      pv[u] = *reinterpret_cast<const uint4*>(Q + (row * H + h) * D + 16 * (blk % NM) +
                                              8 * (l >> 5));
    }
#pragma unroll
    for (int u = 0; u < PER_THREAD; ++u) {
      const int t = threadIdx.x + u * ORDER_WAVES * 64;
      if (t < pieces) *reinterpret_cast<uint4*>(piv + (size_t)t * 16) = pv[u];
    }
    __syncthreads();
    if (!active) continue;
#pragma unroll 2
    for (int j = 0; j < nb / 32; ++j) {
      floatx16_t acc[ORDER_QB];
#pragma unroll
      for (int b = 0; b < ORDER_QB; ++b) acc[b] = floatx16_t{};
#pragma unroll
      for (int m = 0; m < NM; ++m) {
        const bf16x8_t pa =
            *reinterpret_cast<const bf16x8_t*>(piv + (j * NM + m) * 1024 + lane * 16);
#pragma unroll
        for (int b = 0; b < ORDER_QB; ++b)
          acc[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pa, qb[b][m], acc[b], 0, 0, 0);
      }
#pragma unroll
      for (int b = 0; b < ORDER_QB; ++b) {
        const floatx16_t& x = acc[b];
        const float mx = fmaxf(fmaxf(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])),
                                     fmaxf(fmaxf(x[4], x[5]), fmaxf(x[6], x[7]))),
                               fmaxf(fmaxf(fmaxf(x[8], x[9]), fmaxf(x[10], x[11])),
                                     fmaxf(fmaxf(x[12], x[13]), fmaxf(x[14], x[15]))));
        const bool up = mx > best[b];
        best[b] = up ? mx : best[b];
        bblk[b] = up ? base / 32 + j : bblk[b];
#pragma unroll
        for (int r = 0; r < 16; ++r) sv[b][r] = up ? x[r] : sv[b][r];
      }
    }
  }
  if (!active) return;
#pragma unroll
  for (int b = 0; b < ORDER_QB; ++b) {
    int r0 = 15;
#pragma unroll
    for (int r = 14; r >= 0; --r) r0 = sv[b][r] == best[b] ? r : r0;
    int bp = 32 * bblk[b] + 4 * lhalf + 8 * (r0 >> 2) + (r0 & 3);
    const float ob = __shfl_xor(best[b], 32);
    const int op = __shfl_xor(bp, 32);
    if (ob > best[b] || (ob == best[b] && op < bp)) bp = op;
    const int64_t i = i0 + 32 * b + lrow;
    if (lhalf == 0 && i < N) {
      const int g = prank[(int64_t)h * npiv + bp];
      codes[h * N + i] = (uint16_t)g;
      atomicAdd(&counts[((int64_t)h * npiv + g) * ORDER_COPIES + (i & (ORDER_COPIES - 1))], 1);
    }
  }
}

// perm[h*N + pos] = i, positions handed out per (head, pivot) from the
// scanned counts.  The order inside a pivot group is immaterial.
__global__ void order_place_kernel(const uint16_t* __restrict__ codes, int64_t N, int H,
                                   int npiv, int32_t* __restrict__ cursor,
                                   int32_t* __restrict__ perm) {
  const int64_t r = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;   // r = h*N + i
  if (r >= N * H) return;
  const int h = (int)(r / N);
  const int64_t i = r % N;
  const int pos = atomicAdd(
      &cursor[((int64_t)h * npiv + codes[r]) * ORDER_COPIES + (i & (ORDER_COPIES - 1))], 1);
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
  const int64_t np = (int64_t)H * order_pivots(N);
  const int64_t nb = np * ORDER_COPIES;
  return align256((size_t)N * H * 4) + align256((size_t)N * H * 2) + 2 * align256((size_t)nb * 4) +
         align256((size_t)scan_aux_elems(nb) * 4) + align256((size_t)np) +
         align256((size_t)np * 4);
}

hipError_t launch_query_order(const uint16_t* q, int64_t N, int H, int d, void* ws,
                              int32_t** perm_out, hipStream_t s, const int32_t** counts_out,
                              int* npiv_out) {
  const int npiv = order_pivots(N);
  const int64_t nb = (int64_t)H * npiv * ORDER_COPIES;
  char* p = static_cast<char*>(ws);
  int32_t* perm = reinterpret_cast<int32_t*>(p); p += align256((size_t)N * H * 4);
  uint16_t* codes = reinterpret_cast<uint16_t*>(p); p += align256((size_t)N * H * 2);
  int32_t* counts = reinterpret_cast<int32_t*>(p); p += align256((size_t)nb * 4);
  int32_t* cursor = reinterpret_cast<int32_t*>(p); p += align256((size_t)nb * 4);
  int32_t* aux = reinterpret_cast<int32_t*>(p); p += align256((size_t)scan_aux_elems(nb) * 4);
  uint8_t* anchor = reinterpret_cast<uint8_t*>(p); p += align256((size_t)H * npiv);
  int32_t* prank = reinterpret_cast<int32_t*>(p);
  hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)ceil_div(nb, 256)), dim3(256), 0, s,
                     counts, nb);
  const dim3 grid((unsigned)ceil_div(N, ORDER_WAVES * 32 * ORDER_QB), (unsigned)H);
  const dim3 block(ORDER_WAVES * 64);
  void (*code_kernel)(const uint16_t*, int64_t, int, int, const int32_t*, uint16_t*, int32_t*);
  void (*anchor_kernel)(const uint16_t*, int64_t, int, int, uint8_t*);
  switch (d) {      // split-precision rows (3d) are grouped by their high parts
    case 32:
      code_kernel = pivot_code_kernel<32, 32>;
      anchor_kernel = pivot_anchor_kernel<32, 32>;
      break;
    case 64:
      code_kernel = pivot_code_kernel<64, 64>;
      anchor_kernel = pivot_anchor_kernel<64, 64>;
      break;
    case 96:
      code_kernel = pivot_code_kernel<96, 32>;
      anchor_kernel = pivot_anchor_kernel<96, 32>;
      break;
    case 192:
      code_kernel = pivot_code_kernel<192, 64>;
      anchor_kernel = pivot_anchor_kernel<192, 64>;
      break;
    default: return hipErrorInvalidValue;
  }
  hipLaunchKernelGGL(anchor_kernel, dim3((unsigned)ceil_div(npiv, 256), (unsigned)H), dim3(256),
                     0, s, q, N, H, npiv, anchor);
  hipLaunchKernelGGL(pivot_rank_kernel, dim3((unsigned)H), dim3(ORDER_ANCHORS), 0, s, anchor,
                     npiv, prank);
  hipLaunchKernelGGL(code_kernel, grid, block, 0, s, q, N, H, npiv, prank, codes, counts);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // Exclusive scan over (head, pivot, copy): head h's positions start at h*N.
  e = launch_exclusive_scan(counts, cursor, nb, aux, s);
  if (e != hipSuccess) return e;
  const unsigned rows = (unsigned)ceil_div(N * H, 256);
  hipLaunchKernelGGL(order_place_kernel, dim3(rows), dim3(256), 0, s, codes, N, H, npiv,
                     cursor, perm);
  *perm_out = perm;
  if (counts_out != nullptr) *counts_out = counts;
  if (npiv_out != nullptr) *npiv_out = npiv;
  return hipGetLastError();
}

// Pruned selection buffers (see ScanArgs).  The live words of one range of
// query blocks are kept at a time: PRUNE_LIVE_BYTES bound them whatever N is.
namespace {
struct PruneSizes {
  int64_t nkb, nkp, ngr, live_rows, nrange, heavy_max;
  int npiv, live_shift;
  size_t groups, bgroup, kid, kop, bop, live, cnt, rcnt, heavy, parts;
};
PruneSizes prune_sizes(int64_t N, int H, int d) {
  PruneSizes z{};
  z.nkb = ceil_div(N, 32);
  z.npiv = order_pivots(N);
  // each group's last block may be partly empty: at most one block per group
  z.nkp = z.nkb + z.npiv;
  z.ngr = ceil_div(z.nkp, 32);
  const int64_t rows = (int64_t)H * z.nkb;
  // ranges of 2^live_shift query blocks (at least 16), as many as the live
  // words' budget holds (one range up to a few 10^5 nodes: each range is a
  // chain of launches with its own tail)
  const int64_t fit = PRUNE_LIVE_BYTES / (z.ngr * 4);
  z.live_shift = 4;
  while (((int64_t)2 << z.live_shift) <= fit && ((int64_t)1 << z.live_shift) < rows) ++z.live_shift;
  z.live_rows = (int64_t)1 << z.live_shift;
  const int64_t held = rows < z.live_rows ? rows : z.live_rows;
  z.groups = 3 * align256((size_t)H * z.npiv * 4) + align256((size_t)H * 4);
  z.bgroup = align256((size_t)H * z.nkp * 4);
  z.kid = align256((size_t)H * z.nkp * 32 * 4);
  z.kop = align256((size_t)H * z.nkp * (d / 16) * 1024);
  z.bop = align256((size_t)H * z.ngr * ((d == 96 ? 32 : d) / 16 + 1) * 1024);
  z.live = align256((size_t)held * z.ngr * 4);
  z.cnt = align256((size_t)rows * 4);
  z.nrange = ceil_div(rows, z.live_rows);
  z.rcnt = 2 * align256((size_t)z.nrange * 4);
  z.heavy_max = held < PRUNE_HEAVY_MAX ? held : (int64_t)PRUNE_HEAVY_MAX;
  z.heavy = align256((size_t)z.heavy_max * 4) + align256((size_t)z.nrange * 4);
  z.parts = align256((size_t)z.heavy_max * PRUNE_HEAVY_PARTS * 32 * 16 * 8);
  return z;
}
}  // namespace

bool prune_applies(int64_t N, int H, int d, int topk) {
  (void)H;
  // From 2^16 nodes on: below, the streaming pass is faster (N = 31623:
  // 0.48 against 0.68 ms; the pruned pass pays a bound pass and a fixed
  // cost per wavefront).  Up to 2^19: block and word indices are 32-bit
  // shifts of the query block index, and a query block's live words fit the
  // bound pass's LDS.  Rows of 32 or 64 bf16, or the split-precision rows of
  // 96 of the fp32 entry points at d = 32 (the bound holds for any inner
  // product the scan computes; 192-wide rows would leave one workgroup per
  // CU).
  if (!((d == 32 || d == 64 || d == 96) && scan_list_len(topk) > 0 && N >= ((int64_t)1 << 16) &&
        N <= ((int64_t)1 << 19)))
    return false;
  return prune_sizes(N, H, d).ngr <= PRUNE_MAX_WORDS;
}

size_t prune_ws(int64_t N, int H, int d, int topk) {
  if (!prune_applies(N, H, d, topk)) return 0;
  const PruneSizes z = prune_sizes(N, H, d);
  // lists longer than 16 collect their candidates (no heavy parts)
  return z.groups + z.bgroup + z.kid + z.kop + z.bop + z.live + z.cnt + z.rcnt + z.heavy +
         (scan_list_len(topk) <= 16 ? z.parts : 0);
}

void prune_setup(ScanArgs& a, int d, char* w) {
  const PruneSizes z = prune_sizes(a.N, a.H, d);
  const size_t gb = align256((size_t)a.H * z.npiv * 4);
  a.gstart = reinterpret_cast<int32_t*>(w);
  w += gb;
  a.gsize = reinterpret_cast<int32_t*>(w);
  w += gb;
  a.pstart = reinterpret_cast<int32_t*>(w);
  w += gb;
  a.nkp_h = reinterpret_cast<int32_t*>(w);
  w += z.groups - 3 * gb;
  a.bgroup = reinterpret_cast<int32_t*>(w);
  w += z.bgroup;
  a.kid = reinterpret_cast<int32_t*>(w);
  w += z.kid;
  a.kop = reinterpret_cast<uint16_t*>(w);
  w += z.kop;
  a.bop = reinterpret_cast<uint16_t*>(w);
  w += z.bop;
  a.live = reinterpret_cast<uint32_t*>(w);
  w += z.live;
  a.qb_cnt = reinterpret_cast<int32_t*>(w);
  w += z.cnt;
  a.range_cnt = reinterpret_cast<int32_t*>(w);
  w += z.rcnt / 2;
  a.range_stream = reinterpret_cast<int32_t*>(w);
  w += z.rcnt / 2;
  a.heavy_list = reinterpret_cast<int32_t*>(w);
  w += align256((size_t)z.heavy_max * 4);
  a.heavy_cnt = reinterpret_cast<int32_t*>(w);
  w += align256((size_t)z.nrange * 4);
  a.heavy_parts = scan_list_len(a.topk) <= 16 ? reinterpret_cast<uint2*>(w) : nullptr;
  a.heavy_max = (int)z.heavy_max;
  a.nkb = z.nkb;
  a.nkp = z.nkp;
  a.ngr = z.ngr;
  a.live_rows = z.live_rows;
  a.live_shift = z.live_shift;
  a.nrange = z.nrange;
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
