// Internal declarations shared by the libkmip HIP sources (not installed).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "kmip.h"

namespace kmip {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx16_t __attribute__((ext_vector_type(16)));

// ---------------------------------------------------------------- tiling
// Score scan: a workgroup of scan_waves(...) wavefronts, each owning 32 query
// rows of one head (one 32x32 MFMA output block: keys x queries).
constexpr int SCAN_WAVES = 16;                    // one graph, lists of up to 16
constexpr int SCAN_WAVES_LONG = 8;                // longer lists; batched graphs
constexpr int SCAN_QPW = 32;
constexpr int SCAN_QT_MIN = SCAN_WAVES_LONG * SCAN_QPW;   // smallest planned tile
constexpr int SCAN_CAP = 8;                       // per-lane candidate buffer entries
constexpr int SCAN_CHUNKS = 32;                   // threshold pass: key ranges per lane half
constexpr int COLLECT_CAP = 256;                  // candidates per row and lane half

// Key-side backward: consecutive sorted (key, pair) positions per slice.
constexpr int SEG_SLICE = 128;
// Radix sort: elements per block tile; digits of up to 11 bits, so that keys
// of up to 22 bits (N*H < 4M) sort in two passes.
constexpr int SORT_THREADS = 256;
constexpr int SORT_ITEMS = 16;
constexpr int SORT_TILE = SORT_THREADS * SORT_ITEMS;
constexpr int SORT_MAX_BITS = 11;
constexpr int SORT_MAX_BINS = 1 << SORT_MAX_BITS;
// Device-wide exclusive scan tile.
constexpr int SCAN_THREADS = 256;
constexpr int SCAN_ITEMS = 16;
constexpr int SCAN_TILE_ELEMS = SCAN_THREADS * SCAN_ITEMS;

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Smallest list length the scan kernel is instantiated for that holds k.
int scan_list_len(int topk);

// Wavefronts per scan workgroup for a list length: long register lists need
// the VGPR budget of two wavefronts per SIMD.  Batched graphs use 8-wavefront
// workgroups for short lists too: tiles of 256 rows waste less on each
// graph's partial last tile, and two such workgroups share a CU, so one's
// barrier stalls are covered by the other's work.
constexpr int scan_waves(int kp, bool batched = false) {
  return kp <= 16 && !batched ? SCAN_WAVES : SCAN_WAVES_LONG;
}

// Maximum number of query tiles for N nodes in num_graphs graphs (for the
// smallest tile).
inline int64_t scan_max_tiles(int64_t N, int num_graphs) {
  return ceil_div(N, SCAN_QT_MIN) + (num_graphs > 1 ? num_graphs : 0);
}

// ---------------------------------------------------------------- launchers
// All return hipSuccess or the first launch error.  No allocation, no sync.

// Ragged tile plan: tiles of tile_rows queries, tiles[t] = (graph, first
// query) for t < total, (-1, 0) beyond; tile_start is [B+1] scratch.
hipError_t launch_tile_plan(const int32_t* offsets, int num_graphs, int64_t max_tiles,
                            int tile_rows, int32_t* tile_start, int2* tiles, hipStream_t s);

// Score scan in two passes: a threshold pass writing a per-row lower bound
// of the k-th score into thr[N*H], then the exact running top-k seeded with
// it.  Writes idx / score.  One graph: tiles == nullptr, and perm (may be
// null) gives each head's query order [H][N]; batched graphs: the tile plan.
struct ScanArgs {
  const uint16_t* q;
  const uint16_t* k;
  int64_t N;
  int H, topk;
  const int32_t* offsets;
  const int2* tiles;
  int64_t max_tiles;
  const int32_t* perm;
  float* thr;
  int32_t* idx;
  float* score;
  // Lists longer than 16: per-row candidate arrays [2 halves][cap][N*H] of
  // (score bits, key id) and their counts [N*H][2].
  uint2* cand;
  int32_t* cand_cnt;
  int cap;
  // Selection pass: first rank it computes (0, or 16, 32, ... in the passes
  // that recompute rows with overflowing candidate arrays).
  int rank0;
  // Pruned selection (one graph with a query order, rows of 32 or 64 bf16;
  // lists longer than 16 collect candidates instead of selecting; kop ==
  // nullptr: off).  Keys are taken in the query
  // order, in 32-key blocks.  Every pivot group of the order starts a new
  // key block (its last block padded with empty slots), so the keys of a
  // block belong to one group and its bound is tight; nkp = nkb + npiv
  // blocks per head are allocated (padded to ngr groups of 32), nkp_h[h] of
  // them used:
  //   gstart, gsize, pstart [H][npiv]  per group (pivot rank r) its first
  //                               position in the head's order, its size,
  //                               and its first padded key slot (a multiple
  //                               of 32);
  //   bgroup [H][nkp]             the group of padded key block b (-1 past
  //                               nkp_h[h]);
  //   kid  [H][nkp][32]           node id of each padded key slot (-1: an
  //                               empty slot);
  //   kop  [H][nkp][D/16][64][8]  the block's keys in MFMA operand order
  //                               (zero rows in empty slots);
  //   bop  [H][ngr][D/16+1][64][8]  per block a bound row [mid | R e0],
  //                               D + 16 elements, in operand order (see
  //                               key_pack_kernel);
  //   live [wid1 - wid0][ngr]     per query block (wid = h * nkb + block of
  //                               32 positions) a bit per key block whose
  //                               bound reaches one of its thresholds;
  //   qb_cnt [H * nkb]            live key blocks per query block (negated
  //                               for a heavy one left unsplit);
  //   range_cnt [nrange]          live key blocks per range of live_rows
  //                               (= 2^live_shift) query blocks;
  //   range_stream [nrange]       1: the streaming pass takes the range;
  //   heavy_list [heavy_max], heavy_cnt [nrange]  query blocks of the current
  //                               range with many live key blocks (split over
  //                               several wavefronts), and their number per
  //                               range;
  //   heavy_parts [heavy_max][parts][32][16]  the parts' lists per query
  //                               (lists of at most 16 only).
  // A range whose query blocks have on average more than PRUNE_STREAM_NUM /
  // PRUNE_STREAM_DEN of the key blocks live (inputs without enough cluster
  // structure) is left to the streaming selection pass; the pruned pass
  // takes the others.
  const int32_t* order_counts;   // [H][npiv][copies] group sizes from the order
  int npiv;
  int32_t* gstart;
  int32_t* gsize;
  int32_t* pstart;
  int32_t* bgroup;
  int32_t* nkp_h;
  int32_t* kid;
  uint16_t* kop;
  uint16_t* bop;
  uint32_t* live;
  int32_t* qb_cnt;
  int32_t* range_cnt;
  int32_t* range_stream;
  int32_t* heavy_list;
  int32_t* heavy_cnt;
  uint2* heavy_parts;
  int heavy_max;
  int64_t nkb, nkp, ngr, wid0, wid1, live_rows, nrange;
  int live_shift;
};
hipError_t launch_score_topk(const ScanArgs& args, int d, hipStream_t s);
// Pruned selection workspace for one graph of N nodes, H heads, rows of d
// bf16 (0 when the pruned path does not apply): key copy, bound rows, one
// range of live words, per-query-block counts.
constexpr int64_t PRUNE_LIVE_BYTES = (int64_t)16 << 20;
// Heavy query blocks (many live key blocks) split per range (further ones
// run unsplit), and the wavefronts each is split over.
constexpr int PRUNE_HEAVY_MAX = 8192;
constexpr int PRUNE_HEAVY_PARTS = 8;
constexpr int PRUNE_STREAM_NUM = 1, PRUNE_STREAM_DEN = 4;
// Live words (32 key blocks each) per query block the bound pass holds.
constexpr int PRUNE_MAX_WORDS = 704;
bool prune_applies(int64_t N, int H, int d, int topk);
size_t prune_ws(int64_t N, int H, int d, int topk);
// Carves the pruned-selection buffers out of w (prune_ws bytes) into a.
void prune_setup(ScanArgs& a, int d, char* w);
// Per row width (bf16 elements; 96 and 192 are split-precision rows of 32
// and 64 fp32 elements), kp = scan_list_len(topk).
hipError_t launch_scan_d32(int kp, const ScanArgs& a, hipStream_t s);
hipError_t launch_scan_d64(int kp, const ScanArgs& a, hipStream_t s);
hipError_t launch_scan_d96(int kp, const ScanArgs& a, hipStream_t s);
hipError_t launch_scan_d192(int kp, const ScanArgs& a, hipStream_t s);

// Query order for one graph: groups each head's queries by their nearest
// pivot query (largest inner product).  Workspace: query_order_bytes(N, H); *perm points
// into it ([H][N] node ids).
// *counts (if not null) points at the per-(head, pivot rank, copy) group
// counts [H][npiv][ORDER_COPIES] and *npiv receives the pivots per head.
size_t query_order_bytes(int64_t N, int H);
hipError_t launch_query_order(const uint16_t* q, int64_t N, int H, int d, void* ws,
                              int32_t** perm, hipStream_t s, const int32_t** counts = nullptr,
                              int* npiv = nullptr);
constexpr int ORDER_COPIES = 16;

// Split-precision rows for the fp32 entry points: per (node, head) row of d
// fp32 elements x = hi + lo + r (hi = bf16(x), lo = bf16(x - hi)),
// q3 = [q_hi | q_hi | q_lo] and k3 = [k_hi | k_lo | k_hi], bf16 [rows][3d],
// so that q3 . k3 = q_hi.k_hi + q_hi.k_lo + q_lo.k_hi.
hipError_t launch_split_rows(const float* q, const float* k, int64_t rows, int d, uint16_t* q3,
                             uint16_t* k3, hipStream_t s);

// Gather the selected V rows (bf16), softmax over saved scores, weighted sum.
hipError_t launch_gather_av(const uint16_t* v, int64_t N, int H, int d, int topk,
                            const int32_t* topk_idx, const float* topk_score, float* out,
                            hipStream_t s);

// fp32 entry point: recompute the selected scores in fp32 from the fp32 rows
// (overwriting topk_score), then the softmax-weighted sum of fp32 V rows.
hipError_t launch_gather_rescore_av(const float* q, const float* k, const float* v, int64_t N,
                                    int H, int d, int topk, const int32_t* topk_idx,
                                    float* topk_score, float* out, hipStream_t s);

// Backward, query side: dq and the per-pair (p, ds), with the selected
// scores recomputed from q and k.  Q, K and V are bf16 bits, or fp32 when
// f32 is set.
hipError_t launch_bwd_query(const void* q, const void* k, const void* v, bool f32, int64_t N,
                            int H, int d, int topk, const int32_t* topk_idx, const float* dout,
                            float* dq, float2* pairs, hipStream_t s);

// Backward, selection transpose: stable sort of the pairs by key h*N + j
// (padding slots: H*N), carrying each pair's id and its (p, ds); key segment
// pointers key_ptr[H*N + 2].  The pairs array itself is the first pass's
// payload input and is overwritten by later passes.
struct SortScratch {
  uint32_t* keys[2];
  uint32_t* vals[2];      // pair ids
  float2* pay[2];         // (p, ds); pay[0] is the caller's pairs array
  int32_t* hist;          // [tiles][bins] digit counts, then output offsets
  int32_t* colsum;        // [row groups][bins] column sums of hist
  int32_t* binbase;       // [bins + 1] start of each digit in the pass output
  int32_t* bintot;        // [bins] pairs per digit
  int32_t* key_ptr;       // H*N + 2
  int final_buf;          // which of keys/vals/pay holds the sorted result
};
size_t sort_scratch_bytes(int64_t P, int64_t HN);
void sort_scratch_carve(void* base, float2* pairs, int64_t P, int64_t HN, SortScratch* sc);
hipError_t launch_selection_transpose(const int32_t* topk_idx, int64_t N, int H, int topk,
                                      SortScratch* sc, hipStream_t s);

// Backward, key side: dk, dv by segmented reduction over the sorted pairs
// (Q bf16 bits, or fp32 when q_f32 is set).
size_t segreduce_scratch_bytes(int64_t P, int d);
hipError_t launch_bwd_keys(const void* q, bool q_f32, const float* dout, int64_t N, int H,
                           int d, int topk, const SortScratch* sc, double* partials, float* dk,
                           float* dv, hipStream_t s);

// Device-wide exclusive scan of int32 (aux: scan_aux_elems(n) ints).
int64_t scan_aux_elems(int64_t n);
hipError_t launch_exclusive_scan(const int32_t* in, int32_t* out, int64_t n, int32_t* aux,
                                 hipStream_t s);

}  // namespace kmip
