// libkmip C ABI: argument checks, workspace layout and kernel launches.
// The contract of every entry point is documented in include/kmip.h.
#include <mutex>

#include "kmip_internal.h"

using namespace kmip;

// Scratch of kmip_forward_no_workspace: one copy per GPU, held until the
// process ends.  Host code never uses the array's name as an address (on the
// host it is only a stand-in for the symbol); the device address of each
// GPU's copy comes from hipGetSymbolAddress, once per device.
static __device__ __align__(256) unsigned char scratch[KMIP_NO_WORKSPACE_BYTES];

namespace {

constexpr int kVersion = 1 * 10000 + 1 * 100 + 0;

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

bool single_graph(const int32_t* offsets, int num_graphs) {
  return offsets == nullptr || num_graphs <= 1;
}

kmip_status_t check_shape(int64_t N, int H, int d, int topk, int num_graphs) {
  if (N < 1 || H < 1 || num_graphs < 0) return KMIP_ERR_INVALID_VALUE;
  if (d != 32 && d != 64) return KMIP_ERR_UNSUPPORTED;
  if (topk < 1 || topk > 64) return KMIP_ERR_UNSUPPORTED;
  // Key-row offsets inside a scan chunk are 32-bit: (row < 1024) * H * d * 2.
  if ((int64_t)H * d > (int64_t)1 << 20) return KMIP_ERR_UNSUPPORTED;
  const int64_t NH = N * (int64_t)H;
  if (N > (int64_t)INT32_MAX || NH * topk >= (int64_t)INT32_MAX - 1 ||
      NH >= (int64_t)INT32_MAX - 2)
    return KMIP_ERR_UNSUPPORTED;
  if (scan_max_tiles(N, num_graphs) * H >= (int64_t)INT32_MAX) return KMIP_ERR_UNSUPPORTED;
  return KMIP_OK;
}

// Forward workspace: per-row score thresholds [N*H] fp32; then the tile plan
// (batched graphs) or the query order (one graph); then, for lists longer
// than 16, the candidate arrays and their counts.
// Grouping queries pays off only when there are many wavefronts of them;
// small inputs skip it (and its six launches).
bool use_query_order(int64_t N, int H) { return N * H >= 32768; }

size_t collect_ws(int64_t N, int H, int topk) {
  if (scan_list_len(topk) <= 16) return 0;
  return align256((size_t)2 * COLLECT_CAP * N * H * sizeof(uint2)) +
         align256((size_t)2 * N * H * sizeof(int32_t));
}

// One graph with a query order, bf16 rows of 32 or 64, lists of at most 16:
// the pruned selection (its buffers follow the query order).  The entry
// point without a workspace leaves it off: its static array holds the other
// buffers only.
bool use_prune(int64_t N, int H, int d_rows, int topk, int num_graphs, bool prune) {
  return prune && num_graphs <= 1 && use_query_order(N, H) && prune_applies(N, H, d_rows, topk);
}

size_t forward_ws(int64_t N, int H, int d_rows, int topk, int num_graphs, bool prune = true) {
  size_t b = align256((size_t)N * H * sizeof(float));
  if (num_graphs > 1) {
    const int64_t tiles = scan_max_tiles(N, num_graphs);
    b += align256((size_t)(num_graphs + 1) * 4) + align256((size_t)tiles * sizeof(int2));
  } else if (use_query_order(N, H)) {
    b += query_order_bytes(N, H);
    if (use_prune(N, H, d_rows, topk, num_graphs, prune)) b += prune_ws(N, H, d_rows, topk);
  }
  return b + collect_ws(N, H, topk);
}

size_t backward_ws(int64_t N, int H, int d, int topk) {
  const int64_t P = N * H * topk;
  const int64_t HN = N * H;
  return align256((size_t)P * sizeof(float2)) + sort_scratch_bytes(P, HN) +
         segreduce_scratch_bytes(P, d);
}

kmip_status_t launch_status(hipError_t e) { return e == hipSuccess ? KMIP_OK : KMIP_ERR_LAUNCH; }

// fp32 entry points: the split-precision rows q3, k3 (bf16 [N*H][3d] each)
// come first in the forward workspace.
size_t split_ws(int64_t N, int H, int d) { return 2 * align256((size_t)N * H * 3 * d * 2); }

// The selection on validated arguments.  q and k are bf16 rows of d_rows
// elements (d, or 3d for split-precision rows); w is the forward workspace
// past any split rows.
kmip_status_t score_topk_core(const uint16_t* q, const uint16_t* k, int64_t N, int H, int d_rows,
                              int topk, const int32_t* graph_offsets, int num_graphs,
                              int32_t* topk_idx, float* topk_score, char* w, hipStream_t s,
                              bool prune = true) {
  const bool single = single_graph(graph_offsets, num_graphs);
  const int64_t max_tiles = scan_max_tiles(N, num_graphs);
  ScanArgs a{};
  a.q = q;
  a.k = k;
  a.N = N;
  a.H = H;
  a.topk = topk;
  a.max_tiles = max_tiles;
  a.thr = reinterpret_cast<float*>(w);
  a.idx = topk_idx;
  a.score = topk_score;
  w += align256((size_t)N * H * sizeof(float));
  kmip_status_t st = KMIP_OK;
  if (!single) {
    int32_t* tile_start = reinterpret_cast<int32_t*>(w);
    int2* tiles = reinterpret_cast<int2*>(w + align256((size_t)(num_graphs + 1) * 4));
    w += align256((size_t)(num_graphs + 1) * 4) + align256((size_t)max_tiles * sizeof(int2));
    const int tile_rows = scan_waves(scan_list_len(topk), true) * SCAN_QPW;
    st = launch_status(launch_tile_plan(graph_offsets, num_graphs, max_tiles, tile_rows,
                                        tile_start, tiles, s));
    if (st != KMIP_OK) return st;
    a.offsets = graph_offsets;
    a.tiles = tiles;
  } else if (use_query_order(N, H)) {
    int32_t* perm = nullptr;
    st = launch_status(launch_query_order(a.q, N, H, d_rows, w, &perm, s, &a.order_counts,
                                          &a.npiv));
    if (st != KMIP_OK) return st;
    a.perm = perm;
    w += query_order_bytes(N, H);
    if (use_prune(N, H, d_rows, topk, 1, prune)) {
      prune_setup(a, d_rows, w);
      w += prune_ws(N, H, d_rows, topk);
    }
  }
  if (collect_ws(N, H, topk) > 0) {
    a.cand = reinterpret_cast<uint2*>(w);
    w += align256((size_t)2 * COLLECT_CAP * N * H * sizeof(uint2));
    a.cand_cnt = reinterpret_cast<int32_t*>(w);
    a.cap = COLLECT_CAP;
  }
  return launch_status(launch_score_topk(a, d_rows, s));
}

// Argument checks of the selection (kmip_score_topk and kmip_forward).
kmip_status_t check_topk_args(const void* q, const void* k, int64_t N, int H, int d, int topk,
                              const int32_t* graph_offsets, int num_graphs,
                              const int32_t* topk_idx, const float* topk_score,
                              const void* workspace, size_t workspace_bytes) {
  if (!q || !k || !topk_idx || !topk_score) return KMIP_ERR_INVALID_VALUE;
  const kmip_status_t st = check_shape(N, H, d, topk, num_graphs);
  if (st != KMIP_OK) return st;
  if (num_graphs > 1 && graph_offsets == nullptr) return KMIP_ERR_INVALID_VALUE;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(topk_idx, 4) || !aligned(topk_score, 4))
    return KMIP_ERR_INVALID_VALUE;
  const bool single = single_graph(graph_offsets, num_graphs);
  const size_t need = forward_ws(N, H, d, topk, single ? 0 : num_graphs);
  if (workspace == nullptr || workspace_bytes < need) return KMIP_ERR_WORKSPACE;
  if (!aligned(workspace, 16)) return KMIP_ERR_INVALID_VALUE;
  return KMIP_OK;
}

kmip_status_t backward_impl(const void* q, const void* k, const void* v, bool f32, int64_t N,
                            int H, int d, int topk, const int32_t* graph_offsets,
                            int num_graphs, const int32_t* topk_idx, const float* topk_score,
                            const float* dout, float* dq, float* dk, float* dv,
                            void* workspace, size_t workspace_bytes, kmip_stream_t stream) {
  if (!q || !k || !v || !topk_idx || !topk_score || !dout || !dq || !dk || !dv)
    return KMIP_ERR_INVALID_VALUE;
  kmip_status_t st = check_shape(N, H, d, topk, num_graphs);
  if (st != KMIP_OK) return st;
  if (num_graphs > 1 && graph_offsets == nullptr) return KMIP_ERR_INVALID_VALUE;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(dout, 16) ||
      !aligned(dq, 16) || !aligned(dk, 16) || !aligned(dv, 16) || !aligned(topk_idx, 4) ||
      !aligned(topk_score, 4))
    return KMIP_ERR_INVALID_VALUE;
  const size_t need = backward_ws(N, H, d, topk);
  if (workspace == nullptr || workspace_bytes < need) return KMIP_ERR_WORKSPACE;
  if (!aligned(workspace, 256)) return KMIP_ERR_INVALID_VALUE;

  hipStream_t s = static_cast<hipStream_t>(stream);
  const int64_t P = N * H * topk;
  const int64_t HN = N * H;
  char* w = static_cast<char*>(workspace);
  float2* pairs = reinterpret_cast<float2*>(w);
  w += align256((size_t)P * sizeof(float2));
  SortScratch sc;
  sort_scratch_carve(w, pairs, P, HN, &sc);
  w += sort_scratch_bytes(P, HN);
  double* partials = reinterpret_cast<double*>(w);

  st = launch_status(launch_bwd_query(q, k, v, f32, N, H, d, topk, topk_idx, dout, dq, pairs,
                                      s));
  if (st != KMIP_OK) return st;
  st = launch_status(launch_selection_transpose(topk_idx, N, H, topk, &sc, s));
  if (st != KMIP_OK) return st;
  return launch_status(launch_bwd_keys(q, f32, dout, N, H, d, topk, &sc, partials, dk, dv, s));
}

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's copy of `scratch`.
kmip_status_t static_scratch(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return KMIP_ERR_LAUNCH;
  if (dev < 0 || dev >= kMaxDevices) return KMIP_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
      return KMIP_ERR_LAUNCH;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return KMIP_OK;
}

}  // namespace

extern "C" {

const char* kmip_status_string(kmip_status_t status) {
  switch (status) {
    case KMIP_OK: return "KMIP_OK: success";
    case KMIP_ERR_INVALID_VALUE: return "KMIP_ERR_INVALID_VALUE: invalid argument";
    case KMIP_ERR_UNSUPPORTED: return "KMIP_ERR_UNSUPPORTED: unsupported shape (d, topk or size)";
    case KMIP_ERR_WORKSPACE: return "KMIP_ERR_WORKSPACE: workspace too small";
    case KMIP_ERR_LAUNCH: return "KMIP_ERR_LAUNCH: kernel launch failed";
  }
  return "KMIP: unknown status";
}

int kmip_version(void) { return kVersion; }

size_t kmip_forward_workspace_bytes(int64_t N, int H, int d, int topk, int num_graphs) {
  if (check_shape(N, H, d, topk, num_graphs) != KMIP_OK) return 0;
  return forward_ws(N, H, d, topk, num_graphs);
}

size_t kmip_backward_workspace_bytes(int64_t N, int H, int d, int topk, int num_graphs) {
  if (check_shape(N, H, d, topk, num_graphs) != KMIP_OK) return 0;
  return backward_ws(N, H, d, topk);
}

kmip_status_t kmip_score_topk(const void* q, const void* k, int64_t N, int H, int d, int topk,
                              const int32_t* graph_offsets, int num_graphs, int32_t* topk_idx,
                              float* topk_score, void* workspace, size_t workspace_bytes,
                              kmip_stream_t stream) {
  const kmip_status_t st = check_topk_args(q, k, N, H, d, topk, graph_offsets, num_graphs,
                                           topk_idx, topk_score, workspace, workspace_bytes);
  if (st != KMIP_OK) return st;
  return score_topk_core(static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k), N,
                         H, d, topk, graph_offsets, num_graphs, topk_idx, topk_score,
                         static_cast<char*>(workspace), static_cast<hipStream_t>(stream));
}

kmip_status_t kmip_gather_softmax_av(const void* v, int64_t N, int H, int d, int topk,
                                     const int32_t* topk_idx, const float* topk_score,
                                     float* out, kmip_stream_t stream) {
  if (!v || !topk_idx || !topk_score || !out) return KMIP_ERR_INVALID_VALUE;
  kmip_status_t st = check_shape(N, H, d, topk, 0);
  if (st != KMIP_OK) return st;
  if (!aligned(v, 16) || !aligned(out, 16) || !aligned(topk_idx, 4) || !aligned(topk_score, 4))
    return KMIP_ERR_INVALID_VALUE;
  return launch_status(launch_gather_av(static_cast<const uint16_t*>(v), N, H, d, topk,
                                        topk_idx, topk_score, out,
                                        static_cast<hipStream_t>(stream)));
}

kmip_status_t kmip_forward(const void* q, const void* k, const void* v, int64_t N, int H,
                           int d, int topk, const int32_t* graph_offsets, int num_graphs,
                           float* out, int32_t* topk_idx, float* topk_score, void* workspace,
                           size_t workspace_bytes, kmip_stream_t stream) {
  if (!q || !k || !v || !out || !topk_idx || !topk_score) return KMIP_ERR_INVALID_VALUE;
  kmip_status_t st = check_topk_args(q, k, N, H, d, topk, graph_offsets, num_graphs, topk_idx,
                                     topk_score, workspace, workspace_bytes);
  if (st != KMIP_OK) return st;
  if (!aligned(v, 16) || !aligned(out, 16)) return KMIP_ERR_INVALID_VALUE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const uint16_t* qb = static_cast<const uint16_t*>(q);
  const uint16_t* kb = static_cast<const uint16_t*>(k);
  const uint16_t* vb = static_cast<const uint16_t*>(v);
  char* w = static_cast<char*>(workspace);
  st = score_topk_core(qb, kb, N, H, d, topk, graph_offsets, num_graphs, topk_idx, topk_score,
                       w, s);
  if (st != KMIP_OK) return st;
  return launch_status(launch_gather_av(vb, N, H, d, topk, topk_idx, topk_score, out, s));
}

kmip_status_t kmip_forward_no_workspace(const void* q, const void* k, const void* v, int64_t N,
                                        int H, int d, int topk, const int32_t* graph_offsets,
                                        int num_graphs, float* out, int32_t* topk_idx,
                                        float* topk_score, kmip_stream_t stream) {
  if (!q || !k || !v || !out || !topk_idx || !topk_score) return KMIP_ERR_INVALID_VALUE;
  kmip_status_t st = check_shape(N, H, d, topk, num_graphs);
  if (st != KMIP_OK) return st;
  if (num_graphs > 1 && graph_offsets == nullptr) return KMIP_ERR_INVALID_VALUE;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16) ||
      !aligned(topk_idx, 4) || !aligned(topk_score, 4))
    return KMIP_ERR_INVALID_VALUE;
  const bool single = single_graph(graph_offsets, num_graphs);
  if (forward_ws(N, H, d, topk, single ? 0 : num_graphs, false) >
      (size_t)KMIP_NO_WORKSPACE_BYTES)
    return KMIP_ERR_WORKSPACE;
  void* ws = nullptr;
  st = static_scratch(&ws);
  if (st != KMIP_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  st = score_topk_core(static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k), N, H,
                       d, topk, graph_offsets, num_graphs, topk_idx, topk_score,
                       static_cast<char*>(ws), s, false);
  if (st != KMIP_OK) return st;
  return launch_status(launch_gather_av(static_cast<const uint16_t*>(v), N, H, d, topk,
                                        topk_idx, topk_score, out, s));
}

kmip_status_t kmip_backward(const void* q, const void* k, const void* v, int64_t N, int H,
                            int d, int topk, const int32_t* graph_offsets, int num_graphs,
                            const int32_t* topk_idx, const float* topk_score,
                            const float* dout, float* dq, float* dk, float* dv,
                            void* workspace, size_t workspace_bytes, kmip_stream_t stream) {
  return backward_impl(q, k, v, false, N, H, d, topk, graph_offsets, num_graphs, topk_idx,
                       topk_score, dout, dq, dk, dv, workspace, workspace_bytes, stream);
}

size_t kmip_forward_f32_workspace_bytes(int64_t N, int H, int d, int topk, int num_graphs) {
  if (check_shape(N, H, d, topk, num_graphs) != KMIP_OK) return 0;
  return split_ws(N, H, d) + forward_ws(N, H, 3 * d, topk, num_graphs);
}

kmip_status_t kmip_forward_f32(const float* q, const float* k, const float* v, int64_t N, int H,
                               int d, int topk, const int32_t* graph_offsets, int num_graphs,
                               float* out, int32_t* topk_idx, float* topk_score,
                               void* workspace, size_t workspace_bytes, kmip_stream_t stream) {
  if (!q || !k || !v || !out || !topk_idx || !topk_score) return KMIP_ERR_INVALID_VALUE;
  kmip_status_t st = check_shape(N, H, d, topk, num_graphs);
  if (st != KMIP_OK) return st;
  if (num_graphs > 1 && graph_offsets == nullptr) return KMIP_ERR_INVALID_VALUE;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16) ||
      !aligned(topk_idx, 4) || !aligned(topk_score, 4))
    return KMIP_ERR_INVALID_VALUE;
  const bool single = single_graph(graph_offsets, num_graphs);
  const size_t need = split_ws(N, H, d) + forward_ws(N, H, 3 * d, topk, single ? 0 : num_graphs);
  if (workspace == nullptr || workspace_bytes < need) return KMIP_ERR_WORKSPACE;
  if (!aligned(workspace, 16)) return KMIP_ERR_INVALID_VALUE;

  hipStream_t s = static_cast<hipStream_t>(stream);
  char* w = static_cast<char*>(workspace);
  uint16_t* q3 = reinterpret_cast<uint16_t*>(w);
  uint16_t* k3 = reinterpret_cast<uint16_t*>(w + split_ws(N, H, d) / 2);
  st = launch_status(launch_split_rows(q, k, N * H, d, q3, k3, s));
  if (st != KMIP_OK) return st;
  st = score_topk_core(q3, k3, N, H, 3 * d, topk, graph_offsets, num_graphs, topk_idx,
                       topk_score, w + split_ws(N, H, d), s);
  if (st != KMIP_OK) return st;
  return launch_status(
      launch_gather_rescore_av(q, k, v, N, H, d, topk, topk_idx, topk_score, out, s));
}

kmip_status_t kmip_backward_f32(const float* q, const float* k, const float* v, int64_t N,
                                int H, int d, int topk, const int32_t* graph_offsets,
                                int num_graphs, const int32_t* topk_idx,
                                const float* topk_score, const float* dout, float* dq,
                                float* dk, float* dv, void* workspace, size_t workspace_bytes,
                                kmip_stream_t stream) {
  return backward_impl(q, k, v, true, N, H, d, topk, graph_offsets, num_graphs, topk_idx,
                       topk_score, dout, dq, dk, dv, workspace, workspace_bytes, stream);
}

}  // extern "C"
