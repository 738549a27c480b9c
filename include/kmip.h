/*
 * libkmip -- k-Maximum-Inner-Product (k-MIP) attention on AMD Instinct MI355X
 * (gfx950).  C ABI.
 *
 * The operation (page "k-Maximum Inner Product Attention for Graph
 * Transformers and the Expressive Power of GraphGPS", Abstract): for every
 * query node i and head h, score every key node j of the same graph by the
 * inner product s_ij = <q_ih, k_jh>, keep the top-k keys, take a softmax over
 * those k scores and return the softmax-weighted sum of their value rows.
 * The N x N score matrix is never stored: memory is O(N * H * k) beyond the
 * inputs and outputs.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Layout: q, k, v, out, dout, dq, dk, dv are row-major [N][H][d] (the
 *    natural x.view(N, H, d) of an [N, H*d] matrix).  q, k, v are bfloat16
 *    bit patterns (uint16), or fp32 for the *_f32 entry points; every other
 *    floating-point array is fp32.
 *    topk_idx / topk_score are [N][H][topk].
 *  - Ownership: every pointer is device memory owned by the caller.  The
 *    library allocates nothing, keeps no state between calls and is
 *    reentrant; scratch space comes in through `workspace`.  The one
 *    exception is kmip_forward_no_workspace, whose scratch is a per-GPU
 *    library array (see its declaration).
 *  - Streams: all work is enqueued on `stream` (a hipStream_t; NULL is the
 *    default stream).  A return of KMIP_OK means the work was enqueued; the
 *    library never synchronises.
 *  - Graphs: graph_offsets is a device int32 array [num_graphs + 1], monotone,
 *    starting at 0 and ending at N; a query attends only to keys of its own
 *    graph (block-diagonal batching).  graph_offsets == NULL or
 *    num_graphs == 0 means one graph of N nodes.  These device-side
 *    preconditions, and finite inputs, are not checked.
 *  - Semantics: scores are the unscaled inner product (fold a temperature
 *    such as 1/sqrt(d) into q).  Heads are independent.  A query's
 *    candidates include itself.  Ties are broken by ascending node id.  A
 *    graph of n_b < topk nodes uses k_eff = n_b keys; unused slots hold index
 *    -1 and score -inf.  Results are bitwise deterministic.
 *  - Errors: arguments are validated on the host before any HIP call;
 *    nothing is enqueued when a check fails.
 *      null required pointer, N < 1, H < 1, num_graphs < 0,
 *      num_graphs >= 2 with graph_offsets == NULL, q/k/v/out/dout/dq/dk/dv
 *      not 16-byte aligned, workspace not aligned (16 bytes forward,
 *      256 bytes backward)                     -> KMIP_ERR_INVALID_VALUE
 *      d not in {32, 64}, topk not in [1, 64],
 *      N * H * topk >= 2^31, H * d > 2^20        -> KMIP_ERR_UNSUPPORTED
 *      workspace smaller than the *_workspace_bytes figure
 *                                               -> KMIP_ERR_WORKSPACE
 *      a launch error reported by hipGetLastError -> KMIP_ERR_LAUNCH
 */
#ifndef KMIP_H_
#define KMIP_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  KMIP_OK = 0,
  KMIP_ERR_INVALID_VALUE = 1,
  KMIP_ERR_UNSUPPORTED = 2,
  KMIP_ERR_WORKSPACE = 3,
  KMIP_ERR_LAUNCH = 4
} kmip_status_t;

/* A hipStream_t, passed as an opaque pointer so that this header needs no
 * HIP include. */
typedef void* kmip_stream_t;

/* Static, NUL-terminated description of a status code. */
const char* kmip_status_string(kmip_status_t status);

/* Library version: major * 10000 + minor * 100 + patch. */
int kmip_version(void);

/* Bytes of device workspace kmip_forward needs for these sizes (0 is a valid
 * answer).  Depends only on the arguments. */
size_t kmip_forward_workspace_bytes(int64_t N, int H, int d, int topk, int num_graphs);

/* Bytes of device workspace kmip_backward needs for these sizes. */
size_t kmip_backward_workspace_bytes(int64_t N, int H, int d, int topk, int num_graphs);

/*
 * k-MIP attention forward (page "k-Maximum Inner Product Attention for Graph
 * Transformers ...", Abstract: top-k selection by inner product, softmax
 * over the selected scores, weighted sum of the selected value rows).
 *
 *  q, k, v      in   bf16 [N][H][d]
 *  out          out  fp32 [N][H][d]
 *  topk_idx     out  int32 [N][H][topk], global node ids, best first
 *  topk_score   out  fp32 [N][H][topk], the selected inner products (kept for
 *                    kmip_backward)
 *  workspace    scratch of at least kmip_forward_workspace_bytes(...) bytes
 *                    (may be NULL when that figure is 0)
 */
kmip_status_t kmip_forward(const void* q, const void* k, const void* v, int64_t N, int H,
                           int d, int topk, const int32_t* graph_offsets, int num_graphs,
                           float* out, int32_t* topk_idx, float* topk_score,
                           void* workspace, size_t workspace_bytes, kmip_stream_t stream);

/*
 * First stage of kmip_forward: the top-k selection alone (page "k-Maximum
 * Inner Product Attention for Graph Transformers ...", Abstract: the key
 * nodes with the k largest inner products per query).  Writes topk_idx and
 * topk_score exactly as kmip_forward does; the N x N scores exist only as
 * register tiles.  Arguments, workspace and errors as for kmip_forward
 * (v and out are not taken).
 */
kmip_status_t kmip_score_topk(const void* q, const void* k, int64_t N, int H, int d, int topk,
                              const int32_t* graph_offsets, int num_graphs, int32_t* topk_idx,
                              float* topk_score, void* workspace, size_t workspace_bytes,
                              kmip_stream_t stream);

/*
 * Second stage of kmip_forward: softmax over the saved scores of each row and
 * the weighted sum of the selected value rows (same page, Abstract).
 *  v                        in   bf16 [N][H][d]
 *  topk_idx, topk_score     in   as written by kmip_score_topk (rows sorted
 *                                best first; -1 / -inf on unused slots)
 *  out                      out  fp32 [N][H][d]
 * Needs no workspace.  Errors as for kmip_forward.
 */
kmip_status_t kmip_gather_softmax_av(const void* v, int64_t N, int H, int d, int topk,
                                     const int32_t* topk_idx, const float* topk_score,
                                     float* out, kmip_stream_t stream);

/*
 * k-MIP attention backward with the forward selection held fixed (page
 * "k-Maximum Inner Product Attention for Graph Transformers ...", Appendix J,
 * Table 10: the training setting, whose forward and backward passes the page
 * times separately; the gradient is that of the Abstract's operation, which
 * is piecewise constant in the selection).  Gradients of
 * L = sum(dout * out) flow through the selected entries only.  With
 * p = softmax of the selected scores q_i . k_j, dp_ij = dout_i . v_j,
 * D_i = sum_j p_ij dp_ij and ds_ij = p_ij (dp_ij - D_i):
 *   dq_i = sum_j ds_ij k_j,  dk_j = sum_i ds_ij q_i,  dv_j = sum_i p_ij dout_i.
 * Every row of dq, dk and dv is written; keys no query selected get exact
 * zeros.  The key-side sums run in a fixed order (no atomics), so the result
 * is bitwise repeatable.  The selected scores are recomputed from q and k
 * with fp64 sums of the exact products (not read from topk_score), and
 * dp_ij - D_i is evaluated relative to entry 0's dp, so rows whose softmax
 * is nearly one-hot lose no accuracy to cancellation.
 *
 *  q, k, v                 in   bf16 [N][H][d] (as given to kmip_forward)
 *  topk_idx                in   as written by kmip_forward
 *  topk_score              in   as written by kmip_forward (checked for
 *                               non-null; the scores are recomputed)
 *  dout                    in   fp32 [N][H][d]
 *  dq, dk, dv              out  fp32 [N][H][d]
 *  workspace               scratch of at least kmip_backward_workspace_bytes(...)
 */
kmip_status_t kmip_backward(const void* q, const void* k, const void* v, int64_t N, int H,
                            int d, int topk, const int32_t* graph_offsets, int num_graphs,
                            const int32_t* topk_idx, const float* topk_score,
                            const float* dout, float* dq, float* dk, float* dv,
                            void* workspace, size_t workspace_bytes, kmip_stream_t stream);

/*
 * kmip_forward without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP-graph capture, tight serving loops,
 * harnesses that forbid allocation).  Arguments, results and errors are
 * those of kmip_forward; the scratch space (the same layout as
 * kmip_forward's workspace) is a library-owned device array of
 * KMIP_NO_WORKSPACE_BYTES per GPU, held until the process ends, on the device
 * current at the call (which must be the stream's device).
 *
 *  - Limit: sizes whose kmip_forward_workspace_bytes(...) exceeds
 *    KMIP_NO_WORKSPACE_BYTES return KMIP_ERR_WORKSPACE before anything is
 *    enqueued (about 3 * 10^6 (node, head) rows for topk <= 16; lists longer
 *    than 16 need 4 KB per row, so about 8000 rows).
 *  - Races: every call on one GPU uses the same scratch array, so calls whose
 *    work may overlap on that GPU (different streams, other threads) race;
 *    serialise them.  Calls on one stream are ordered and safe.
 *  - The first call on a device looks up the array's device address
 *    (hipGetSymbolAddress); no call allocates or frees memory.
 */
#define KMIP_NO_WORKSPACE_BYTES (32u << 20)

kmip_status_t kmip_forward_no_workspace(const void* q, const void* k, const void* v, int64_t N,
                                        int H, int d, int topk, const int32_t* graph_offsets,
                                        int num_graphs, float* out, int32_t* topk_idx,
                                        float* topk_score, kmip_stream_t stream);

/*
 * fp32-input variants.  The page's own k-MIP timings (same page, Tables 15
 * and 16) use fp32 inputs and arithmetic; these entry points take q, k, v as
 * fp32 [N][H][d] and are otherwise identical to kmip_forward / kmip_backward
 * (outputs, layouts, ties, padding, errors).
 *
 * Scores.  Each element is split as x = hi + lo + r with hi = bf16(x) and
 * lo = bf16(x - hi) (round to nearest even), and the matrix cores evaluate
 * q_hi.k_hi + q_hi.k_lo + q_lo.k_hi with fp32 accumulation of exact bf16
 * products.  The score error is at most about (3 * 2^-18 + 3d * 2^-24) *
 * sum_c |q_c k_c|, where rounding q and k to bf16 first would cost ~2^-8
 * relative.  The selection, its order and its tie rule refer to these
 * scores.  topk_score then holds each selected key's score recomputed in
 * fp32 from the fp32 rows (d products, fp32 accumulation), and the softmax
 * uses those (kmip_backward_f32 recomputes them in fp64), so neither the
 * output nor the gradients inherit the split's error; consecutive saved scores may therefore be out of order by
 * up to twice the split error.  The weighted sum reads fp32 v rows.  Every
 * element of q and k must be finite and below the bf16 maximum (~3.39e38) in
 * magnitude.
 *
 * Workspace: kmip_forward_f32_workspace_bytes(...), which is the
 * kmip_forward figure plus the split rows (about 12 * N * H * d bytes).
 */
size_t kmip_forward_f32_workspace_bytes(int64_t N, int H, int d, int topk, int num_graphs);

kmip_status_t kmip_forward_f32(const float* q, const float* k, const float* v, int64_t N, int H,
                               int d, int topk, const int32_t* graph_offsets, int num_graphs,
                               float* out, int32_t* topk_idx, float* topk_score,
                               void* workspace, size_t workspace_bytes, kmip_stream_t stream);

/*
 * Backward of kmip_forward_f32 (the selection held fixed, as kmip_backward):
 * q, k, v fp32 [N][H][d], topk_idx / topk_score as written by
 * kmip_forward_f32, workspace of kmip_backward_workspace_bytes(...) bytes.
 * The scores q.k and the products dout.v enter fp64 sums exactly, as in
 * kmip_backward.
 */
kmip_status_t kmip_backward_f32(const float* q, const float* k, const float* v, int64_t N,
                                int H, int d, int topk, const int32_t* graph_offsets,
                                int num_graphs, const int32_t* topk_idx,
                                const float* topk_score, const float* dout, float* dq,
                                float* dk, float* dv, void* workspace, size_t workspace_bytes,
                                kmip_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* KMIP_H_ */
