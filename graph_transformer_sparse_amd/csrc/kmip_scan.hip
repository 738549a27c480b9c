// Score scan with a fused running top-k (the O(N^2) part of k-MIP attention)
// and the ragged tile plan.
//
// Page "k-Maximum Inner Product Attention for Graph Transformers and the
// Expressive Power of GraphGPS", Abstract: each query keeps the key nodes with
// the k largest inner products, found by a top-k operation over scores that
// are never stored as an N x N matrix.
//
// Design (gfx950):
//  * A workgroup owns 128 query rows of one head and one graph (4 wavefronts
//    x 32 queries).  Each wavefront keeps its Q block in VGPRs as the MFMA B
//    operand for the whole scan.
//  * The graph's keys stream through LDS in chunks (coalesced 16-byte global
//    loads, double buffered, rows padded by 16 bytes so the MFMA A-operand
//    reads are free of bank conflicts).
//  * v_mfma_f32_32x32x16_bf16 computes a 32 keys x 32 queries score block
//    (fp32 accumulation of exact bf16 products).  Lane l holds query l%32 and
//    16 of the 32 keys, so every lane sees a private half of each query's key
//    stream, in ascending key order.
//  * Per lane: a sorted top-k list in registers and a threshold (the list's
//    k-th score).  A block is rejected with a max tree and one compare.  Hits
//    are appended to a per-lane LDS candidate buffer; when any lane's buffer
//    is nearly full the whole wavefront drains in lockstep, inserting
//    candidates into its register list, so the costly insertions run with
//    most lanes active.
//  * At the end the two half-lists of a query (lanes l and l^32) are merged
//    by rank counting with the tie rule (score descending, id ascending) and
//    written as the final topk_idx / topk_score rows.
#include "kmip_internal.h"

namespace kmip {
namespace {

constexpr float kInf = __builtin_inff();

template <int D>
struct ScanShape {
  static constexpr int NM = D / 16;                 // K=16 MFMAs per 32x32 block
  static constexpr int ROWB = 2 * D + 16;           // padded LDS bytes per key row
  static constexpr int TK = (D == 32) ? 128 : 64;   // keys per LDS chunk
  static constexpr int SUBT = TK / 32;              // 32-key sub-blocks per chunk
  static constexpr int CHUNK_BYTES = TK * ROWB;
  static constexpr int PPR = (2 * D) / 16;          // 16-byte pieces per key row
  static constexpr int PPT = TK * PPR / (SCAN_WAVES * 64);  // pieces per thread
  static_assert(TK * PPR % (SCAN_WAVES * 64) == 0, "chunk must split evenly");
};

// Insert (s, j) into a descending list.  The caller guarantees s beats the
// k-th entry.  Keys reach a lane in ascending id order, so on equal scores
// the entry already present (smaller id) stays first: strict compare.
template <int KP>
__device__ __forceinline__ void list_insert(float (&ls)[KP], int (&lj)[KP], float s, int j) {
  bool b[KP];
#pragma unroll
  for (int t = 0; t < KP; ++t) b[t] = s > ls[t];
#pragma unroll
  for (int t = KP - 1; t >= 1; --t) {
    ls[t] = b[t - 1] ? ls[t - 1] : (b[t] ? s : ls[t]);
    lj[t] = b[t - 1] ? lj[t - 1] : (b[t] ? j : lj[t]);
  }
  ls[0] = b[0] ? s : ls[0];
  lj[0] = b[0] ? j : lj[0];
}

// Largest float below x (x finite or -inf; -inf stays -inf).
__device__ __forceinline__ float next_down(float x) {
  if (x == -kInf) return x;
  if (x == 0.f) return __uint_as_float(0x80000001u);
  const unsigned u = __float_as_uint(x);
  return __uint_as_float(x > 0.f ? u - 1u : u + 1u);
}

// One kernel, two passes (PRE selects the pass).
//
// Pass 1 (PRE): the same MFMA scan, keeping only the running maximum of each
// of SCAN_CHUNKS consecutive chunks of every lane's key stream.  Chunk maxima
// are scores of distinct keys, so the k-th largest of a query's 2*SCAN_CHUNKS
// chunk maxima is a lower bound T on its k-th largest score; it is written to
// thr_buf.  A key with score < T cannot be selected.
//
// Pass 2 (!PRE): the exact running top-k, seeded with the threshold
// next_down(T) (a key scoring exactly T may still win on id), so that only a
// handful of keys per query ever reach the insertion path.
template <int D, int KP, bool PRE>
__global__ __launch_bounds__(SCAN_WAVES * 64) void score_topk_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, int64_t N, int H,
    int topk, const int32_t* __restrict__ offsets, int single_graph,
    const int2* __restrict__ tiles, float* __restrict__ thr_buf,
    int32_t* __restrict__ out_idx, float* __restrict__ out_score) {
  using S = ScanShape<D>;
  static_assert(SCAN_CAP * 8 == SCAN_CHUNKS * 4, "candidate and chunk areas share LDS");
  __shared__ __attribute__((aligned(16))) unsigned char kbuf[2 * S::CHUNK_BYTES];
  __shared__ __attribute__((aligned(16))) unsigned char wbuf[SCAN_WAVES * SCAN_CAP * 64 * 8];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int64_t lin = blockIdx.x;
  const int h = (int)(lin % H);
  const int64_t tile = lin / H;

  int64_t q0, kb, ke;
  if (single_graph) {
    q0 = tile * SCAN_QT;
    kb = 0;
    ke = N;
  } else {
    const int2 t = tiles[tile];
    if (t.x < 0) return;                 // beyond the planned tiles
    q0 = t.y;
    kb = offsets[t.x];
    ke = offsets[t.x + 1];
  }
  if (q0 >= ke) return;
  const int64_t q1 = (q0 + SCAN_QT < ke) ? q0 + SCAN_QT : ke;

  const int lrow = lane & 31;
  const int lhalf = lane >> 5;
  const int64_t qrow = q0 + wave * SCAN_QPW + lrow;
  const bool qvalid = qrow < q1;
  const bool wave_active = (q0 + wave * SCAN_QPW) < q1;
  const int64_t orow = qrow * H + h;

  // MFMA B operand: Q[query][16m + 8*lhalf .. +7] for query = lane%32.
  bf16x8_t qb[S::NM];
  {
    const int64_t ql = qvalid ? qrow : (q1 - 1);
    const uint16_t* qp = Q + (ql * H + h) * D + 8 * lhalf;
#pragma unroll
    for (int m = 0; m < S::NM; ++m) qb[m] = *reinterpret_cast<const bf16x8_t*>(qp + 16 * m);
  }

  // Slots [0, KP-topk) hold +inf sentinels that nothing displaces, so the
  // live top-k always occupies the tail and its k-th score is ls[KP-1].
  const int nsent = KP - topk;
  float ls[KP];
  int lj[KP];
#pragma unroll
  for (int t = 0; t < KP; ++t) {
    ls[t] = t < nsent ? kInf : -kInf;
    lj[t] = -1;
  }

  // Pass 1 state: running chunk maximum; chunk i of this lane at cml[i*64].
  const int64_t nkeys = ke - kb;
  const int nsub = (int)((nkeys + 31) / 32);
  const int spc = (nsub + SCAN_CHUNKS - 1) / SCAN_CHUNKS;   // sub-blocks per chunk
  float* cml = reinterpret_cast<float*>(wbuf) + wave * SCAN_CHUNKS * 64 + lane;
  float cm = -kInf;
  // Pass 2 state: reject threshold and the lane's candidate buffer.
  float thr = kInf;
  int cnt = 0;
  uint2* cb = reinterpret_cast<uint2*>(wbuf) + wave * SCAN_CAP * 64 + lane;
  if constexpr (PRE) {
#pragma unroll 1
    for (int i = 0; i < SCAN_CHUNKS; ++i) cml[i * 64] = -kInf;
  } else {
    if (qvalid) thr = next_down(thr_buf[orow]);
  }
  // Retire the operand loads here so that the loop's MFMAs never wait on the
  // vector-memory counter, which the K prefetch keeps busy.
  __builtin_amdgcn_s_waitcnt(0x0f70);   // vmcnt(0)

  auto drain = [&]() __attribute__((always_inline)) {
    for (int c = 0; __ballot(c < cnt) != 0ull; ++c) {
      if (c < cnt) {
        const uint2 e = cb[c * 64];
        const float sv = __uint_as_float(e.x);
        if (sv > thr) {
          list_insert<KP>(ls, lj, sv, (int)e.y);
          thr = fmaxf(thr, ls[KP - 1]);
        }
      }
    }
    cnt = 0;
  };

  const int nchunks = (int)((nkeys + S::TK - 1) / S::TK);

  // Each thread moves PPT 16-byte pieces of a key chunk: global -> VGPR -> LDS.
  uint4 stg0, stg1;
  static_assert(S::PPT == 2, "two staging pieces per thread");
  const int prow0 = tid / S::PPR, ppart0 = tid % S::PPR;
  const int prow1 = (tid + SCAN_WAVES * 64) / S::PPR, ppart1 = (tid + SCAN_WAVES * 64) % S::PPR;
  const uint16_t* kh = K + (int64_t)h * D;
  const int64_t kstride = (int64_t)H * D;
#define KMIP_GLOAD(c)                                                              \
  {                                                                                \
    int64_t k0 = kb + (int64_t)(c) * S::TK + prow0;                                \
    int64_t k1 = kb + (int64_t)(c) * S::TK + prow1;                                \
    k0 = k0 < ke ? k0 : ke - 1;                                                    \
    k1 = k1 < ke ? k1 : ke - 1;                                                    \
    stg0 = *reinterpret_cast<const uint4*>(kh + k0 * kstride + ppart0 * 8);        \
    stg1 = *reinterpret_cast<const uint4*>(kh + k1 * kstride + ppart1 * 8);        \
  }
#define KMIP_LSTORE(buf)                                                           \
  {                                                                                \
    unsigned char* kd = kbuf + (buf) * S::CHUNK_BYTES;                             \
    *reinterpret_cast<uint4*>(kd + prow0 * S::ROWB + ppart0 * 16) = stg0;          \
    *reinterpret_cast<uint4*>(kd + prow1 * S::ROWB + ppart1 * 16) = stg1;          \
  }

  KMIP_GLOAD(0);
  KMIP_LSTORE(0);
  __syncthreads();

  for (int c = 0; c < nchunks; ++c) {
    if (c + 1 < nchunks) KMIP_GLOAD(c + 1);
    const unsigned char* kc = kbuf + (c & 1) * S::CHUNK_BYTES;
    const int64_t cbase = kb + (int64_t)c * S::TK;
    const bool partial = cbase + S::TK > ke;
    if (wave_active) {
      // Software pipeline: the MFMAs of sub-block st+1 are issued before the
      // scores of sub-block st are examined.
      floatx16_t acc[2];
#define KMIP_MFMA(st, dst)                                                          \
  {                                                                               \
    dst = floatx16_t{};                                                           \
    _Pragma("unroll") for (int m = 0; m < S::NM; ++m) {                           \
      const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(                      \
          kc + ((st) * 32 + lrow) * S::ROWB + m * 32 + lhalf * 16);               \
      dst = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qb[m], dst, 0, 0, 0);      \
    }                                                                             \
  }
      KMIP_MFMA(0, acc[0]);
#pragma unroll
      for (int st = 0; st < S::SUBT; ++st) {
        if (st + 1 < S::SUBT) KMIP_MFMA(st + 1, acc[(st + 1) & 1]);
        // acc[r] = <k_key, q_query>, key = key0 + 8*(r/4) + (r%4), query = lane%32.
        const int key0 = (int)(cbase + st * 32 + 4 * lhalf);
        float s[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) s[r] = acc[st & 1][r];
        if (partial) {
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (key0 + 8 * (r >> 2) + (r & 3) >= ke) s[r] = -kInf;
        }
        if constexpr (PRE) {
          cm = fmaxf(fmaxf(fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3])),
                           fmaxf(fmaxf(s[4], s[5]), fmaxf(s[6], s[7]))),
                     fmaxf(fmaxf(fmaxf(s[8], s[9]), fmaxf(s[10], s[11])),
                           fmaxf(fmaxf(s[12], s[13]), fmaxf(fmaxf(s[14], s[15]), cm))));
          const int t = c * S::SUBT + st;              // sub-block index, uniform
          if ((t + 1) % spc == 0 || t + 1 == nsub) {
            if (t < nsub) cml[(t / spc) * 64] = cm;
            cm = -kInf;
          }
        } else {
          float g[4];
#pragma unroll
          for (int qq = 0; qq < 4; ++qq)
            g[qq] = fmaxf(fmaxf(s[4 * qq], s[4 * qq + 1]), fmaxf(s[4 * qq + 2], s[4 * qq + 3]));
          const float mx = fmaxf(fmaxf(g[0], g[1]), fmaxf(g[2], g[3]));
          if (__ballot(mx > thr) != 0ull) {
            // At most 4 appends per passing quarter: make room first, so the
            // sub-block has a single drain site.
            int room = cnt;
#pragma unroll
            for (int qq = 0; qq < 4; ++qq) room += g[qq] > thr ? 4 : 0;
            if (__ballot(room > SCAN_CAP) != 0ull) drain();
#pragma unroll
            for (int qq = 0; qq < 4; ++qq) {
              if (__ballot(g[qq] > thr) != 0ull) {
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                  const float sv = s[4 * qq + r];
                  if (sv > thr) {
                    cb[cnt * 64] = make_uint2(__float_as_uint(sv), (unsigned)(key0 + 8 * qq + r));
                    ++cnt;
                  }
                }
              }
            }
          }
        }
      }
#undef KMIP_MFMA
    }
    if (c + 1 < nchunks) KMIP_LSTORE((c + 1) & 1);
    __syncthreads();
  }
#undef KMIP_GLOAD
#undef KMIP_LSTORE
  if (!wave_active) return;

  if constexpr (PRE) {
    // k-th largest of the query's chunk maxima: this lane's and its partner's
    // (lane ^ 32 scans the other half of the same query's keys).
    __builtin_amdgcn_wave_barrier();
    const float* cmp = reinterpret_cast<const float*>(wbuf) + wave * SCAN_CHUNKS * 64 + (lane ^ 32);
    float t = -kInf;
#pragma unroll 1
    for (int i = 0; i < 2 * SCAN_CHUNKS; ++i) {
      const float v = (i & 1) ? cmp[(i >> 1) * 64] : cml[(i >> 1) * 64];
      if (v > t) {
        list_insert<KP>(ls, lj, v, 0);
        t = ls[KP - 1];
      }
    }
    if (qvalid && lhalf == 0) thr_buf[orow] = t;
    return;
  } else {
    drain();

    // Merge the two half-lists of each query by rank: live entry t of my list
    // (slots [nsent, KP)) lands at (t - nsent) + the number of partner live
    // entries ordered before it.  Lower-half lanes win exact (score, id)
    // ties, which only padding entries (-inf, -1) can produce.
    float ps[KP];
    int pj[KP];
#pragma unroll
    for (int t = 0; t < KP; ++t) {
      ps[t] = __shfl_xor(ls[t], 32);
      pj[t] = __shfl_xor(lj[t], 32);
    }
    if (!qvalid) return;
    const bool lower = lhalf == 0;
    int32_t* oi = out_idx + orow * topk;
    float* os = out_score + orow * topk;
#pragma unroll
    for (int t = 0; t < KP; ++t) {
      if (t >= nsent) {
        int rank = t - nsent;
#pragma unroll
        for (int u = 0; u < KP; ++u) {
          const bool before = u >= nsent &&
                              (ps[u] > ls[t] ||
                               (ps[u] == ls[t] && (lower ? pj[u] < lj[t] : pj[u] <= lj[t])));
          rank += before ? 1 : 0;
        }
        if (rank < topk) {
          oi[rank] = lj[t];
          os[rank] = lj[t] < 0 ? -kInf : ls[t];
        }
      }
    }
  }
}

// ------------------------------------------------------------------ tile plan
constexpr int PLAN_THREADS = 1024;

// One block: tile_start[b] = sum over earlier graphs of ceil(n_b / SCAN_QT).
__global__ __launch_bounds__(PLAN_THREADS) void tile_count_scan_kernel(
    const int32_t* __restrict__ offsets, int B, int32_t* __restrict__ tile_start) {
  __shared__ int32_t buf[PLAN_THREADS];
  int32_t carry = 0;
  for (int base = 0; base < B; base += PLAN_THREADS) {
    const int b = base + (int)threadIdx.x;
    int32_t c = 0;
    if (b < B) {
      const int32_t nb = offsets[b + 1] - offsets[b];
      c = nb > 0 ? (nb + SCAN_QT - 1) / SCAN_QT : 0;
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

__global__ void tile_fill_kernel(const int32_t* __restrict__ offsets, int B,
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
  tiles[t] = make_int2(lo, offsets[lo] + (int)(t - tile_start[lo]) * SCAN_QT);
}

template <int D, int KP>
hipError_t launch_scan_t(const uint16_t* q, const uint16_t* k, int64_t N, int H, int topk,
                         const int32_t* offsets, int single, const int2* tiles,
                         int64_t ntiles, float* thr, int32_t* idx, float* score, hipStream_t s) {
  const dim3 grid((unsigned)(ntiles * H)), block(SCAN_WAVES * 64);
  hipLaunchKernelGGL((score_topk_kernel<D, KP, true>), grid, block, 0, s, q, k, N, H, topk,
                     offsets, single, tiles, thr, idx, score);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((score_topk_kernel<D, KP, false>), grid, block, 0, s, q, k, N, H, topk,
                     offsets, single, tiles, thr, idx, score);
  return hipGetLastError();
}

template <int D>
hipError_t launch_scan_d(int kp, const uint16_t* q, const uint16_t* k, int64_t N, int H,
                         int topk, const int32_t* offsets, int single, const int2* tiles,
                         int64_t ntiles, float* thr, int32_t* idx, float* score, hipStream_t s) {
  switch (kp) {
    case 5: return launch_scan_t<D, 5>(q, k, N, H, topk, offsets, single, tiles, ntiles, thr, idx, score, s);
    case 8: return launch_scan_t<D, 8>(q, k, N, H, topk, offsets, single, tiles, ntiles, thr, idx, score, s);
    case 15: return launch_scan_t<D, 15>(q, k, N, H, topk, offsets, single, tiles, ntiles, thr, idx, score, s);
    case 16: return launch_scan_t<D, 16>(q, k, N, H, topk, offsets, single, tiles, ntiles, thr, idx, score, s);
    case 32: return launch_scan_t<D, 32>(q, k, N, H, topk, offsets, single, tiles, ntiles, thr, idx, score, s);
    case 45: return launch_scan_t<D, 45>(q, k, N, H, topk, offsets, single, tiles, ntiles, thr, idx, score, s);
    case 48: return launch_scan_t<D, 48>(q, k, N, H, topk, offsets, single, tiles, ntiles, thr, idx, score, s);
    case 64: return launch_scan_t<D, 64>(q, k, N, H, topk, offsets, single, tiles, ntiles, thr, idx, score, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

int scan_list_len(int topk) {
  static const int lens[] = {5, 8, 15, 16, 32, 45, 48, 64};
  for (int L : lens)
    if (topk <= L) return L;
  return -1;
}

hipError_t launch_tile_plan(const int32_t* offsets, int num_graphs, int64_t max_tiles,
                            int32_t* tile_start, int2* tiles, hipStream_t s) {
  hipLaunchKernelGGL(tile_count_scan_kernel, dim3(1), dim3(PLAN_THREADS), 0, s, offsets,
                     num_graphs, tile_start);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const unsigned blocks = (unsigned)ceil_div(max_tiles, 256);
  hipLaunchKernelGGL(tile_fill_kernel, dim3(blocks), dim3(256), 0, s, offsets, num_graphs,
                     tile_start, max_tiles, tiles);
  return hipGetLastError();
}

hipError_t launch_score_topk(const uint16_t* q, const uint16_t* k, int64_t N, int H, int d,
                             int topk, const int32_t* offsets, int num_graphs,
                             const int2* tiles, int64_t max_tiles, float* thr,
                             int32_t* topk_idx, float* topk_score, hipStream_t s) {
  const int kp = scan_list_len(topk);
  const int single = (offsets == nullptr || num_graphs <= 1) ? 1 : 0;
  const int64_t ntiles = single ? ceil_div(N, SCAN_QT) : max_tiles;
  if (d == 32)
    return launch_scan_d<32>(kp, q, k, N, H, topk, offsets, single, tiles, ntiles, thr,
                             topk_idx, topk_score, s);
  if (d == 64)
    return launch_scan_d<64>(kp, q, k, N, H, topk, offsets, single, tiles, ntiles, thr,
                             topk_idx, topk_score, s);
  return hipErrorInvalidValue;
}

}  // namespace kmip
