// Score-scan kernels, included once per head dimension by kmip_scan_d*.hip
// (one translation unit per dimension, so the instantiations compile in
// parallel).
//
// Page "k-Maximum Inner Product Attention for Graph Transformers and the
// Expressive Power of GraphGPS", Abstract: each query keeps the key nodes with
// the k largest inner products, found by a top-k operation over scores that
// are never stored as an N x N matrix.
//
// Design (gfx950):
//  * Work is split into sub-tiles of query rows of one head and one graph: a
//    workgroup of W wavefronts, each owning 32 rows (W = 16 for one graph
//    and lists of at most 16; W = 8 for longer lists and for batched
//    graphs).  A wavefront keeps its Q rows in VGPRs as MFMA B operands for
//    the whole scan.
//  * The graph's keys stream through an LDS ring of two chunks (64 KB, 1024
//    keys at d = 32, in the threshold pass; 32 KB in the selection pass, which
//    also holds candidate buffers), fetched with direct global->LDS loads one
//    chunk ahead.  A chunk is stored in MFMA operand order (see ScanShape), so
//    each A operand is one contiguous, conflict-free 1 KB LDS read.
//  * v_mfma_f32_32x32x16_bf16 scores 32 keys x 32 queries (fp32 accumulation
//    of exact bf16 products).  Lane l holds query l%32 and 16 of the 32 keys,
//    so each lane sees a private half of every query's key stream, in
//    ascending key order.
//  * Two passes.  The threshold pass scores a sample of the chunks (with
//    lists of at most 16: every chunk below 2^14 keys, every fourth up to
//    2^16 keys, every sixteenth beyond, and eight times sparser still when
//    the queries are grouped; every second for longer lists) and keeps, per
//    lane and query, the top-k of the maxima of SCAN_CHUNKS consecutive
//    ranges of those keys (uniform, lockstep insertions).  These maxima are
//    scores of distinct keys, so the k-th largest over both halves is a lower
//    bound T of the query's k-th score.  With grouped queries a window pass
//    (window_thresh_kernel) raises T with the exact k-th score over the keys
//    of nearby positions in the query order.
//    The selection pass then runs the exact running top-k seeded with
//    next_down(T): a block of scores is rejected with a max tree and one
//    compare, rare hits go to a per-lane LDS candidate buffer, and buffers
//    are drained in lockstep into per-lane register lists.  At the end the
//    two half-lists of a query (lanes l, l^32) are merged under the tie rule
//    (score descending, id ascending).  Lists longer than 16 collect their
//    candidates in per-row arrays instead (COLLECT below).
//  * One graph: each head's queries are first grouped by their nearest of
//    about N/96 pivot queries (largest inner product), the groups placed in
//    the order of their pivots' nearest anchor, so a wavefront's 32 queries
//    tend to share their candidate keys.  A persistent grid of exactly the co-resident
//    workgroups, each taking an equal contiguous range of query blocks (no
//    partial last round), with logical ids permuted so that the workgroups of
//    one XCD share a head and its keys in that XCD's L2.  Batched graphs: one
//    workgroup per planned sub-tile; sub-blocks past a graph's last key are
//    skipped.
#pragma once
#include "kmip_internal.h"

namespace kmip {
namespace {

constexpr float kInf = __builtin_inff();
constexpr int QB = 1;                       // query blocks of 32 per wavefront
// Per pass: LDS chunk size in 16 KB units (LPW: 1 KB loads per wavefront and
// chunk), ring depth, and sub-blocks per batch (LDS reads, then MFMAs, then
// scores).  Large chunks amortise the workgroup barrier of every chunk; the
// selection pass keeps room for its candidate buffers.  With a ring of two,
// chunk c + 1 is fetched while chunk c is scored.
#ifndef KMIP_SCAN_BATCH
#define KMIP_SCAN_BATCH 2
#endif
#ifndef KMIP_PRE_SAMPLE
#define KMIP_PRE_SAMPLE 4
#endif
// Scan modes.  THRESH: per-row lower bound T of the k-th score.  SELECT:
// exact running top-k in per-lane register lists.  COLLECT (lists longer
// than 16): every key scoring above next_down(T) is appended to a per-row
// candidate array, and a second kernel selects the top-k from it; rows whose
// arrays overflow are then recomputed by SELECT.
// RANK: SELECT restricted to the rows whose candidate arrays overflowed,
// computing 16 ranks of each per call (see Scanner::run).
constexpr int M_THRESH = 0, M_SELECT = 1, M_COLLECT = 2, M_RANK = 3;
template <int MODE> struct PassCfg;
// SAMPLE: THRESH scores every SAMPLE-th chunk only.  Any subset of a
// query's keys yields a valid lower bound of its k-th score; a sparser subset
// gives a looser bound, i.e. more candidates in the later pass.
template <> struct PassCfg<M_THRESH> {
  static constexpr int LPW = 4, NBUF = 2, BATCH = KMIP_SCAN_BATCH, SAMPLE = KMIP_PRE_SAMPLE;
};
template <> struct PassCfg<M_SELECT> {
  static constexpr int LPW = 2, NBUF = 2, BATCH = KMIP_SCAN_BATCH, SAMPLE = 1;
};
template <> struct PassCfg<M_RANK> : PassCfg<M_SELECT> {};
template <> struct PassCfg<M_COLLECT> {
  static constexpr int LPW = 2, NBUF = 2, BATCH = KMIP_SCAN_BATCH, SAMPLE = 1;
};

// Chunk layout in LDS ("operand order"): the chunk is a sequence of 1 KB
// blocks, one per (32-key sub-block st, K-slice m of the MFMA), block index
// st * NM + m.  Inside a block, lane l's 16 bytes sit at l * 16 and hold the
// bf16 elements [16m + 8(l/32), 16m + 8(l/32) + 8) of key st*32 + l%32: the
// A operand of v_mfma_f32_32x32x16_bf16 for that lane.  A wavefront then reads
// each operand as one contiguous 1 KB ds_read_b128 (no bank conflicts), and
// the direct global->LDS load that fills a block writes it in the same lane
// order.
//
// D = 96 and 192 are the rows of the split-precision scan (three bf16 terms
// per fp32 element pair, see kmip_split.hip); their chunks hold three
// operand blocks per wavefront.
template <int D, int MODE, int W>
struct ScanShape {
  static constexpr int NM = D / 16;                 // K=16 MFMAs per 32x32 block
  static constexpr int ROWB = 2 * D;                // bytes per key row
  static constexpr int LPW = D % 3 == 0 ? 3 : PassCfg<MODE>::LPW;  // blocks per wave
  static constexpr int NBUF = PassCfg<MODE>::NBUF;   // LDS ring depth
  static constexpr int SAMPLE = PassCfg<MODE>::SAMPLE;  // chunk stride
  static constexpr int CHUNK_BYTES = 1024 * W * LPW;
  static constexpr int TK = CHUNK_BYTES / ROWB;      // keys per chunk
  static constexpr int SUBT = TK / 32;               // 32-key sub-blocks per chunk
  static_assert(SUBT * NM == W * LPW, "LPW operand blocks per wavefront");
  static_assert(NBUF == 2 || NBUF == 3, "ring depth");
};

// Insert (s, j) into a descending list.  The caller guarantees s beats the
// k-th entry.  Keys reach a lane in ascending id order, so on equal scores
// the entry already present (smaller id) stays first: strict compare.  With
// p the first slot that s beats, slot t >= 1 becomes ls[t] (t < p), s
// (t = p) or ls[t-1] (t > p), which for a descending list is the median of
// (ls[t], ls[t-1], s): one v_med3 per slot; ids follow the compares.
template <int KP>
__device__ __forceinline__ void list_insert(float (&ls)[KP], int (&lj)[KP], float s, int j) {
  static_assert(KP <= 16, "register lists of the selection pass");
  bool b[KP];
#pragma unroll
  for (int t = 0; t < KP; ++t) b[t] = s > ls[t];
#pragma unroll
  for (int t = KP - 1; t >= 1; --t) {
    lj[t] = b[t] ? (b[t - 1] ? lj[t - 1] : j) : lj[t];
    ls[t] = __builtin_amdgcn_fmed3f(ls[t], ls[t - 1], s);
  }
  lj[0] = b[0] ? j : lj[0];
  ls[0] = fmaxf(ls[0], s);
}

template <int KP>
__device__ __forceinline__ void value_insert(float (&ls)[KP], float s) {
#pragma unroll
  for (int t = KP - 1; t >= 1; --t) ls[t] = __builtin_amdgcn_fmed3f(ls[t], ls[t - 1], s);
  ls[0] = fmaxf(ls[0], s);
}

// Largest float below x (x finite or -inf; -inf stays -inf).
__device__ __forceinline__ float next_down(float x) {
  if (x == -kInf) return x;
  if (x == 0.f) return __uint_as_float(0x80000001u);
  const unsigned u = __float_as_uint(x);
  return __uint_as_float(x > 0.f ? u - 1u : u + 1u);
}

// Largest of a lane's 16 scores of a 32x32 block, as one max and seven
// three-input maxima.  The hit path tests quarters with plain compares, so
// that the compiler shares no partial maxima with it and keeps this tree.
__device__ __forceinline__ float block_max(const floatx16_t& x) {
  const float m0 = fmaxf(fmaxf(x[0], x[1]), x[2]);
  const float m1 = fmaxf(fmaxf(x[3], x[4]), x[5]);
  const float m2 = fmaxf(fmaxf(x[6], x[7]), x[8]);
  const float m3 = fmaxf(fmaxf(x[9], x[10]), x[11]);
  const float m4 = fmaxf(fmaxf(x[12], x[13]), x[14]);
  return fmaxf(fmaxf(fmaxf(m0, m1), m2), fmaxf(fmaxf(m3, m4), x[15]));
}

// Some score of quarter qq (scores 4qq .. 4qq + 3) exceeds t.
__device__ __forceinline__ bool quarter_hit(const floatx16_t& x, int qq, float t) {
  return (x[4 * qq] > t) | (x[4 * qq + 1] > t) | (x[4 * qq + 2] > t) | (x[4 * qq + 3] > t);
}

// Pruned selection: the streaming pass takes the range of query blocks
// that wid belongs to (decided once the range's bound pass has run).
__device__ __forceinline__ bool prune_range_stream(const ScanArgs& a, int64_t wid) {
  return a.range_stream[(int)wid >> a.live_shift] != 0;
}

struct SubTile {
  int h;
  int64_t q0, q1;     // query rows [q0, q1)
  int64_t kb, ke;     // key range of the graph
};

template <int D, int KP, int MODE, int W>
struct Scanner {
  static constexpr bool PRE = MODE == M_THRESH;
  static constexpr bool RANK = MODE == M_RANK;
  static constexpr bool SEL = MODE == M_SELECT || RANK;   // register-list selection
  // uint2 entries of LDS per wavefront: the candidate buffer (SCAN_CAP per
  // lane); after the last drain the same space holds the upper lanes' lists
  // for the merge.
  static constexpr int CBW = SCAN_CAP * 64;
  using S = ScanShape<D, MODE, W>;
  // Chunk stride of this pass.  Long lists take a denser sample: their
  // candidates must fit the per-row arrays of the collecting pass.
  static constexpr int SAMPLE = PRE && KP > 16 ? 2 : S::SAMPLE;
  unsigned char* kbuf;        // S::NBUF chunks (read side)
  unsigned kbuf_lds;          // LDS byte address of kbuf (direct-load side)
  uint2* cbuf;                // per-lane candidate buffers (SELECT)
  const ScanArgs& a;
  const uint16_t* Q;
  const uint16_t* K;
  const int32_t* perm;        // query order per head, [H][N] (one graph), or null
  int64_t N;
  int H, topk;
  float* thr_buf;
  int32_t* out_idx;
  float* out_score;

  // Direct global->LDS load of chunk c into ring slot `slot`: wave w fills
  // operand blocks w + i * W (i < LPW), lane l writing 16 bytes at
  // l * 16 of the block.  The address is a per-chunk uniform base (SGPRs)
  // plus a 32-bit lane offset; rows past the graph's last key re-read the
  // last key.  Written as inline assembly so that the compiler does not treat
  // ring reads as aliasing the loads in flight: completion is tracked by the
  // explicit vmcnt waits of the chunk loop.  The instruction writes no VGPR.
  __device__ __forceinline__ void issue(const SubTile& t, int c, int slot, int wave, int lane) {
    const int64_t first = t.kb + (int64_t)c * S::TK;
    const int64_t left = t.ke - first;
    const int rmax = (int)(left < S::TK ? left : S::TK) - 1;
    const uint16_t* base = K + (first * H + t.h) * D;
#pragma unroll
    for (int i = 0; i < S::LPW; ++i) {
      const int blk = wave + i * W;
      const int row = (blk / S::NM) * 32 + (lane & 31);
      const int piece = 2 * (blk % S::NM) + (lane >> 5);
      const unsigned off =
          (unsigned)(row < rmax ? row : rmax) * (unsigned)(H * S::ROWB) + (unsigned)piece * 16u;
      const unsigned lds =
          kbuf_lds + (unsigned)(slot * S::CHUNK_BYTES + blk * 1024);
      asm volatile("global_load_lds_dwordx4 %0, %1" ::"v"(off), "s"(base),
                   "{m0}"(__builtin_amdgcn_readfirstlane(lds))
                   : "memory");
    }
  }

  static __device__ __forceinline__ int64_t uniform64(int64_t v) {
    const int lo = __builtin_amdgcn_readfirstlane((int)(v & 0xffffffff));
    const int hi = __builtin_amdgcn_readfirstlane((int)(v >> 32));
    return (int64_t)(((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo);
  }

  __device__ __forceinline__ void run(const SubTile& tin) {
    // The sub-tile is the same for the whole workgroup: keep it in SGPRs.
    const SubTile t{__builtin_amdgcn_readfirstlane(tin.h), uniform64(tin.q0), uniform64(tin.q1),
                    uniform64(tin.kb), uniform64(tin.ke)};
    // The wave index is uniform: keep it (and all that derives from it) scalar.
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lrow = lane & 31, lhalf = lane >> 5;
    const int64_t nkeys = t.ke - t.kb;
    const int nchunks = (int)((nkeys + S::TK - 1) / S::TK);
    // Chunks scored by this pass: c = j * sample for j < nproc.  With short
    // lists the stride follows the graph's size: every chunk below 2^14 keys
    // (there the bound from a sample is so loose that the selection pass
    // spends most of its time on candidates: the 64-graph batch of 500-5000
    // nodes and N = 8192 measured 9-15 % faster than at stride 4), SAMPLE up
    // to 2^16 keys (stride 2 at N = 31623 was 5 % slower), 4 * SAMPLE from
    // 2^16 keys on (1-2 % faster than 2 * SAMPLE at N = 10^5 and 5 * 10^5).
    // With a query order the window pass (window_thresh_kernel) supplies the
    // tight bound, and this sample only guards inputs without cluster
    // structure: 8 times sparser (N = 10^5: 3.10 -> 3.02 ms for the whole
    // selection; dropping it entirely gained no more).
    // Long lists on the pruned path (whose ranges with cluster structure also
    // get the window bound) sample every fourth chunk: at N = 10^5, k = 45
    // the threshold pass 1.79 -> 1.05 ms, with candidate arrays of 256 per
    // lane half, which then almost never overflow (every sixteenth chunk, or
    // every fourth with 128 entries, left so many rows overflowing that the
    // rank passes cost more than was saved).
    const int sparse = perm != nullptr ? 8 : 1;
    const int sample = PRE && KP > 16 && a.kop != nullptr ? 2 * SAMPLE
                       : !(PRE && KP <= 16)       ? SAMPLE
                       : nkeys >= (int64_t)1 << 16 ? 4 * SAMPLE * sparse
                       : nkeys >= (int64_t)1 << 14 ? SAMPLE * sparse
                                                   : 1;
    const int nproc = (nchunks + sample - 1) / sample;

    // The ring may still be read by slower waves of the previous sub-tile.
    __syncthreads();

    int64_t qrow[QB];
    bool qvalid[QB], bact[QB];
    bf16x8_t qb[QB][S::NM];
#pragma unroll
    for (int b = 0; b < QB; ++b) {
      const int64_t first = t.q0 + (wave * QB + b) * 32;
      // Positions [q0, q1) index the head's query order; rows are node ids.
      const int64_t pos = first + lrow;
      bact[b] = first < t.q1;
      qvalid[b] = pos < t.q1;
      const int64_t pl = qvalid[b] ? pos : t.q1 - 1;
      qrow[b] = perm ? (int64_t)perm[t.h * N + pl] : pl;
      const uint16_t* qp = Q + (qrow[b] * H + t.h) * D + 8 * lhalf;
#pragma unroll
      for (int m = 0; m < S::NM; ++m) qb[b][m] = *reinterpret_cast<const bf16x8_t*>(qp + 16 * m);
    }
    // Rows this call writes.  A rank pass (after COLLECT) recomputes only the
    // rows whose candidate arrays overflowed; after the pruned selection the
    // selection pass takes only the query blocks left to it (qb_cnt at least
    // dense_min).  Both skip sub-tiles with no such row.
    bool keep[QB];
    bool wave_rows = bact[0];
#pragma unroll
    for (int b = 0; b < QB; ++b) keep[b] = qvalid[b];
    bool filtered = RANK;
    if constexpr (RANK) {
      const int64_t r = qrow[0] * H + t.h;
      keep[0] = qvalid[0] && (a.cand_cnt[2 * r] > a.cap || a.cand_cnt[2 * r + 1] > a.cap);
      wave_rows = __ballot(keep[0]) != 0ull;
    } else if constexpr ((MODE == M_SELECT || MODE == M_COLLECT) && (D == 32 || D == 64 || D == 96)) {
      static_assert(QB == 1, "one query block per wavefront");
      if (a.range_stream != nullptr) {
        filtered = true;
        wave_rows = bact[0] && prune_range_stream(a, t.h * a.nkb + t.q0 / 32 + wave);
        keep[0] = keep[0] && wave_rows;
      }
    }
    if (filtered) {
      // The first ring word serves as the workgroup's flag: no key load is
      // in flight here and every wavefront is past the previous sub-tile.
      volatile int* wg_flag = reinterpret_cast<volatile int*>(kbuf);
      if (tid == 0) *wg_flag = 0;
      __syncthreads();
      if (wave_rows && lane == 0) *wg_flag = 1;
      __syncthreads();
      const bool any = *wg_flag != 0;
      __syncthreads();                        // all have read it before the ring is refilled
      if (!any) return;                       // uniform over the workgroup
    }
    const bool wave_active = wave_rows;
    const int aoff = lane * 16;

    // This call computes ranks [rank0, rank0 + kk) of each row: all of them
    // (rank0 = 0, kk = topk) except in the rank passes that recompute rows
    // with overflowing candidate arrays for lists longer than 16, 16 ranks
    // at a time.  A rank pass keeps only keys ordered after the row's entry
    // rank0 - 1 (score descending, id ascending), written by the pass before.
    const int rank0 = RANK ? a.rank0 : 0;
    const int kk = topk - rank0 < KP ? topk - rank0 : KP;
    float ubs = kInf;
    int ubj = -1;
    if constexpr (RANK) {
      if (rank0 > 0 && keep[0]) {
        const int64_t r = (qrow[0] * H + t.h) * topk + rank0 - 1;
        ubs = out_score[r];
        ubj = out_idx[r];
        if (ubj < 0) ubs = -kInf;           // the row has no keys past rank0 - 1
      }
    }
    // Lists: slots [0, KP-kk) hold +inf sentinels that nothing displaces, so
    // the live top-kk occupies the tail and its kk-th score is ls[.][KP-1].
    const int nsent = KP - kk;
    float ls[QB][KP];
    int lj[QB][KP];
#pragma unroll
    for (int b = 0; b < QB; ++b)
#pragma unroll
      for (int i = 0; i < KP; ++i) {
        ls[b][i] = i < nsent ? kInf : -kInf;
        lj[b][i] = -1;
      }
    float thr[QB], cm[QB];
#pragma unroll
    for (int b = 0; b < QB; ++b) {
      cm[b] = -kInf;
      thr[b] = kInf;
      if constexpr (!PRE) {
        if (qvalid[b]) thr[b] = next_down(thr_buf[qrow[b] * H + t.h]);
      }
    }
    // Q operands and thresholds have arrived before the first key load is
    // issued, so the chunk loop waits on key loads only.
    __builtin_amdgcn_s_waitcnt(0x0f70);
#pragma unroll
    for (int j = 0; j < S::NBUF - 1; ++j)
      if (j < nproc) issue(t, j * sample, j, wave, lane);

    // Scored sub-blocks: all of the first nproc - 1 scored chunks, plus the
    // part of the last one that holds keys.
    const int last_keys = (int)(nkeys - (int64_t)(nproc - 1) * sample * S::TK);
    const int nsub = (nproc - 1) * S::SUBT + ((last_keys < S::TK ? last_keys : S::TK) + 31) / 32;
    // Key ranges per lane half: a query's bound is the k-th largest of
    // 2 * NCH range maxima, so long lists need proportionally more ranges.
    constexpr int NCH = KP <= 16 ? SCAN_CHUNKS : 4 * KP;
    const int spc = (nsub + NCH - 1) / NCH;                   // sub-blocks per range
    int cleft = spc;                                          // sub-blocks left in chunk
    int cnt = 0;
    uint2* cb = cbuf + wave * CBW + lane;                     // entry c at cb[c * 64]
    // COLLECT: candidates of row r, this lane's half, go to
    // cand[(lhalf * cap + n) * NH + r] for n < cap; ccnt keeps counting past
    // cap so that overflow is visible.
    const int64_t NH = N * H;
    int ccnt[QB];
    int64_t crow[QB];
#pragma unroll
    for (int b = 0; b < QB; ++b) {
      ccnt[b] = 0;
      crow[b] = qrow[b] * H + t.h;
    }

    auto drain = [&]() __attribute__((always_inline)) {
      for (int c = 0; __ballot(c < cnt) != 0ull; ++c) {
        if (c < cnt) {
          const uint2 e = cb[c * 64];
          const float sv = __uint_as_float(e.x);
          const int key = (int)(e.y & 0x7fffffffu);
          const int tag = (int)(e.y >> 31);
#pragma unroll
          for (int b = 0; b < QB; ++b) {
            if constexpr (RANK) {
              if (tag == b && sv > thr[b] && (sv < ubs || (sv == ubs && key > ubj))) {
                list_insert<KP>(ls[b], lj[b], sv, key);
                thr[b] = fmaxf(thr[b], ls[b][KP - 1]);
              }
            } else if constexpr (SEL) {
              if (tag == b && sv > thr[b]) {
                list_insert<KP>(ls[b], lj[b], sv, key);
                thr[b] = fmaxf(thr[b], ls[b][KP - 1]);
              }
            }
          }
        }
      }
      cnt = 0;
    };

    for (int j = 0; j < nproc; ++j) {
      const int c = j * sample;
      // Chunk c's loads (LPW instructions per wavefront) were followed by
      // those of at most NBUF - 2 later chunks.
      if constexpr (S::NBUF == 3) {
        static_assert(S::LPW <= 15, "vmcnt field");
        if (j + 1 < nproc) __builtin_amdgcn_s_waitcnt(0x0f70 | S::LPW);
        else __builtin_amdgcn_s_waitcnt(0x0f70);
      } else {
        __builtin_amdgcn_s_waitcnt(0x0f70);
      }
      __syncthreads();
      if (j + S::NBUF - 1 < nproc)
        issue(t, (j + S::NBUF - 1) * sample, (j + S::NBUF - 1) % S::NBUF, wave, lane);
      if (!wave_active) continue;
      const unsigned char* kc = kbuf + (j % S::NBUF) * S::CHUNK_BYTES;
      const int crel = c * S::TK;                 // first key of the chunk, graph-relative
      const int nk = (int)nkeys;
      const bool partial = crel + S::TK > nk;

      // Sub-blocks are processed in batches of BS: all LDS reads of the
      // batch, then all its MFMAs (independent accumulation chains), then the
      // scores, so a wavefront keeps several MFMAs in flight.
      constexpr int BS = PassCfg<MODE>::BATCH < S::SUBT ? PassCfg<MODE>::BATCH : S::SUBT;
      static_assert(S::SUBT % BS == 0, "batches tile the chunk");
      floatx16_t acc[BS][QB];
      bf16x8_t areg[BS][S::NM];
      auto aload = [&](int st, int slot) __attribute__((always_inline)) {
#pragma unroll
        for (int m = 0; m < S::NM; ++m)
          areg[slot][m] =
              *reinterpret_cast<const bf16x8_t*>(kc + (st * S::NM + m) * 1024 + aoff);
      };
      auto mfma = [&](int slot_a, int slot) __attribute__((always_inline)) {
#pragma unroll
        for (int b = 0; b < QB; ++b) acc[slot][b] = floatx16_t{};
#pragma unroll
        for (int m = 0; m < S::NM; ++m) {
#pragma unroll
          for (int b = 0; b < QB; ++b)
            if (bact[b])
              acc[slot][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                  areg[slot_a][m], qb[b][m], acc[slot][b], 0, 0, 0);
        }
      };
      auto examine = [&](int st, int slot) __attribute__((always_inline)) {
        // acc[r] = <k_key, q_query>, key = key0 + 8*(r/4) + (r%4), query = lane%32.
        const int rel0 = crel + st * 32 + 4 * lhalf;
        const int key0 = (int)t.kb + rel0;
        floatx16_t(&s)[QB] = acc[slot];
        if (partial) {
#pragma unroll
          for (int b = 0; b < QB; ++b)
#pragma unroll
            for (int r = 0; r < 16; ++r)
              if (rel0 + 8 * (r >> 2) + (r & 3) >= nk) s[b][r] = -kInf;
        }
        if constexpr (PRE) {
#pragma unroll
          for (int b = 0; b < QB; ++b)
            cm[b] = fmaxf(fmaxf(fmaxf(fmaxf(s[b][0], s[b][1]), fmaxf(s[b][2], s[b][3])),
                                fmaxf(fmaxf(s[b][4], s[b][5]), fmaxf(s[b][6], s[b][7]))),
                          fmaxf(fmaxf(fmaxf(s[b][8], s[b][9]), fmaxf(s[b][10], s[b][11])),
                                fmaxf(fmaxf(s[b][12], s[b][13]),
                                      fmaxf(fmaxf(s[b][14], s[b][15]), cm[b]))));
          const int ti = j * S::SUBT + st;            // scored sub-block index, uniform
          if (--cleft == 0 || ti + 1 == nsub) {
            cleft = spc;
#pragma unroll
            for (int b = 0; b < QB; ++b) {
              if (cm[b] > ls[b][KP - 1]) value_insert<KP>(ls[b], cm[b]);
              cm[b] = -kInf;
            }
          }
        } else if constexpr (MODE == M_COLLECT) {
          bool hit = false;
#pragma unroll
          for (int b = 0; b < QB; ++b) hit = hit || (block_max(s[b]) > thr[b]);
          if (__ballot(hit) != 0ull) {
#pragma unroll
            for (int b = 0; b < QB; ++b)
#pragma unroll
              for (int qq = 0; qq < 4; ++qq) {
                if (__ballot(quarter_hit(s[b], qq, thr[b])) != 0ull) {
#pragma unroll
                  for (int r = 0; r < 4; ++r) {
                    const float sv = s[b][4 * qq + r];
                    if (sv > thr[b]) {
                      if (ccnt[b] < a.cap)
                        a.cand[(int64_t)(lhalf * a.cap + ccnt[b]) * NH + crow[b]] =
                            make_uint2(__float_as_uint(sv), (unsigned)(key0 + 8 * qq + r));
                      ++ccnt[b];
                    }
                  }
                }
              }
          }
        } else {
          bool hit = false;
#pragma unroll
          for (int b = 0; b < QB; ++b) hit = hit || (block_max(s[b]) > thr[b]);
          if (__ballot(hit) != 0ull) {
            bool g[QB][4];
#pragma unroll
            for (int b = 0; b < QB; ++b)
#pragma unroll
              for (int qq = 0; qq < 4; ++qq) g[b][qq] = quarter_hit(s[b], qq, thr[b]);
            // Appends go in halves of two quarters (at most 8 = SCAN_CAP per
            // lane): make room first, so each half has a single drain site.
            // A lane with a hit in a quarter writes all four scores, without
            // branches, at its next slot, which only advances on a hit (the
            // room check keeps those slots below SCAN_CAP).
            static_assert(SCAN_CAP >= 8, "a half sub-block appends up to 8 scores");
#pragma unroll
            for (int b = 0; b < QB; ++b)
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
              int room = cnt;
#pragma unroll
              for (int qq = 2 * hf; qq < 2 * hf + 2; ++qq) room += g[b][qq] ? 4 : 0;
              if (__ballot(room > SCAN_CAP) != 0ull) drain();
#pragma unroll
              for (int qq = 2 * hf; qq < 2 * hf + 2; ++qq) {
                if (g[b][qq]) {
#pragma unroll
                  for (int r = 0; r < 4; ++r) {
                    const float sv = s[b][4 * qq + r];
                    cb[cnt * 64] = make_uint2(__float_as_uint(sv),
                                              (unsigned)(key0 + 8 * qq + r) | ((unsigned)b << 31));
                    cnt += sv > thr[b] ? 1 : 0;
                  }
                }
              }
            }
          }
        }
      };
#pragma unroll
      for (int st0 = 0; st0 < S::SUBT; st0 += BS) {
        if (crel + st0 * 32 >= nk) break;       // only padding left in a last chunk
#pragma unroll
        for (int i = 0; i < BS; ++i) aload(st0 + i, i);
#pragma unroll
        for (int i = 0; i < BS; ++i) mfma(i, i);
#pragma unroll
        for (int i = 0; i < BS; ++i) examine(st0 + i, i);
      }
    }
    if (!wave_active) return;

    if constexpr (PRE) {
      // k-th largest chunk maximum over both halves of each query.
#pragma unroll
      for (int b = 0; b < QB; ++b) {
        float ps[KP];
#pragma unroll
        for (int i = 0; i < KP; ++i) ps[i] = __shfl_xor(ls[b][i], 32);
#pragma unroll
        for (int i = 0; i < KP; ++i)
          if (i >= nsent && ps[i] > ls[b][KP - 1]) value_insert<KP>(ls[b], ps[i]);
        if (qvalid[b] && lhalf == 0) thr_buf[qrow[b] * H + t.h] = ls[b][KP - 1];
      }
    } else if constexpr (MODE == M_COLLECT) {
#pragma unroll
      for (int b = 0; b < QB; ++b)
        if (qvalid[b]) a.cand_cnt[2 * crow[b] + lhalf] = ccnt[b];
    } else {
      drain();
      const bool lower = lhalf == 0;
      static_assert(KP <= 16 && QB == 1 && SCAN_CAP * 64 >= 32 * 16,
                    "register lists; 32 rows of 16 entries per region");
      // Two-pointer merge of the half-lists of each query (lanes l, l ^ 32)
      // under (score descending, id ascending): the upper lane publishes its
      // live entries, best first, in the drained candidate buffer; the lower
      // lane walks them beside its own list and writes the top-kk in order,
      // at ranks rank0, rank0 + 1, ...  Only padding entries (-inf, -1) can
      // tie exactly; the lower lane's go first.
      uint2* wl = cbuf + wave * CBW;
      if (!lower) {
#pragma unroll
        for (int i = 0; i < KP; ++i)
          if (i >= nsent)
            wl[lrow * 16 + (i - nsent)] =
                make_uint2(__float_as_uint(ls[0][i]), (unsigned)lj[0][i]);
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      if (lower && keep[0]) {
        int32_t* oi = out_idx + (qrow[0] * H + t.h) * topk + rank0;
        float* os = out_score + (qrow[0] * H + t.h) * topk + rank0;
        const uint2* pl = wl + lrow * 16;
        int u = 0, r = 0;
        uint2 pu = pl[0];
        auto emit = [&](float sv, int j) __attribute__((always_inline)) {
          const float sc = j < 0 ? -kInf : sv;
          oi[r] = j;
          os[r] = sc;
          ++r;
        };
#pragma unroll
        for (int i = 0; i < KP; ++i) {
          if (i >= nsent) {
            const float sv = ls[0][i];
            const int j = lj[0][i];
            while (r < kk && u < kk &&
                   (__uint_as_float(pu.x) > sv ||
                    (__uint_as_float(pu.x) == sv && (int)pu.y < j))) {
              emit(__uint_as_float(pu.x), (int)pu.y);
              ++u;
              pu = pl[u < 16 ? u : 15];
            }
            if (r < kk) emit(sv, j);
          }
        }
        while (r < kk) {                      // r < kk implies u < kk
          emit(__uint_as_float(pu.x), (int)pu.y);
          ++u;
          pu = pl[u < 16 ? u : 15];
        }
      }
    }
  }
};

// Persistent grid for one graph: nwg workgroups split the H * nbph query
// blocks (32 rows each) into equal contiguous ranges.  Batched graphs: one
// workgroup per (planned tile, head).
// W wavefronts per workgroup; short lists keep 128 VGPRs (four wavefronts
// per SIMD: one 16-wavefront or two 8-wavefront workgroups per CU).
template <int D, int KP, int MODE, int W>
__global__ __attribute__((amdgpu_flat_work_group_size(1, W * 64),
                          amdgpu_waves_per_eu(KP <= 16 ? 4 : 2)))
void score_topk_kernel(ScanArgs a, int nwg) {
  const int64_t N = a.N;
  const int H = a.H;
  const int2* tiles = a.tiles;
  const int32_t* offsets = a.offsets;
  constexpr int SUB_ROWS = W * QB * 32;
  using S = ScanShape<D, MODE, W>;
  // One LDS block: the key ring, then (SELECT) the candidate buffers.
  constexpr int KB = S::NBUF * S::CHUNK_BYTES;
  constexpr int CB = Scanner<D, KP, MODE, W>::SEL ? W * Scanner<D, KP, MODE, W>::CBW * 8 : 0;
  __shared__ __attribute__((aligned(1024))) unsigned char kbuf[KB + CB];
  uint2* cbuf = reinterpret_cast<uint2*>(kbuf + KB);
  const unsigned kbuf_lds =
      (unsigned)(uintptr_t)(__attribute__((address_space(3))) unsigned char*)kbuf;
  Scanner<D, KP, MODE, W> sc{kbuf,   kbuf_lds, cbuf,   a,      a.q,   a.k,
                             a.perm, a.N,      a.H,    a.topk, a.thr, a.idx, a.score};
  // Query blocks [b, be) of the flattened (head, 32-row block) space for one
  // graph; a single planned sub-tile for batched graphs.
  const int64_t nbph = (N + 31) / 32;
  int64_t b = 0, be = 0;
  int rh = 0;
  int64_t rq0 = 0, rq1 = 0, rkb = 0, rke = 0;
  if (tiles == nullptr) {
    // Logical id: the 8 XCDs receive workgroups round-robin; give each XCD a
    // contiguous range so its workgroups share a head (and its keys in L2).
    const int per = nwg / 8;
    const int L = (int)(blockIdx.x % 8) * per + (int)(blockIdx.x / 8);
    const int64_t total = nbph * H;
    b = total * L / nwg;
    be = total * (L + 1) / nwg;
  } else {
    const int2 tl = tiles[blockIdx.x / H];
    if (tl.x < 0) return;                 // beyond the planned tiles
    rh = (int)(blockIdx.x % H);
    rkb = offsets[tl.x];
    rke = offsets[tl.x + 1];
    if (tl.y >= rke) return;
    rq0 = tl.y;
    rq1 = tl.y + SUB_ROWS < rke ? tl.y + SUB_ROWS : rke;
    be = 1;
  }
  while (b < be) {
    SubTile st;
    if (tiles == nullptr) {
      // Spread the remaining blocks evenly over the sub-tiles still needed.
      const int h = (int)(b / nbph);
      const int64_t nb0 = b % nbph;
      const int64_t rem = be - b;
      const int64_t nst = (rem + W * QB - 1) / (W * QB);
      int64_t n = (rem + nst - 1) / nst;
      n = n < nbph - nb0 ? n : nbph - nb0;
      st = SubTile{h, nb0 * 32, (nb0 + n) * 32 < N ? (nb0 + n) * 32 : N, 0, N};
      b += n;
    } else {
      st = SubTile{rh, rq0, rq1, rkb, rke};
      b = be;
    }
    sc.run(st);
  }
}

// Co-resident workgroups of a kernel on this device (one graph: the
// persistent grid size, a multiple of 8 so each XCD gets an equal share).
template <typename Kern>
int resident_workgroups(Kern kern, int threads) {
  int dev = 0, cus = 0, per_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void*>(kern),
                                                   threads, 0) != hipSuccess)
    return 0;
  const int n = cus * (per_cu > 0 ? per_cu : 1);
  return n >= 8 ? n - n % 8 : 8;
}

template <int D, int KP, int MODE>
hipError_t launch_pass(const ScanArgs& a, hipStream_t s) {
  if (a.tiles == nullptr) {
    constexpr int W = scan_waves(KP, false);
    auto kern = score_topk_kernel<D, KP, MODE, W>;
    const int nwg = resident_workgroups(kern, W * 64);
    if (nwg <= 0) return hipErrorInvalidDevice;
    hipLaunchKernelGGL(kern, dim3((unsigned)nwg), dim3(W * 64), 0, s, a, nwg);
  } else {
    constexpr int W = scan_waves(KP, true);
    hipLaunchKernelGGL((score_topk_kernel<D, KP, MODE, W>), dim3((unsigned)(a.max_tiles * a.H)),
                       dim3(W * 64), 0, s, a, 0);
  }
  return hipGetLastError();
}

// Insert (s, j) into a descending list under (score descending, id
// ascending); candidates may come in any order.
template <int KP>
__device__ __forceinline__ void ordered_insert(float (&ls)[KP], int (&lj)[KP], float s, int j) {
  bool b[KP];
#pragma unroll
  for (int t = 0; t < KP; ++t) b[t] = s > ls[t] || (s == ls[t] && (unsigned)j < (unsigned)lj[t]);
#pragma unroll
  for (int t = KP - 1; t >= 1; --t) {
    ls[t] = b[t - 1] ? ls[t - 1] : (b[t] ? s : ls[t]);
    lj[t] = b[t - 1] ? lj[t - 1] : (b[t] ? j : lj[t]);
  }
  ls[0] = b[0] ? s : ls[0];
  lj[0] = b[0] ? j : lj[0];
}

// Top-k of each row's collected candidates, one thread per row.  Rows whose
// arrays overflowed are left to the SELECT pass.  Empty slots hold (-inf, -1)
// and rank after every candidate ((unsigned)-1 is the largest id); +inf
// sentinels fill slots [0, KP - topk).
template <int KP>
__global__ __launch_bounds__(256) void collect_topk_kernel(ScanArgs a) {
  const int64_t NH = a.N * a.H;
  const int64_t r = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (r >= NH) return;
  const int c0 = a.cand_cnt[2 * r], c1 = a.cand_cnt[2 * r + 1];
  if (c0 > a.cap || c1 > a.cap) return;
  const int nsent = KP - a.topk;
  float ls[KP];
  int lj[KP];
#pragma unroll
  for (int i = 0; i < KP; ++i) {
    ls[i] = i < nsent ? kInf : -kInf;
    lj[i] = -1;
  }
  // Candidates are read eight at a time, so that eight loads are in flight
  // before the first insertion waits for its entry.  (Slower, at N = 10^5,
  // k = 45: a first pass finding the k-th score with value lists, so that
  // only the kept candidates and their ties are inserted, 1.36 against
  // 1.16 ms, the candidates being read twice; two lanes per row, one per
  // lane half's array, merged through LDS, 1.35 ms, each half list
  // inserting more of its candidates.)
  constexpr int PF = 8;
  for (int hf = 0; hf < 2; ++hf) {
    const int n = hf ? c1 : c0;
    const uint2* src = a.cand + (int64_t)hf * a.cap * NH + r;
    for (int u0 = 0; u0 < n; u0 += PF) {
      uint2 e[PF];
#pragma unroll
      for (int i = 0; i < PF; ++i)
        e[i] = u0 + i < n ? src[(int64_t)(u0 + i) * NH] : make_uint2(__float_as_uint(-kInf), ~0u);
#pragma unroll
      for (int i = 0; i < PF; ++i) {
        const float sv = __uint_as_float(e[i].x);
        const int j = (int)e[i].y;
        if (u0 + i < n &&
            (sv > ls[KP - 1] || (sv == ls[KP - 1] && (unsigned)j < (unsigned)lj[KP - 1])))
          ordered_insert<KP>(ls, lj, sv, j);
      }
    }
  }
  int32_t* oi = a.idx + r * a.topk;
  float* os = a.score + r * a.topk;
#pragma unroll
  for (int i = 0; i < KP; ++i) {
    if (i >= nsent) {
      oi[i - nsent] = lj[i];
      os[i - nsent] = lj[i] < 0 ? -kInf : ls[i];
    }
  }
}

// Window bound (one graph, with a query order).  Each workgroup takes WIN_ROWS
// consecutive positions [q0, q1) of one head's query order and scores its
// queries against the keys of the positions [q0 - WIN_HALF, q1 + WIN_HALF)
// (cut to a multiple of 32 keys): the nodes grouped next to them, which for
// inputs with cluster structure hold most of each query's best keys.  The
// window's keys are dealt round-robin over its NB 32-key sub-blocks (window
// key w goes to sub-block w % NB, row w / NB), so every sub-block samples the
// whole window.  Per lane, the maximum of each sub-block's 16 scores enters a
// top-k value list; these are scores of distinct keys, so the k-th largest
// over both lane halves is a lower bound of the query's k-th score, and the
// row's threshold becomes the larger of it and the sampled bound already
// there.  Keys are gathered into LDS in MFMA operand order with plain loads,
// one chunk of sub-blocks at a time.
constexpr int WIN_WAVES = 8;
constexpr int WIN_ROWS = WIN_WAVES * 32;
constexpr int WIN_HALF = 1024;
constexpr int WIN_CHUNK_BYTES = 16384;   // 16 KB: 106 against 112 us at 32 KB (more workgroups per CU)

template <int D, int KP>
__global__ __launch_bounds__(WIN_WAVES * 64) void window_thresh_kernel(ScanArgs a) {
  constexpr int NM = D / 16;
  constexpr int TK = WIN_CHUNK_BYTES / (2 * D) / 32 * 32;   // keys per chunk
  constexpr int SUBT = TK / 32;
  constexpr int MAXW = WIN_ROWS + 2 * WIN_HALF;
  __shared__ __attribute__((aligned(1024))) unsigned char kbuf[SUBT * NM * 1024];
  __shared__ int32_t ids[MAXW];
  const int64_t N = a.N;
  const int H = a.H;
  const int h = blockIdx.y;
  const int64_t q0 = (int64_t)blockIdx.x * WIN_ROWS;
  if (q0 >= N) return;                          // uniform over the workgroup
  const int64_t q1 = q0 + WIN_ROWS < N ? q0 + WIN_ROWS : N;
  const int64_t w0 = q0 > WIN_HALF ? q0 - WIN_HALF : 0;
  const int64_t w1 = q1 + WIN_HALF < N ? q1 + WIN_HALF : N;
  const int NB = (int)((w1 - w0) / 32);          // sub-blocks; the window is nw = 32 NB keys
  if (NB == 0) return;
  const int nw = NB * 32;
  const int32_t* perm = a.perm + (int64_t)h * N;
  for (int t = threadIdx.x; t < nw; t += blockDim.x) ids[t] = perm[w0 + t];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lrow = lane & 31, lhalf = lane >> 5;
  const bool wave_active = q0 + wave * 32 < q1;
  const int64_t pos = q0 + wave * 32 + lrow;
  const bool qvalid = pos < q1;
  const int64_t qrow = perm[qvalid ? pos : q1 - 1];
  bf16x8_t qb[NM];
  const uint16_t* qp = a.q + (qrow * H + h) * D + 8 * lhalf;
#pragma unroll
  for (int m = 0; m < NM; ++m) qb[m] = *reinterpret_cast<const bf16x8_t*>(qp + 16 * m);
  const int nsent = KP - a.topk;
  float ls[KP];
#pragma unroll
  for (int i = 0; i < KP; ++i) ls[i] = i < nsent ? kInf : -kInf;
  __syncthreads();                              // ids are in LDS

  for (int b0 = 0; b0 < NB; b0 += SUBT) {
    const int nsb = NB - b0 < SUBT ? NB - b0 : SUBT;
    // Piece t: lane t % 64 of operand block t / 64 (sub-block b0 + blk / NM,
    // K-slice blk % NM); row r of sub-block b is window key r * NB + b.
    for (int t = tid; t < nsb * NM * 64; t += WIN_WAVES * 64) {
      const int blk = t >> 6, l = t & 63;
      const int64_t node = ids[(l & 31) * NB + b0 + blk / NM];
      *reinterpret_cast<uint4*>(kbuf + (size_t)t * 16) = *reinterpret_cast<const uint4*>(
          a.k + (node * H + h) * D + 16 * (blk % NM) + 8 * (l >> 5));
    }
    __syncthreads();
    if (wave_active) {
      for (int st = 0; st < nsb; ++st) {
        floatx16_t acc = {};
#pragma unroll
        for (int m = 0; m < NM; ++m)
          acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              *reinterpret_cast<const bf16x8_t*>(kbuf + (st * NM + m) * 1024 + lane * 16), qb[m],
              acc, 0, 0, 0);
        const float mx = block_max(acc);
        if (mx > ls[KP - 1]) value_insert<KP>(ls, mx);
      }
    }
    __syncthreads();                            // the chunk is read before it is refilled
  }
  if (!wave_active) return;
  float ps[KP];
#pragma unroll
  for (int i = 0; i < KP; ++i) ps[i] = __shfl_xor(ls[i], 32);
#pragma unroll
  for (int i = 0; i < KP; ++i)
    if (i >= nsent && ps[i] > ls[KP - 1]) value_insert<KP>(ls, ps[i]);
  if (qvalid && lhalf == 0) {
    float* t = a.thr + qrow * H + h;
    *t = fmaxf(*t, ls[KP - 1]);
  }
}

#include "kmip_prune.h"

template <int D, int KP>
hipError_t launch_scan_t(const ScanArgs& a, hipStream_t s) {
  hipError_t e = launch_pass<D, KP, M_THRESH>(a, s);
  if (e != hipSuccess) return e;
  if (a.perm != nullptr) {
    hipLaunchKernelGGL((window_thresh_kernel<D, KP>),
                       dim3((unsigned)ceil_div(a.N, WIN_ROWS), (unsigned)a.H),
                       dim3(WIN_WAVES * 64), 0, s, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if constexpr (KP > 16) {
    // Long lists: collect candidates (the pruned pass for the ranges it
    // keeps, the streaming pass for the rest), select from them, then
    // recompute the rows whose candidate arrays overflowed (that pass
    // usually only checks the counts).
    ScanArgs c = a;
    c.range_stream = nullptr;
    if constexpr (D == 32 || D == 64 || D == 96) {
      if (a.kop != nullptr) {
        e = launch_prune<D, 16, true>(a, s);
        if (e != hipSuccess) return e;
        c.range_stream = a.range_stream;
      }
    }
    e = launch_pass<D, KP, M_COLLECT>(c, s);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(collect_topk_kernel<KP>, dim3((unsigned)ceil_div(a.N * a.H, 256)),
                       dim3(256), 0, s, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    // Rows whose arrays overflowed: exact selection with 16-entry register
    // lists, 16 ranks per pass, each pass keeping the keys ordered after the
    // previous pass's last entry.
    for (int r0 = 0; r0 < a.topk; r0 += 16) {
      ScanArgs b = a;
      b.rank0 = r0;
      e = launch_pass<D, 16, M_RANK>(b, s);
      if (e != hipSuccess) return e;
    }
    return hipSuccess;
  } else {
    ScanArgs b = a;
    b.cand_cnt = nullptr;
    b.range_stream = nullptr;                  // SELECT writes every row...
    if constexpr (D == 32 || D == 64 || D == 96) {
      if (a.kop != nullptr) {                  // ...but those of the pruned pass
        // short lists run the pruned pass with 8-entry lists (sentinels fill
        // the rest): 5-entry instantiations compile to far more registers
        e = launch_prune<D, (KP < 8 ? 8 : KP)>(a, s);
        if (e != hipSuccess) return e;
        b.range_stream = a.range_stream;
      }
    }
    return launch_pass<D, KP, M_SELECT>(b, s);
  }
}

template <int D>
hipError_t launch_scan_d(int kp, const ScanArgs& a, hipStream_t s) {
  switch (kp) {
    case 5: return launch_scan_t<D, 5>(a, s);
    case 8: return launch_scan_t<D, 8>(a, s);
    case 15: return launch_scan_t<D, 15>(a, s);
    case 16: return launch_scan_t<D, 16>(a, s);
    case 32: return launch_scan_t<D, 32>(a, s);
    case 45: return launch_scan_t<D, 45>(a, s);
    case 48: return launch_scan_t<D, 48>(a, s);
    case 64: return launch_scan_t<D, 64>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace
}  // namespace kmip
