// Pruned selection pass (one graph with a query order; rows of 32 or 64
// bf16; lists of at most 16).  Included by kmip_scan_kernels.h, whose helpers
// (next_down, block_max, quarter_hit, ordered_insert, resident_workgroups) it
// uses.
//
// The exact top-k of a query is decided by the keys that score above the
// lower bound T of its k-th score (the threshold and window passes).  Keys
// are taken in the query order, which groups nodes by their nearest pivot
// query: for inputs with cluster structure the 32 keys of a block of that
// order point the same way, and one bound per (query, block)
//   q . k  <=  q . mid + |q| R             (|k - mid| <= R, Euclidean norms)
// rules most blocks out for a wavefront's 32 queries (which sit next to
// each other in the same order).  A block never straddles two groups (the
// last block of a group is padded with empty slots): a block holding the
// tail of one group and the head of the next has a wide box, and on the
// clustered inputs that padding halves the live blocks.  Kernels:
//
//   group_layout_kernel  per pivot group of the order its size, first
//                      position and first key slot, every group starting a
//                      new 32-key block;
//   key_pack_kernel    keys of each head in query order, per 32-key block in
//                      MFMA operand order, and the block's bound row
//                      [mid | R] (R widened to cover fp32 rounding);
//   bound_live_kernel  per query block of 32 positions, the bound of every
//                      key block under the queries' thresholds: a bit per
//                      key block whose bound reaches one of them;
//   pruned_select_kernel  each wavefront scores only its live key blocks,
//                      loaded straight into registers, with the register
//                      top-k of the streaming pass; keys come out of id
//                      order, so lists insert under (score descending, id
//                      ascending) and a candidate need only reach the
//                      current k-th score.
//
// Query blocks with many live key blocks (inputs without cluster structure)
// stay with the streaming selection pass, which then skips all others.
//
// Exactness.  The score of (q, k) is one fp32 MFMA result; with M the largest
// |k_c| of the block, it differs from q . k by at most 2^-19 |q|_1 M <=
// 2^-19 sqrt(d) |q| M (32 products, each exact in fp32, at most 32 roundings
// of 2^-24).  The bound is a (d + 1)-term MFMA result, within 2^-17.4
// sqrt(d) |q| M of its exact value (|mid_c| <= M, the norm and R rounded up
// to bf16, R <= 2 sqrt(d) M + pad).  R is widened by pad = 2^-13 sqrt(d) M,
// which adds 2^-13 sqrt(d) |q| M to the bound: more than both errors, so a
// key whose computed score passes a threshold lies in a block whose computed
// bound passes it too.  (Against a per-element box bound q . mid + |q| . rad,
// this ball bound leaves about a third fewer blocks live on the clustered
// inputs, with d / 16 + 1 operand slices instead of d / 8.)  Split rows: the
// low parts are within 2^-8 of the high parts elementwise, so the 96 exact
// products of a score sum to at most (1 + 2^-7) |q_hi|_1 M and the score is
// within 2^-17.4 sqrt(d) |q_hi| M of q3 . k3; the bound's d + 2 terms (R, L,
// G and both norms rounded up) are within 2^-17 sqrt(d) |q_hi| M; the same
// pad on R, times |q_hi|, covers both.
#pragma once

constexpr int PR_WAVES = 16;              // bound pass: wavefronts per workgroup
constexpr int PS_WAVES = 4;               // pruned selection: wavefronts per workgroup
constexpr float PR_PAD = 0x1p-13f;        // radius widening relative to sqrt(d) max |k|
template <int D> constexpr float PR_SQRT_D = D == 32 ? 5.6569f : D == 64 ? 8.0f : 9.7980f;  // >= sqrt(D)
constexpr int PR_MAX_WORDS = PRUNE_MAX_WORDS;  // live words per query block
constexpr int PR_LPW = 2;                 // bound pass: operand pieces per wavefront per batch
constexpr int PR_NBUF = 3;                // bound pass: ring slots
// Pruned selection: key blocks in flight per wavefront.  Two, so that four
// workgroups (16 wavefronts) share a CU's LDS at rows of 32: at the bench
// workload 1.63 ms for kmip_score_topk against 1.75 ms with four blocks in
// flight (three workgroups per CU) and 1.73 ms with three.
constexpr int PS_NPF = 2;
// Split-precision rows (D = 96: q3 = [q_hi | q_hi | q_lo], k3 = [k_hi | k_lo |
// k_hi] of d = 32 elements each) are bounded through their high parts:
//   q3 . k3 = q_hi . k_hi + q_hi . k_lo + q_lo . k_hi
//          <= q_hi . mid + |q_hi| (R + L) + |q_lo| G
// with mid, R the centre and radius of the block's k_hi, L and G the largest
// |k_lo| and |k_hi|.  Bound dimensions and bound-row slices per row width:
template <int D> constexpr int PR_DB = D == 96 ? 32 : D;
template <int D> constexpr int PR_NB = PR_DB<D> / 16 + 1;
constexpr int PR_HEAVY = 512;             // live key blocks above which a query block is heavy
constexpr int PH_PARTS = PRUNE_HEAVY_PARTS;  // wavefronts sharing a heavy query block

// bf16 bits <-> float.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
// Smallest bf16 value >= x (x >= 0, finite).
__device__ __forceinline__ uint32_t bf16_bits_up(float x) {
  const uint32_t u = __float_as_uint(x);
  const uint32_t t = u & 0xffff0000u;
  return (t == u ? t : t + 0x10000u) >> 16;
}

// Per head (one workgroup): each group's size (the sum of its copies'
// counts), first position in the head's order (exclusive scan of the sizes)
// and first padded key slot (exclusive scan of the sizes rounded up to 32),
// then the group of every padded key block (-1 past the head's last).
constexpr int GL_THREADS = 1024;
__global__ __launch_bounds__(GL_THREADS) void group_layout_kernel(ScanArgs a) {
  __shared__ int s0[GL_THREADS], s1[GL_THREADS];
  const int h = blockIdx.x, t = threadIdx.x;
  const int npiv = a.npiv;
  const int per = (npiv + GL_THREADS - 1) / GL_THREADS;
  const int r0 = t * per < npiv ? t * per : npiv;
  const int r1 = r0 + per < npiv ? r0 + per : npiv;
  const int32_t* cnt = a.order_counts + (int64_t)h * npiv * ORDER_COPIES;
  auto gsz = [&](int r) __attribute__((always_inline)) {
    int n = 0;
#pragma unroll
    for (int c = 0; c < ORDER_COPIES; ++c) n += cnt[r * ORDER_COPIES + c];
    return n;
  };
  int sz = 0, pz = 0;
  for (int r = r0; r < r1; ++r) {
    const int n = gsz(r);
    sz += n;
    pz += (n + 31) & ~31;
  }
  s0[t] = sz;
  s1[t] = pz;
  __syncthreads();
  for (int o = 1; o < GL_THREADS; o <<= 1) {       // inclusive scans
    const int x0 = t >= o ? s0[t - o] : 0, x1 = t >= o ? s1[t - o] : 0;
    __syncthreads();
    s0[t] += x0;
    s1[t] += x1;
    __syncthreads();
  }
  int g = s0[t] - sz, p = s1[t] - pz;
  const int64_t gb = (int64_t)h * npiv;
  int32_t* bg = a.bgroup + (int64_t)h * a.nkp;
  for (int r = r0; r < r1; ++r) {
    const int n = gsz(r);
    a.gstart[gb + r] = g;
    a.gsize[gb + r] = n;
    a.pstart[gb + r] = p;
    const int pn = (n + 31) & ~31;
    for (int b = p >> 5; b < (p + pn) >> 5; ++b) bg[b] = r;
    g += n;
    p += pn;
  }
  const int nkph = s1[GL_THREADS - 1] >> 5;
  if (t == 0) a.nkp_h[h] = nkph;
  for (int64_t b = nkph + t; b < a.nkp; b += GL_THREADS) bg[b] = -1;
}

// One wavefront per padded key block b of head blockIdx.y (blocks past the
// head's last, up to the group multiple, get zero bound rows).  Lane l holds
// slot l % 32 of the block (position pstart + 32 b + l % 32 - pstart[r] of
// the order, r the block's group, while inside the group; an empty slot
// otherwise) and, for K-slice m, its elements 8 (2m + l / 32) .. + 7:
// exactly the A operand lane l supplies for that slice.
//   kop[((h nkp + b) NM + m) 512 + 8 l + e]
//   kid[(h nkp + b) 32 + l]                           for l < 32
//   bop[((h ngr + g) (NM + 1) + m') 512 + 8 (r + 32 s) + e]   for block 32 g + r:
//       slices m' < NM hold mid, element 16 m' + 8 s + e; slice NM holds R
//       in element 0 and zeros.
template <int D>
__global__ __launch_bounds__(256) void key_pack_kernel(ScanArgs a) {
  constexpr int NM = D / 16;
  const int lane = threadIdx.x & 63, lrow = lane & 31, lhalf = lane >> 5;
  const int h = blockIdx.y;
  if (blockIdx.x == 0 && h == 0)
    for (int64_t r = threadIdx.x; r < a.nrange; r += 256) a.range_cnt[r] = a.heavy_cnt[r] = 0;
  const int64_t b = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (b >= a.ngr * 32) return;
  const int64_t N = a.N;
  const int H = a.H;
  const int64_t g = b / 32;
  const int br = (int)(b % 32);
  constexpr int NMD = PR_DB<D> / 16;                  // slices of bounded dimensions
  uint16_t* bo = a.bop + (((int64_t)h * a.ngr + g) * PR_NB<D>) * 512 + (br + 32 * lhalf) * 8;
  const int r = b < a.nkp ? a.bgroup[(int64_t)h * a.nkp + b] : -1;
  if (r < 0) {
    if (lrow == 0) {
#pragma unroll
      for (int m = 0; m < PR_NB<D>; ++m) *reinterpret_cast<uint4*>(bo + m * 512) = uint4{0, 0, 0, 0};
    }
    return;
  }
  const int64_t gr = (int64_t)h * a.npiv + r;
  const int o = (int)(b * 32 + lrow) - a.pstart[gr];
  const bool valid = o < a.gsize[gr];
  const int64_t pos = a.gstart[gr] + (valid ? o : 0);
  const int64_t node = a.perm[(int64_t)h * N + pos];
  if (lhalf == 0) a.kid[((int64_t)h * a.nkp + b) * 32 + lrow] = valid ? (int32_t)node : -1;
  const uint16_t* src = a.k + (node * H + h) * D + 8 * lhalf;
  uint4 v[NM];
#pragma unroll
  for (int m = 0; m < NM; ++m)
    v[m] = valid ? *reinterpret_cast<const uint4*>(src + 16 * m) : uint4{0, 0, 0, 0};
  uint16_t* ko = a.kop + (((int64_t)h * a.nkp + b) * NM) * 512 + lane * 8;
#pragma unroll
  for (int m = 0; m < NM; ++m) *reinterpret_cast<uint4*>(ko + m * 512) = v[m];

  // Bounded elements: the whole row, or for split rows the high part
  // (slices 0 .. NMD - 1); M (amax) over those elements.
  float hi[8 * NMD], lo[8 * NMD], xs[8 * NMD];
  float amax = 0.f, lo2 = 0.f, hi2 = 0.f;
#pragma unroll
  for (int m = 0; m < NM; ++m) {
    const uint32_t w[4] = {v[m].x, v[m].y, v[m].z, v[m].w};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float x = (e & 1) ? bf16_hi(w[e >> 1]) : bf16_lo(w[e >> 1]);
      if (m < NMD) {
        xs[8 * m + e] = x;
        hi[8 * m + e] = valid ? x : -kInf;
        lo[8 * m + e] = valid ? x : kInf;
        amax = fmaxf(amax, valid ? fabsf(x) : 0.f);
        hi2 = fmaf(x, x, hi2);
      } else if (m < 2 * NMD) {
        lo2 = fmaf(x, x, lo2);                 // split rows: k_lo
      }
    }
  }
  // over the 32 rows of this lane's half, then M over the whole block
#pragma unroll
  for (int o = 1; o < 32; o <<= 1) {
#pragma unroll
    for (int c = 0; c < 8 * NMD; ++c) {
      hi[c] = fmaxf(hi[c], __shfl_xor(hi[c], o));
      lo[c] = fminf(lo[c], __shfl_xor(lo[c], o));
    }
  }
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) amax = fmaxf(amax, __shfl_xor(amax, o));
  // The centre: the middle of each element's range, truncated to bf16 (any
  // centre will do; the radius is measured from the rounded one).  The
  // radius: the largest distance of a row to it, over the rows of the block.
  float d2 = 0.f;
  uint32_t mb[8 * NMD];
#pragma unroll
  for (int c = 0; c < 8 * NMD; ++c) {
    const float mid = __uint_as_float(__float_as_uint(0.5f * hi[c] + 0.5f * lo[c]) & 0xffff0000u);
    mb[c] = __float_as_uint(mid) >> 16;
    const float t = valid ? xs[c] - mid : 0.f;
    d2 = fmaf(t, t, d2);
  }
  d2 += __shfl_xor(d2, 32);
  lo2 += __shfl_xor(lo2, 32);                  // (empty slots hold zero rows)
  hi2 += __shfl_xor(hi2, 32);
#pragma unroll
  for (int o = 1; o < 32; o <<= 1) {
    d2 = fmaxf(d2, __shfl_xor(d2, o));
    lo2 = fmaxf(lo2, __shfl_xor(lo2, o));
    hi2 = fmaxf(hi2, __shfl_xor(hi2, o));
  }
  if (lrow == 0) {
    // R >= every row's distance (the fp32 sum and root are within 2^-19 of
    // it, relative), plus the pad that covers the scores' rounding; split
    // rows add L = max |k_lo| to it and G = max |k_hi| (both rounded up).
    const float up = 1.f + 0x1p-16f;
    float R = sqrtf(d2) * up + PR_PAD * PR_SQRT_D<PR_DB<D>> * amax;
    uint32_t gbits = 0u;
    if constexpr (D == 96) {
      R += sqrtf(lo2) * up;
      gbits = bf16_bits_up(sqrtf(hi2) * up);
    }
#pragma unroll
    for (int m = 0; m < NMD; ++m) {
      uint32_t wm[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) wm[i] = mb[8 * m + 2 * i] | (mb[8 * m + 2 * i + 1] << 16);
      *reinterpret_cast<uint4*>(bo + m * 512) = uint4{wm[0], wm[1], wm[2], wm[3]};
    }
    *reinterpret_cast<uint4*>(bo + NMD * 512) =
        uint4{lhalf == 0 ? (bf16_bits_up(R) | (gbits << 16)) : 0u, 0u, 0u, 0u};
  }
}

// Bound pass over the query blocks [wid0, wid1) (wid = h * nkb + block).
// Persistent grid of nwg workgroups of PR_WAVES wavefronts; a sub-tile is up
// to PR_WAVES consecutive query blocks of one head, wavefront w taking block
// w.  The head's bound rows stream through a PR_NBUF-slot LDS ring, GPB
// groups of 32 key blocks per slot (PR_LPW 1 KB operand pieces per
// wavefront), two slots ahead.  Each wavefront scores its 32 queries, as
// [q | |q| e0], against 32 bound rows per MFMA chain (queries as the A operand,
// so that a lane's 16 results belong to one key block); a key block is live
// if its bound exceeds next_down(T) of one of the queries.  The live words
// gather in LDS and go out after the sub-tile: live[(wid - wid0) ngr + g]
// (bit r: key block 32 g + r), qb_cnt[wid], the range's total in
// range_cnt, and the heavy query blocks (more than PR_HEAVY live key blocks)
// in heavy_list / heavy_cnt.
template <int D>
__global__ __launch_bounds__(PR_WAVES * 64) void bound_live_kernel(ScanArgs a, int nwg) {
  constexpr int NMD = PR_DB<D> / 16, NMB = PR_NB<D>;
  constexpr int PIECES = PR_WAVES * PR_LPW;
  constexpr int GPB = PIECES / NMB / 2 * 2;            // groups per slot (even)
  constexpr int SLOT = PIECES * 1024;
  static_assert(GPB >= 2, "two groups per slot at least");
  __shared__ __attribute__((aligned(1024))) unsigned char ring[PR_NBUF * SLOT];
  __shared__ uint32_t wsh[PR_WAVES * PR_MAX_WORDS];
  const unsigned ring_lds =
      (unsigned)(uintptr_t)(__attribute__((address_space(3))) unsigned char*)ring;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lrow = lane & 31, lhalf = lane >> 5;
  const int64_t N = a.N;
  const int H = a.H;
  const int64_t nkb = a.nkb, ngr = a.ngr;
  const int nbatch = (int)((ngr + GPB - 1) / GPB);
  const int per = nwg / 8;
  const int L = (int)(blockIdx.x % 8) * per + (int)(blockIdx.x / 8);
  const int64_t total = a.wid1 - a.wid0;
  int64_t b = a.wid0 + total * L / nwg;
  const int64_t be = a.wid0 + total * (L + 1) / nwg;
  uint32_t* ws = wsh + wave * PR_MAX_WORDS;

  // Batch ib into ring slot `slot`: piece p = wave + i * PR_WAVES is slice
  // p % NMB of group GPB ib + p / NMB (past the last group, or past the
  // batch's GPB NMB pieces: the last piece again, never read), so every
  // wavefront always issues PR_LPW loads.
  auto issue = [&](int h, int ib, int slot) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < PR_LPW; ++i) {
      const int p = wave + i * PR_WAVES;
      const int pp = p < GPB * NMB ? p : GPB * NMB - 1;
      int64_t g = (int64_t)ib * GPB + pp / NMB;
      g = g < ngr ? g : ngr - 1;
      const uint16_t* base = a.bop + (((int64_t)h * ngr + g) * NMB + pp % NMB) * 512;
      asm volatile("global_load_lds_dwordx4 %0, %1" ::"v"((unsigned)lane * 16u), "s"(base),
                   "{m0}"(__builtin_amdgcn_readfirstlane(
                       ring_lds + (unsigned)(slot * SLOT + p * 1024)))
                   : "memory");
    }
  };

  while (b < be) {
    const int h = (int)(b / nkb);
    const int64_t nb0 = b % nkb;
    const int64_t rem = be - b;
    const int64_t nst = (rem + PR_WAVES - 1) / PR_WAVES;
    int64_t n = (rem + nst - 1) / nst;
    n = n < nkb - nb0 ? n : nkb - nb0;
    const int64_t wid = b + wave;
    const int64_t nkph = a.nkp_h[h];
    b += n;
    __syncthreads();                        // the previous sub-tile is done with the ring
    const bool active = wave < n;
    const int64_t pos = (nb0 + (active ? wave : 0)) * 32 + lrow;
    const bool qvalid = active && pos < N;
    const int64_t qrow = a.perm[(int64_t)h * N + (pos < N ? pos : N - 1)];
    const uint16_t* qp = a.q + (qrow * H + h) * D + 8 * lhalf;
    // A operand [q | |q| e0]: the row, then its Euclidean norm (rounded up
    // to bf16, the fp32 sum and root being within 2^-19 of it, relative) as
    // element 0 of one more slice, against [mid | R e0] of the key blocks.
    // Split rows: [q_hi | |q_hi| e0 + |q_lo| e1] against [mid | R e0 + G e1].
    bf16x8_t qb[NMB];
    float qq = 0.f, ql = 0.f;
    auto sq = [&](const uint4& w, float& acc) __attribute__((always_inline)) {
      const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float x0 = bf16_lo(ww[i]), x1 = bf16_hi(ww[i]);
        acc = fmaf(x0, x0, acc);
        acc = fmaf(x1, x1, acc);
      }
    };
#pragma unroll
    for (int m = 0; m < NMD; ++m) {
      const uint4 w = *reinterpret_cast<const uint4*>(qp + 16 * m);
      qb[m] = *reinterpret_cast<const bf16x8_t*>(&w);
      sq(w, qq);
      if constexpr (D == 96) sq(*reinterpret_cast<const uint4*>(qp + 16 * (2 * NMD + m)), ql);
    }
    qq += __shfl_xor(qq, 32);
    ql += __shfl_xor(ql, 32);
    {
      const float up = 1.f + 0x1p-16f;
      const uint32_t e01 = bf16_bits_up(sqrtf(qq) * up) |
                           (D == 96 ? bf16_bits_up(sqrtf(ql) * up) << 16 : 0u);
      const uint4 w = {lhalf == 0 ? e01 : 0u, 0u, 0u, 0u};
      qb[NMD] = *reinterpret_cast<const bf16x8_t*>(&w);
    }
    const float thr = qvalid ? next_down(a.thr[qrow * H + h]) : kInf;
    // The MFMA below puts the queries on the rows: lane l then holds key
    // block l % 32 against queries 8 (r / 4) + 4 (l / 32) + r % 4, r < 16,
    // whose thresholds it takes from the lanes that loaded them.
    float tq[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) tq[r] = __shfl(thr, 8 * (r >> 2) + 4 * lhalf + (r & 3));
    // Operands in, and the previous sub-tile's stores done, before the ring
    // loads: from here on the ring loads are this wavefront's only vector
    // memory operations, so the counts below are exact.
    __builtin_amdgcn_s_waitcnt(0x0f70);
    issue(h, 0, 0);
    if (nbatch > 1) issue(h, 1, 1);
    uint32_t wacc = 0u;
    int cnt = 0;
    for (int ib = 0; ib < nbatch; ++ib) {
      if (ib + 1 < nbatch) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(PR_LPW) : "memory");
      else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
      if (ib + 2 < nbatch) issue(h, ib + 2, (ib + 2) % PR_NBUF);
      if (!active) continue;
      const unsigned char* kc = ring + (ib % PR_NBUF) * SLOT;
      // two groups at a time: independent MFMA chains
#pragma unroll
      for (int gg = 0; gg < GPB; gg += 2) {
        const int64_t g = (int64_t)ib * GPB + gg;
        if (g >= ngr) break;
        floatx16_t ab[2] = {};
#pragma unroll
        for (int m = 0; m < NMB; ++m)
#pragma unroll
          for (int u = 0; u < 2; ++u)
            ab[u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                qb[m],
                *reinterpret_cast<const bf16x8_t*>(kc + ((gg + u) * NMB + m) * 1024 + lane * 16),
                ab[u], 0, 0, 0);
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int64_t gu = g + u;
          if (gu >= ngr) break;
          // lane l: key block 32 gu + l % 32; a key block is live if some
          // lane of either half has a query whose bound passes
          uint64_t any = 0ull;
#pragma unroll
          for (int r = 0; r < 16; ++r) any |= __ballot(ab[u][r] > tq[r]);
          uint32_t mask = (uint32_t)any | (uint32_t)(any >> 32);
          const int64_t nv = nkph - gu * 32;
          mask = nv <= 0 ? 0u : nv < 32 ? mask & ((1u << nv) - 1u) : mask;
          cnt += __builtin_popcount(mask);
          if ((int)(gu & 63) == lane) wacc = mask;
          if ((gu & 63) == 63 || gu == ngr - 1) {
            const int64_t w = (gu & ~(int64_t)63) + lane;
            if (w <= gu) ws[w] = wacc;
            wacc = 0u;
          }
        }
      }
    }
    if (active) {
      uint32_t* lw = a.live + (wid - a.wid0) * ngr;
      for (int64_t w = lane; w < ngr; w += 64) lw[w] = ws[w];
      if (lane == 0) {
        atomicAdd(a.range_cnt + ((int)wid >> a.live_shift), cnt);
        // a heavy block without a place in the heavy list (-cnt) runs unsplit
        int c = cnt;
        if (cnt > PR_HEAVY) {
          const int slot = atomicAdd(a.heavy_cnt + ((int)wid >> a.live_shift), 1);
          if (slot < a.heavy_max) a.heavy_list[slot] = (int32_t)wid;
          else c = -cnt;
        }
        a.qb_cnt[wid] = c;
      }
    }
  }
}

// Better entry under (score descending, id ascending); empty entries
// (-inf, -1) come last.
__device__ __forceinline__ bool prune_before(uint2 x, uint2 y) {
  const float a = __uint_as_float(x.x), b = __uint_as_float(y.x);
  return a > b || (a == b && x.y < y.y);
}

// The selection of one query block (wid) over a share of its live key
// blocks by one wavefront: the key blocks of live words start, start +
// stride, start + 2 stride, ... (word g covers key blocks 32 g .. 32 g + 31),
// in ascending order, through the wavefront's NPF-slot LDS ring (each slot
// filled by direct global->LDS loads: operand slices, then the 32 key ids;
// NPF - 1 blocks ahead, the waits counting the ring loads, the only vector
// memory operations of the block loop besides the occasional reload of the
// live words, whose own waits are stricter).  Leaves each lane's half-list
// (top KP under (score descending, id ascending), +inf sentinels in slots
// [0, KP - topk)) in ls / lj.
//
// COL (lists longer than 16): no lists; every key above the seed goes to the
// row's candidate array, cand[(lhalf cap + n) N H + row] for n < cap, and the
// lane's count (past cap when the array overflowed) to cand_cnt[2 row +
// lhalf], as the streaming collecting pass does.
template <int D, int KP, int NPF, bool COL = false>
__device__ __forceinline__ void prune_wave(const ScanArgs& a, int64_t wid, int start, int stride,
                                           unsigned char* wring, uint2* wcb, float (&ls)[KP],
                                           int (&lj)[KP], int64_t& qrow_out, bool& qvalid_out) {
  constexpr int NM = D / 16;
  constexpr int SLOT = NM * 1024 + 256;            // operand slices, then 64 ids
  constexpr int LPB = NM + 1;                      // ring loads per block
  const int lane = threadIdx.x & 63;
  const int lrow = lane & 31, lhalf = lane >> 5;
  const int64_t N = a.N;
  const int H = a.H;
  const int topk = a.topk;
  const int64_t nkb = a.nkb, ngr = a.ngr;
  const int h = (int)(wid / nkb);
  const int64_t pos = (wid % nkb) * 32 + lrow;
  const bool qvalid = pos < N;
  const int64_t qrow = a.perm[(int64_t)h * N + (qvalid ? pos : N - 1)];
  qrow_out = qrow;
  qvalid_out = qvalid;
  const int64_t NH = N * H;
  const int64_t crow = qrow * H + h;
  int ccnt = 0;
  (void)NH;
  (void)crow;
  bf16x8_t qb[NM];
  {
    const uint16_t* qp = a.q + (qrow * H + h) * D + 8 * lhalf;
#pragma unroll
    for (int m = 0; m < NM; ++m) qb[m] = *reinterpret_cast<const bf16x8_t*>(qp + 16 * m);
  }
  float thr = qvalid ? next_down(a.thr[qrow * H + h]) : kInf;
  const int nsent = KP - topk;
#pragma unroll
  for (int i = 0; i < KP; ++i) {
    ls[i] = i < nsent ? kInf : -kInf;
    lj[i] = -1;
  }
  int cnt = 0;
  uint2* cb = wcb + lane;
  // Entries of the candidate buffer into the list under (score descending,
  // id ascending).  Keys come out of id order; as long as no candidate ties
  // a listed score, the one-med3-per-slot insertion keeps that order.  The
  // first tie (exact float equality, rare) puts the lane's equal runs in id
  // order and switches it to the full comparator for good.  The candidate
  // bound stays one step below the k-th score, so a key tying it with a
  // smaller id still reaches the buffer.
  bool ordered = false;
  auto sort_runs = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int pass = 0; pass < KP; ++pass) {
#pragma unroll
      for (int t = 1 + (pass & 1); t < KP; t += 2) {
        if (ls[t] == ls[t - 1] && (unsigned)lj[t] < (unsigned)lj[t - 1]) {
          const int x = lj[t];
          lj[t] = lj[t - 1];
          lj[t - 1] = x;
        }
      }
    }
  };
  auto drain = [&]() __attribute__((always_inline)) {
#pragma unroll 1
    for (int c = 0; __ballot(c < cnt) != 0ull; ++c) {
      if (c < cnt) {
        const uint2 e = cb[c * 64];
        const float sv = __uint_as_float(e.x);
        const int key = (int)e.y;
        if (sv > ls[KP - 1] || (sv == ls[KP - 1] && (unsigned)key < (unsigned)lj[KP - 1])) {
          if (!ordered) {
            bool tie = false;
#pragma unroll
            for (int t = 0; t < KP; ++t) tie = tie || ls[t] == sv;
            if (tie) {
              sort_runs();
              ordered = true;
            }
          }
          if (ordered) ordered_insert<KP>(ls, lj, sv, key);
          else list_insert<KP>(ls, lj, sv, key);
        }
      }
    }
    thr = fmaxf(thr, next_down(ls[KP - 1]));
    cnt = 0;
  };

  // Live key blocks: this wavefront's words are start + stride j, j <
  // nmine, taken from the one holding the query block's own position
  // onward, cyclically (its nearest keys first, so the running k-th score
  // rises early and later blocks take fewer candidates); lane l holds word
  // j = (jfirst + j0 + l) mod nmine of the current group of 64.  Block and
  // word indices fit 32 bits (N <= 2^19).
  const uint32_t* lw = a.live + (wid - a.wid0) * ngr;
  const int ngr32 = (int)ngr;
  const int nmine = ngr32 > start ? (ngr32 - start + stride - 1) / stride : 0;
  // the word of the padded key block nearest the query block's positions
  const int64_t nkph = a.nkp_h[h];
  const int own = (int)(((wid % nkb) * nkph / nkb) >> 5);
  int jfirst = own > start ? (own - start + stride - 1) / stride : 0;
  jfirst = jfirst < nmine ? jfirst : 0;
  auto word_of = [&](int j) __attribute__((always_inline)) {
    const int jj = jfirst + j;
    return start + stride * (jj < nmine ? jj : jj - nmine);
  };
  int j0 = 0;
  uint32_t wv = lane < nmine ? lw[word_of(lane)] : 0u;
  uint64_t nz = __ballot(wv != 0u);
  uint32_t bits = 0u;
  int wbase = 0;
  auto next = [&]() __attribute__((always_inline)) -> int {
    while (bits == 0u) {
      if (nz == 0ull) {
        j0 += 64;
        if (j0 >= nmine) return -1;
        wv = j0 + lane < nmine ? lw[word_of(j0 + lane)] : 0u;
        nz = __ballot(wv != 0u);
        continue;
      }
      const int w = __builtin_ctzll(nz);
      nz &= nz - 1ull;
      bits = (uint32_t)__builtin_amdgcn_readlane((int)wv, w);
      wbase = word_of(j0 + w) * 32;
    }
    const int blk = wbase + __builtin_ctz(bits);
    bits &= bits - 1u;
    return blk;
  };

  // Per wavefront: one base for the head's key copy and one for its key
  // ids; each load's block is a 32-bit lane offset.
  const uint16_t* kbase = a.kop + (int64_t)h * a.nkp * NM * 512;
  const int32_t* pb = a.kid + (int64_t)h * a.nkp * 32;
  const unsigned wring_lds =
      (unsigned)(uintptr_t)(__attribute__((address_space(3))) unsigned char*)wring;
  // Block b into ring slot i (an exhausted slot loads block 0, never scored,
  // so every fill is LPB loads): slice m from the operand-order copy (lane
  // l's 16 bytes at l * 16), then the ids of slots 0..31 (lanes 32..63
  // repeat them; empty slots hold -1 and zero keys, and are never
  // appended).
  auto fill = [&](int i, int bq) __attribute__((always_inline)) {
    const unsigned bb = bq < 0 ? 0u : (unsigned)bq;
    const unsigned sl = wring_lds + (unsigned)(i * SLOT);
    const unsigned voff = bb * (unsigned)(NM * 1024) + (unsigned)lane * 16u;
#pragma unroll
    for (int m = 0; m < NM; ++m) {
      asm volatile("global_load_lds_dwordx4 %0, %1" ::"v"(voff + (unsigned)(m * 1024)),
                   "s"(kbase), "{m0}"(__builtin_amdgcn_readfirstlane(sl + (unsigned)(m * 1024)))
                   : "memory");
    }
    asm volatile("global_load_lds_dword %0, %1" ::"v"((bb * 32u + (unsigned)lrow) * 4u),
                 "s"(pb), "{m0}"(__builtin_amdgcn_readfirstlane(sl + (unsigned)(NM * 1024)))
                 : "memory");
  };
  // Everything this wavefront loaded so far has arrived: from here the ring
  // loads are counted.
  __builtin_amdgcn_s_waitcnt(0x0f70);
  static_assert(NPF >= 2 && NPF <= 4, "blocks in flight");
  // the next NPF blocks (bq0 first); slot `slot` holds bq0
  int bq0 = next(), bq1 = -1, bq2 = -1, bq3 = -1;
  fill(0, bq0);
  bq1 = next();
  fill(1, bq1);
  if constexpr (NPF > 2) {
    bq2 = next();
    fill(2, bq2);
  }
  if constexpr (NPF > 3) {
    bq3 = next();
    fill(3, bq3);
  }

  auto process = [&](int slot, int bb) __attribute__((always_inline)) {
    // the slot's loads were followed by those of the NPF - 1 other slots
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"((NPF - 1) * LPB) : "memory");
    const unsigned char* sl = wring + slot * SLOT;
    floatx16_t s = {};
#pragma unroll
    for (int m = 0; m < NM; ++m)
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
          *reinterpret_cast<const bf16x8_t*>(sl + m * 1024 + lane * 16), qb[m], s, 0, 0, 0);
    // s[r]: key row 8 (r / 4) + 4 lhalf + r % 4 of the block, query lrow.
    // Empty slots (zero rows of the copy) may pass this test; they are never
    // appended.
    (void)bb;
    if (__ballot(block_max(s) > thr) == 0ull) return;
    const int32_t* ids = reinterpret_cast<const int32_t*>(sl + NM * 1024);
    bool gq[4];
#pragma unroll
    for (int qq = 0; qq < 4; ++qq) gq[qq] = quarter_hit(s, qq, thr);
    if constexpr (COL) {
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) {
        if (gq[qq]) {
          const int4 id4 = *reinterpret_cast<const int4*>(ids + 8 * qq + 4 * lhalf);
          const int idv[4] = {id4.x, id4.y, id4.z, id4.w};
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float sv = s[4 * qq + r];
            if (sv > thr && idv[r] >= 0) {
              if (ccnt < a.cap)
                a.cand[(int64_t)(lhalf * a.cap + ccnt) * NH + crow] =
                    make_uint2(__float_as_uint(sv), (unsigned)idv[r]);
              ++ccnt;
            }
          }
        }
      }
      return;
    }
    static_assert(SCAN_CAP >= 8, "a half block appends up to 8 scores");
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      int room = cnt;
#pragma unroll
      for (int qq = 2 * hf; qq < 2 * hf + 2; ++qq) room += gq[qq] ? 4 : 0;
      if (__ballot(room > SCAN_CAP) != 0ull) drain();
#pragma unroll
      for (int qq = 2 * hf; qq < 2 * hf + 2; ++qq) {
        if (gq[qq]) {
          const int4 id4 = *reinterpret_cast<const int4*>(ids + 8 * qq + 4 * lhalf);
          const int idv[4] = {id4.x, id4.y, id4.z, id4.w};
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float sv = s[4 * qq + r];
            cb[cnt * 64] = make_uint2(__float_as_uint(sv), (unsigned)idv[r]);
            cnt += ((sv > thr) & (idv[r] >= 0)) ? 1 : 0;
          }
        }
      }
    }
  };

  // One copy of the block step: the slot index and the queue of block ids
  // rotate (blocks come out of next() in order, so once bq0 is -1 all are).
  int slot = 0;
#pragma unroll 1
  while (bq0 >= 0) {
    process(slot, bq0);
    const int nb = next();
    fill(slot, nb);
    bq0 = bq1;
    bq1 = NPF > 2 ? bq2 : nb;
    bq2 = NPF > 3 ? bq3 : nb;
    bq3 = nb;
    slot = slot + 1 == NPF ? 0 : slot + 1;
  }
  // the ring loads still in flight land in this wavefront's own slots
  __builtin_amdgcn_s_waitcnt(0x0f70);
  if constexpr (COL) {
    if (qvalid) a.cand_cnt[2 * crow + lhalf] = ccnt;
  } else {
    drain();
  }
}

// One wavefront per query block wid in [wid0, wid1) of a range left to this
// pass, with at most PR_HEAVY live key blocks, or more but no place in the
// heavy list (qb_cnt negative).  Workgroups of PS_WAVES
// wavefronts; logical ids grouped per XCD (gridDim.x is a multiple of 8),
// so each XCD's L2 serves neighbouring query blocks, which share most live
// key blocks.
template <int D, int KP, bool COL = false>
__global__ __launch_bounds__(PS_WAVES * 64) __attribute__((amdgpu_waves_per_eu(3))) void pruned_select_kernel(ScanArgs a) {
  static_assert(KP <= 16, "register lists");
  constexpr int CBW = COL ? 1 : SCAN_CAP * 64;
  constexpr int SLOT = (D / 16) * 1024 + 256;
  __shared__ __attribute__((aligned(1024))) unsigned char ring[PS_WAVES * PS_NPF * SLOT];
  __shared__ __attribute__((aligned(16))) uint2 cbuf[PS_WAVES * CBW];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lrow = lane & 31, lhalf = lane >> 5;
  const int64_t per = gridDim.x / 8;
  const int64_t L = (int64_t)(blockIdx.x % 8) * per + blockIdx.x / 8;
  const int64_t wid = a.wid0 + L * PS_WAVES + wave;
  if (wid >= a.wid1) return;
  if (prune_range_stream(a, wid)) return;              // left to the streaming pass
  // (lists longer than 16 take every query block here: their candidate
  // counts are per lane)
  if (!COL && a.qb_cnt[wid] > PR_HEAVY) return;        // left to the parts (below)
  const int H = a.H, topk = a.topk;
  const int h = (int)(wid / a.nkb);
  float ls[KP];
  int lj[KP];
  int64_t qrow;
  bool qvalid;
  uint2* wl = cbuf + wave * CBW;
  prune_wave<D, KP, PS_NPF, COL>(a, wid, 0, 1, ring + wave * (PS_NPF * SLOT), wl, ls, lj, qrow,
                                 qvalid);
  if constexpr (COL) return;

  // Two-pointer merge of the half-lists of each query (lanes l, l ^ 32)
  // under (score descending, id ascending), as in the streaming pass.
  const int nsent = KP - topk;
  const bool lower = lhalf == 0;
  if (!lower) {
#pragma unroll
    for (int i = 0; i < KP; ++i)
      if (i >= nsent) wl[lrow * 16 + (i - nsent)] = make_uint2(__float_as_uint(ls[i]), (unsigned)lj[i]);
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  if (lower && qvalid) {
    int32_t* oi = a.idx + (qrow * H + h) * topk;
    float* os = a.score + (qrow * H + h) * topk;
    const uint2* pl = wl + lrow * 16;
    int u = 0, r = 0;
    uint2 pu = pl[0];
    auto emit = [&](float sv, int j) __attribute__((always_inline)) {
      oi[r] = j;
      os[r] = j < 0 ? -kInf : sv;
      ++r;
    };
#pragma unroll
    for (int i = 0; i < KP; ++i) {
      if (i >= nsent) {
        const float sv = ls[i];
        const int j = lj[i];
        while (r < topk && u < topk &&
               (__uint_as_float(pu.x) > sv || (__uint_as_float(pu.x) == sv && (int)pu.y < j))) {
          emit(__uint_as_float(pu.x), (int)pu.y);
          ++u;
          pu = pl[u < 16 ? u : 15];
        }
        if (r < topk) emit(sv, j);
      }
    }
    while (r < topk) {
      emit(__uint_as_float(pu.x), (int)pu.y);
      ++u;
      pu = pl[u < 16 ? u : 15];
    }
  }
}

// Heavy query blocks (more than PR_HEAVY live key blocks) of the range, in
// PH_PARTS parts: part p of heavy block i takes the live words p, p +
// PH_PARTS, ... and writes, per query, its two half-lists merged (top-k
// under (score descending, id ascending)) to
//   parts[((i PH_PARTS + p) 32 + query) 16 + r],  r < topk.
// One wavefront per part; the grid covers heavy_max * PH_PARTS parts, and
// wavefronts past heavy_cnt * PH_PARTS (heavy_list as the bound pass left
// it) return at once (a persistent loop over the parts measured slower).
template <int D, int KP>
__global__ __launch_bounds__(PS_WAVES * 64) __attribute__((amdgpu_waves_per_eu(3))) void pruned_part_kernel(ScanArgs a) {
  static_assert(KP <= 16, "register lists");
  constexpr int CBW = SCAN_CAP * 64;
  constexpr int SLOT = (D / 16) * 1024 + 256;
  __shared__ __attribute__((aligned(1024))) unsigned char ring[PS_WAVES * PS_NPF * SLOT];
  __shared__ __attribute__((aligned(16))) uint2 cbuf[PS_WAVES * CBW];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lrow = lane & 31, lhalf = lane >> 5;
  const int nh = a.heavy_cnt[(int)a.wid0 >> a.live_shift];
  const int nparts = (nh < a.heavy_max ? nh : a.heavy_max) * PH_PARTS;
  const int t = blockIdx.x * PS_WAVES + wave;
  if (t >= nparts) return;
  if (prune_range_stream(a, a.wid0)) return;           // the whole range streams
  const int topk = a.topk;
  const int nsent = KP - topk;
  uint2* wl = cbuf + wave * CBW;
  {
    const int hi = t / PH_PARTS, part = t % PH_PARTS;
    const int64_t wid = a.heavy_list[hi];
    float ls[KP];
    int lj[KP];
    int64_t qrow;
    bool qvalid;
    prune_wave<D, KP, PS_NPF>(a, wid, part, PH_PARTS, ring + wave * (PS_NPF * SLOT), wl, ls, lj,
                              qrow, qvalid);
    (void)qrow;
    (void)qvalid;
    if (lhalf == 1) {
#pragma unroll
      for (int i = 0; i < KP; ++i)
        if (i >= nsent) wl[lrow * 16 + (i - nsent)] = make_uint2(__float_as_uint(ls[i]), (unsigned)lj[i]);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    if (lhalf == 0) {
      uint2* o = a.heavy_parts + ((int64_t)t * 32 + lrow) * 16;
      const uint2* pl = wl + lrow * 16;
      int u = 0, r = 0;
      uint2 pu = pl[0];
#pragma unroll
      for (int i = 0; i < KP; ++i) {
        if (i >= nsent) {
          const uint2 mine = make_uint2(__float_as_uint(ls[i]), (unsigned)lj[i]);
          while (r < topk && u < topk && prune_before(pu, mine)) {
            o[r++] = pu;
            ++u;
            pu = pl[u < 16 ? u : 15];
          }
          if (r < topk) o[r++] = mine;
        }
      }
      while (r < topk) {
        o[r++] = pu;
        ++u;
        pu = pl[u < 16 ? u : 15];
      }
    }
  }
}

// One thread per (heavy block, query), eight heavy blocks per workgroup
// (persistent over heavy_cnt): the heads of the query's PH_PARTS lists sit in
// registers, and after each output entry only the list that supplied it is
// read again, so the merge is PH_PARTS - 1 compares per entry.
template <int KP>
__global__ __launch_bounds__(256) void pruned_merge_kernel(ScanArgs a) {
  constexpr int LS = 32 * 16;                          // entries between parts
  if (prune_range_stream(a, a.wid0)) return;
  const int nh0 = a.heavy_cnt[(int)a.wid0 >> a.live_shift];
  const int nh = nh0 < a.heavy_max ? nh0 : a.heavy_max;
  const int topk = a.topk;
  const int H = a.H;
  const int q = threadIdx.x & 31;
  const uint2 none = make_uint2(__float_as_uint(-kInf), 0xffffffffu);
  for (int hi = blockIdx.x * 8 + (int)(threadIdx.x >> 5); hi < nh; hi += gridDim.x * 8) {
    const int64_t wid = a.heavy_list[hi];
    const int h = (int)(wid / a.nkb);
    const int64_t pos = (wid % a.nkb) * 32 + q;
    if (pos >= a.N) continue;
    const uint2* src = a.heavy_parts + ((int64_t)hi * PH_PARTS * 32 + q) * 16;
    uint2 cur[PH_PARTS];
    int at[PH_PARTS];
#pragma unroll
    for (int p = 0; p < PH_PARTS; ++p) {
      at[p] = 0;
      cur[p] = src[p * LS];                            // topk >= 1: entry 0 exists
    }
    const int64_t row = a.perm[(int64_t)h * a.N + pos];
    int32_t* oi = a.idx + (row * H + h) * topk;
    float* os = a.score + (row * H + h) * topk;
    for (int r = 0; r < topk; ++r) {
      int best = 0;
      uint2 e = cur[0];
#pragma unroll
      for (int p = 1; p < PH_PARTS; ++p) {
        if (prune_before(cur[p], e)) {
          e = cur[p];
          best = p;
        }
      }
      const int jj = (int)e.y;
      oi[r] = jj;
      os[r] = jj < 0 ? -kInf : __uint_as_float(e.x);
#pragma unroll
      for (int p = 0; p < PH_PARTS; ++p) {
        if (p == best) {
          ++at[p];
          cur[p] = at[p] < topk ? src[p * LS + at[p]] : none;
        }
      }
    }
  }
}

// After a range's bound pass: whether the streaming pass takes the range
// (more than PRUNE_STREAM_NUM / PRUNE_STREAM_DEN of its key blocks live on
// average).
__global__ void prune_decide_kernel(ScanArgs a) {
  const int r = (int)a.wid0 >> a.live_shift;
  const int64_t rows = a.wid1 - a.wid0;
  a.range_stream[r] = (int64_t)a.range_cnt[r] * PRUNE_STREAM_DEN >= rows * a.nkb * PRUNE_STREAM_NUM;
}

// Group layout, key copy and bound rows, then per range of query blocks the
// bound pass and the pruned selection: light query blocks, the parts of heavy
// ones, their merge (COL: every query block collects its candidates in one
// wavefront).  range_stream then tells the streaming pass which ranges are
// its own.
template <int D, int KP, bool COL = false>
hipError_t launch_prune(const ScanArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(group_layout_kernel, dim3((unsigned)a.H), dim3(GL_THREADS), 0, s, a);
  hipLaunchKernelGGL(key_pack_kernel<D>, dim3((unsigned)ceil_div(a.ngr * 32, 4), (unsigned)a.H),
                     dim3(256), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  auto bk = bound_live_kernel<D>;
  const int nwg = resident_workgroups(bk, PR_WAVES * 64);
  auto pk = pruned_part_kernel<D, KP>;
  if (nwg <= 0) return hipErrorInvalidDevice;
  const int64_t total = (int64_t)a.H * a.nkb;
  for (int64_t r = 0; r < total; r += a.live_rows) {
    ScanArgs b = a;
    b.wid0 = r;
    b.wid1 = r + a.live_rows < total ? r + a.live_rows : total;
    hipLaunchKernelGGL(bk, dim3((unsigned)nwg), dim3(PR_WAVES * 64), 0, s, b, nwg);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(prune_decide_kernel, dim3(1), dim3(1), 0, s, b);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t wgs = ceil_div(b.wid1 - b.wid0, PS_WAVES);
    hipLaunchKernelGGL((pruned_select_kernel<D, KP, COL>), dim3((unsigned)(8 * ceil_div(wgs, 8))),
                       dim3(PS_WAVES * 64), 0, s, b);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    if constexpr (COL) continue;
    hipLaunchKernelGGL(pk, dim3((unsigned)ceil_div((int64_t)a.heavy_max * PH_PARTS, PS_WAVES)),
                       dim3(PS_WAVES * 64), 0, s, b);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(pruned_merge_kernel<KP>,
                       dim3((unsigned)ceil_div((int64_t)a.heavy_max, 8)), dim3(256), 0, s, b);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}
