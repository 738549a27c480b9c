"""Host-side reconstruction of the score scan's address arithmetic.

For one-graph launches (the persistent grid of score_topk_kernel) this
re-derives, from the formulas the kernel uses, every index it forms:

* the split of the H * ceil(N/32) query blocks over nwg workgroups and the
  sub-tiles each workgroup walks (rows, query-order positions);
* the key rows and 32-bit lane offsets of the direct global->LDS chunk loads
  (`Scanner::issue`), and the LDS bytes they write in the chunk ring;
* the per-lane candidate buffer entries and the merge area (selection pass),
  the per-row candidate arrays and counts (collecting pass), and the output
  slots.

and checks each against the size of what it indexes.  Two GPU memory
faults were recorded in a former long-list selection pass,
`score_topk_kernel<32, 45, 1, 8>` (45-entry lists partly in scratch) at
N = 10^5, H = 4 with 256 workgroups of 512 threads and 64 KB of LDS, both
times with many rows whose candidate arrays had overflowed.  The first case
below re-derives that launch: every index it forms stays inside its buffer,
so the cause was not found in the address arithmetic.  That kernel is no
longer built; overflowing rows are now recomputed by rank passes of the
16-entry selection kernel, whose launches are checked too.  CPU only.
"""
import math

import numpy as np

import pytest

SCAN_QPW = 32
SCAN_CAP = 8
COLLECT_CAP = 256
M_THRESH, M_SELECT, M_COLLECT = 0, 1, 2
QB = 1


def shape(D, mode, W):
    lpw_cfg = {M_THRESH: 4, M_SELECT: 2, M_COLLECT: 2}[mode]
    nbuf = 2
    NM = D // 16
    ROWB = 2 * D
    LPW = 3 if D % 3 == 0 else lpw_cfg
    CHUNK = 1024 * W * LPW
    TK = CHUNK // ROWB
    SUBT = TK // 32
    assert SUBT * NM == W * LPW
    return dict(NM=NM, ROWB=ROWB, LPW=LPW, NBUF=nbuf, CHUNK=CHUNK, TK=TK, SUBT=SUBT)


def lds_bytes(D, KP, mode, W):
    s = shape(D, mode, W)
    kb = s["NBUF"] * s["CHUNK"]
    cb = W * SCAN_CAP * 64 * 8 if mode == M_SELECT else 0
    return kb, cb


def subtiles(N, H, W, nwg):
    """(workgroup, head, q0, q1) in the order each workgroup walks them."""
    nbph = (N + 31) // 32
    total = nbph * H
    out = []
    for L in range(nwg):
        b, be = total * L // nwg, total * (L + 1) // nwg
        while b < be:
            h, nb0 = b // nbph, b % nbph
            rem = be - b
            nst = -(-rem // (W * QB))
            n = min(-(-rem // nst), nbph - nb0)
            out.append((L, h, nb0 * 32, min((nb0 + n) * 32, N)))
            b += n
    return out


def check_launch(N, H, D, KP, mode, W, nwg, topk, sample=1, rank0=0):
    s = shape(D, mode, W)
    NH = N * H
    tiles = subtiles(N, H, W, nwg)
    # every (head, row) is covered exactly once, and each sub-tile fits W
    # wavefronts of 32 rows
    seen = [0] * (NH)
    for (_, h, q0, q1) in tiles:
        assert 0 <= q0 < q1 <= N and q1 - q0 <= W * QB * 32
        for pos in range(q0, q1):
            seen[h * N + pos] += 1
    assert min(seen) == 1 and max(seen) == 1

    kb_bytes, cb_bytes = lds_bytes(D, KP, mode, W)
    CBW = SCAN_CAP * 64
    # query positions: pl is clamped to [q0, q1 - 1]; perm has H*N entries
    for (_, h, q0, q1) in tiles[:: max(1, len(tiles) // 64)]:
        for wave in range(W):
            first = q0 + wave * QB * 32
            for lrow in (0, 31):
                pos = first + lrow
                pl = pos if pos < q1 else q1 - 1
                assert 0 <= h * N + pl < NH
    # key chunk loads: the graph is [0, N); rows past the end re-read the last
    nchunks = -(-N // s["TK"])
    nproc = -(-nchunks // sample)
    for j in list(range(min(nproc, 3))) + [nproc - 1]:
        c = j * sample
        first = c * s["TK"]
        left = N - first
        assert left >= 1
        rmax = min(left, s["TK"]) - 1
        for wave in (0, W - 1):
            for i in range(s["LPW"]):
                blk = wave + i * W
                for lane in (0, 31, 32, 63):
                    row = (blk // s["NM"]) * 32 + (lane & 31)
                    piece = 2 * (blk % s["NM"]) + (lane >> 5)
                    r = row if row < rmax else rmax
                    off = r * (H * s["ROWB"]) + piece * 16
                    assert off < 2 ** 32
                    # element index of the 16 bytes read, inside [N][H][D]
                    elem = ((first + r) * H + (H - 1)) * D + off % s["ROWB"] // 2
                    assert elem + 8 <= NH * D
                    for slot in range(s["NBUF"]):
                        lds = slot * s["CHUNK"] + blk * 1024 + lane * 16
                        assert lds + 16 <= kb_bytes
    if mode == M_SELECT:
        # candidate buffer entry c of lane l, wave w: cbuf[w*CBW + l + 64c],
        # c < SCAN_CAP (a drain runs before an append could pass it)
        for wave in (0, W - 1):
            for lane in (0, 63):
                e = wave * CBW + lane + 64 * (SCAN_CAP - 1)
                assert kb_bytes + 8 * (e + 1) <= kb_bytes + cb_bytes
        if KP <= 16:                               # merge area: 32 rows of 16 entries
            assert 31 * 16 + 15 < CBW
    if mode == M_COLLECT:
        # cand[(lhalf*cap + n)*NH + r], n < cap; cand_cnt[2r + lhalf]
        assert (1 * COLLECT_CAP + COLLECT_CAP - 1) * NH + (NH - 1) < 2 * COLLECT_CAP * NH
        assert 2 * (NH - 1) + 1 < 2 * NH
    # outputs: (row*H + h)*topk + rank0 + r, r < kk = min(KP, topk - rank0);
    # a rank pass also reads entry rank0 - 1 of the row
    kk = min(KP, topk - rank0)
    assert kk >= 1 and ((N - 1) * H + H - 1) * topk + rank0 + kk - 1 < NH * topk
    if rank0 > 0:
        assert 0 <= rank0 - 1 < topk
    return kb_bytes + cb_bytes


def test_recorded_fault_launch_shape_stays_in_bounds():
    # the former score_topk_kernel<32, 45, 1, 8>: 256 workgroups x 512
    # threads (grid 131072), 64 KB of LDS, as in the records
    lds = check_launch(N=100000, H=4, D=32, KP=45, mode=M_SELECT, W=8, nwg=256, topk=45)
    assert lds == 65536


@pytest.mark.parametrize("rank0", [0, 16, 32])
def test_long_list_rank_passes_stay_in_bounds(rank0):
    # score_topk_kernel<32, 16, 1, 16> recomputing overflowing rows of k = 45:
    # one 1024-thread workgroup per CU (128 KB of LDS)
    lds = check_launch(N=100000, H=4, D=32, KP=16, mode=M_SELECT, W=16, nwg=256, topk=45,
                       rank0=rank0)
    assert lds == 131072


@pytest.mark.parametrize("N,H,D,KP,mode,W,nwg,topk,sample", [
    (100000, 4, 32, 45, M_COLLECT, 8, 256, 45, 1),
    (100000, 4, 32, 45, M_THRESH, 8, 256, 45, 2),
    (100000, 4, 32, 15, M_SELECT, 16, 256, 15, 1),
    (100000, 4, 32, 15, M_THRESH, 16, 256, 15, 32),
    (500000, 4, 32, 15, M_SELECT, 16, 256, 15, 1),
    (31623, 4, 32, 15, M_SELECT, 16, 256, 15, 1),
    (8192, 4, 64, 8, M_SELECT, 16, 256, 8, 1),
    (16384, 2, 96, 15, M_SELECT, 16, 256, 15, 1),
    (12288, 4, 32, 16, M_SELECT, 16, 256, 45, 1),
])
def test_one_graph_launches_stay_in_bounds(N, H, D, KP, mode, W, nwg, topk, sample):
    lds = check_launch(N, H, D, KP, mode, W, nwg, topk, sample)
    assert lds <= 160 * 1024


def test_partition_is_contiguous_per_workgroup():
    tiles = subtiles(100000, 4, 8, 256)
    nbph = math.ceil(100000 / 32)
    by_wg = {}
    for (L, h, q0, q1) in tiles:
        by_wg.setdefault(L, []).append(h * nbph * 32 + q0)
    for L, starts in by_wg.items():
        assert starts == sorted(starts)


# ---------------------------------------------------------------- pruned selection
PR_WAVES, PS_WAVES, PR_MAX_WORDS, PR_LPW, PR_NBUF, PS_NPF = 16, 4, 704, 2, 3, 2


def order_pivots(N):
    return min(max((N // 96) & ~31, 32), 16384)


def pruned_sizes(N, H, D):
    """(nkb, nkp, ngr, live_rows): query blocks, padded key blocks per head
    (each pivot group starts a new block), live words, and ranges of 2^s
    query blocks (s >= 4), as many as 16 MiB of live words hold."""
    nkb = -(-N // 32)
    nkp = nkb + order_pivots(N)
    ngr = -(-nkp // 32)
    rows = H * nkb
    fit = (16 << 20) // (ngr * 4)
    shift = 4
    while (2 << shift) <= fit and (1 << shift) < rows:
        shift += 1
    return nkb, nkp, ngr, 1 << shift


def group_layout(sizes):
    """group_layout_kernel for one head: first positions, first padded slots
    and the group of every padded key block."""
    gstart = np.concatenate([[0], np.cumsum(sizes)[:-1]])
    padded = (sizes + 31) // 32 * 32
    pstart = np.concatenate([[0], np.cumsum(padded)[:-1]])
    bgroup = np.repeat(np.arange(sizes.size), padded // 32)
    return gstart, pstart, bgroup


def check_pruned(N, H, D, nwg=256, seed=0):
    """Every index formed by group_layout_kernel, key_pack_kernel,
    bound_live_kernel and pruned_select_kernel (elements of kop / kid / bop /
    live and the group tables, LDS offsets) against the sizes the host gives
    those buffers."""
    NM, NMB = D // 16, (32 if D == 96 else D) // 16 + 1   # split rows: bounds on the high part
    NPF = PS_NPF
    nkb, nkp, ngr, live_rows = pruned_sizes(N, H, D)
    npiv = order_pivots(N)
    kop_elems, bop_elems = H * nkp * NM * 512, H * ngr * NMB * 512
    kid_elems = H * nkp * 32
    assert ngr <= PR_MAX_WORDS and -(-ngr // 64) * 64 <= PR_MAX_WORDS
    # group layout: any split of N positions into npiv groups (empty ones
    # included) fills at most nkp blocks, and every slot maps back inside
    # its group and the head's order
    rng = np.random.default_rng(seed)
    worst = np.full(npiv, N // npiv)
    worst[: N - worst.sum()] += 1
    for sizes in (worst, np.bincount(rng.integers(0, npiv, N), minlength=npiv),
                  np.r_[np.full(npiv - 1, 1), N - npiv + 1]):
        assert sizes.sum() == N and sizes.size == npiv
        gstart, pstart, bgroup = group_layout(sizes)
        nkph = bgroup.size
        assert nkph <= nkp
        for b in (0, nkph // 2, nkph - 1):
            r = bgroup[b]
            for l in (0, 31):
                o = b * 32 + l - pstart[r]
                assert 0 <= o < 32 * -(-sizes[r] // 32)
                if o < sizes[r]:
                    assert 0 <= gstart[r] + o < N
    # key_pack_kernel: grid (ceil(32 ngr / 4), H) x 4 wavefronts
    for h in (0, H - 1):
        for b in (0, nkb - 1, nkp - 1, nkp, ngr * 32 - 1):
            if b >= ngr * 32:
                continue
            g, br = b // 32, b % 32
            for lane in (0, 31, 32, 63):
                lh = lane >> 5
                for m in range(NMB):
                    e = ((h * ngr + g) * NMB + m) * 512 + (br + 32 * lh) * 8
                    assert 0 <= e and e + 8 <= bop_elems
                if b < nkp:
                    assert h * nkp + b < H * nkp               # bgroup
                    assert (h * nkp + b) * 32 + (lane & 31) < kid_elems
                    assert h * npiv + npiv - 1 < H * npiv      # gstart / gsize / pstart
                    for m in range(NM):
                        node = N - 1
                        assert (node * H + h) * D + 8 * lh + 16 * m + 8 <= N * H * D
                        e = ((h * nkp + b) * NM + m) * 512 + lane * 8
                        assert e + 8 <= kop_elems
    # bound_live_kernel: ranges of live_rows query blocks, sub-tiles of <= 16
    total = H * nkb
    nrange = -(-total // live_rows)
    GPB = PR_WAVES * PR_LPW // NMB // 2 * 2
    assert GPB >= 2 and GPB * NMB <= PR_WAVES * PR_LPW
    SLOT = PR_WAVES * PR_LPW * 1024
    assert PR_NBUF * SLOT + PR_WAVES * PR_MAX_WORDS * 4 <= 160 * 1024
    covered = 0
    for r0 in range(0, total, live_rows):
        r1 = min(total, r0 + live_rows)
        seen = set()
        for L in range(nwg):
            b, be = r0 + (r1 - r0) * L // nwg, r0 + (r1 - r0) * (L + 1) // nwg
            while b < be:
                h, nb0 = b // nkb, b % nkb
                rem = be - b
                nst = -(-rem // PR_WAVES)
                n = min(-(-rem // nst), nkb - nb0)
                assert 1 <= n <= PR_WAVES
                for w in range(n):
                    wid = b + w
                    assert wid not in seen and r0 <= wid < r1
                    seen.add(wid)
                    assert (wid - r0) * ngr + ngr - 1 < min(live_rows, total) * ngr
                    assert wid < total and wid // live_rows < nrange
                b += n
        assert len(seen) == r1 - r0
        covered += len(seen)
        # ring loads: wavefront w, piece p = w + i * PR_WAVES, batch ib (groups
        # past the last one re-read the last)
        for ib in (0, -(-ngr // GPB) - 1):
            for w in range(PR_WAVES):
                for i in range(PR_LPW):
                    p = w + i * PR_WAVES
                    pp = min(p, GPB * NMB - 1)
                    g = min(ib * GPB + pp // NMB, ngr - 1)
                    e = ((H - 1) * ngr + g) * NMB * 512 + (pp % NMB) * 512 + 63 * 8
                    assert e + 8 <= bop_elems
                    lds = (PR_NBUF - 1) * SLOT + p * 1024 + 63 * 16
                    assert lds + 16 <= PR_NBUF * SLOT
        # pruned_select_kernel: 8 * ceil(ceil(n / 4) / 8) workgroups
        wgs = -(-(r1 - r0) // PS_WAVES)
        grid = 8 * -(-wgs // 8)
        per = grid // 8
        logical = sorted((bx % 8) * per + bx // 8 for bx in range(grid))
        assert logical == list(range(grid))
        # the largest wid it scores and the block reads
        assert r0 + (grid - 1) * PS_WAVES + 3 >= r1 - 1
        PSLOT = NM * 1024 + 256
        assert PS_WAVES * NPF * PSLOT + PS_WAVES * 8 * 64 * 8 <= 160 * 1024
        if D == 32:                                   # four workgroups per CU
            assert PS_WAVES * NPF * PSLOT + PS_WAVES * 8 * 64 * 8 <= 40 * 1024
        if D == 96:                                   # two workgroups per CU
            assert PS_WAVES * NPF * PSLOT + PS_WAVES * 8 * 64 * 8 <= 80 * 1024
        for bb in (0, nkb - 1, nkp - 1):
            for m in range(NM):
                e = (H - 1) * nkp * NM * 512 + 63 * 8 + (bb * NM + m) * 512
                assert e + 8 <= kop_elems
                lds = (PS_WAVES - 1) * NPF * PSLOT + (NPF - 1) * PSLOT + m * 1024 + 63 * 16
                assert lds + 16 <= PS_WAVES * NPF * PSLOT
            # ids: lane offset (32 bb + l % 32) * 4 from kid + h nkp 32
            for lane in (0, 31, 63):
                off = (bb * 32 + (lane & 31)) * 4
                assert (H - 1) * nkp * 32 + off // 4 < kid_elems and off < (1 << 32)
            lds = (NPF - 1) * PSLOT + NM * 1024 + 63 * 4
            assert lds + 4 <= NPF * PSLOT
    assert covered == total
    return nkb, ngr, live_rows


@pytest.mark.parametrize("N,H,D", [(100000, 4, 32), (100000, 4, 96), (31623, 4, 32), (8192, 4, 32), (16384, 2, 64),
                                   (500000, 4, 32), (524288, 4, 64), (9000, 4, 32)])
def test_pruned_selection_indices_stay_in_bounds(N, H, D):
    nkb, ngr, live_rows = check_pruned(N, H, D)
    assert min(live_rows, H * nkb) * ngr * 4 <= 16 << 20


@pytest.mark.parametrize("N,H", [(100000, 4), (500000, 4), (8192, 4), (40000, 1)])
def test_heavy_parts_and_merge_stay_in_bounds(N, H):
    """pruned_part_kernel / pruned_merge_kernel: heavy query block i (i <
    heavy_max, slots past it are never written) in PARTS parts; part t = i
    PARTS + p writes entries ((t 32 + q) 16 + r), r < topk <= 16, and the
    merge reads entries ((i PARTS 32 + q) 16) + p 32 16 + at, at < topk; the
    parts' words p, p + PARTS, ... cover each word once."""
    PARTS, HMAX = 8, 8192
    nkb, nkp, ngr, live_rows = pruned_sizes(N, H, 32)
    heavy_max = min(live_rows, H * nkb, HMAX)
    size = heavy_max * PARTS * 32 * 16
    i, q, p, r = heavy_max - 1, 31, PARTS - 1, 15
    t = i * PARTS + p
    assert (t * 32 + q) * 16 + r < size
    assert (i * PARTS * 32 + q) * 16 + p * 32 * 16 + r < size
    words = sorted(w for p in range(PARTS) for w in range(p, ngr, PARTS))
    assert words == list(range(ngr))
