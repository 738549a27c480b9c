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

import pytest

SCAN_QPW = 32
SCAN_CAP = 8
COLLECT_CAP = 128
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
