"""libkmip loads, exports every symbol its header declares, and rejects bad
arguments on the host (before any HIP call).  CPU only: no kernel runs."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kmip.h")

torch = pytest.importorskip("torch")
from graph_transformer_sparse_amd import kmip  # noqa: E402

# These cases pass fake device pointers and rely on host validation failing
# first; they are meant for machines without a GPU.
pytestmark = pytest.mark.skipif(torch.cuda.is_available(),
                                reason="host-validation tests use fake device pointers")

OK, INVALID, UNSUPPORTED, WORKSPACE = 0, 1, 2, 3
FAKE = ctypes.c_void_p(1 << 20)       # aligned, never dereferenced: validation fails first


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kmip_[a-z0-9_]+)\s*\(", text)))


def test_header_symbols_exported():
    L = kmip.lib()
    names = declared_functions()
    assert set(names) == set(kmip.EXPORTED)
    for n in names:
        assert hasattr(L, n), n


def test_status_strings_and_version():
    assert kmip.status_string(OK).startswith("KMIP_OK")
    assert "workspace" in kmip.status_string(WORKSPACE)
    assert kmip.version() >= 10000


def _fwd(q=FAKE, k=FAKE, v=FAKE, N=128, H=2, d=32, topk=15, offs=None, B=0, out=FAKE,
         idx=FAKE, score=FAKE, ws=None, ws_bytes=0):
    return kmip.lib().kmip_forward(q, k, v, N, H, d, topk, offs, B, out, idx, score, ws,
                                   ws_bytes, None)


def _bwd(N=128, H=2, d=32, topk=15, ws=FAKE, ws_bytes=1 << 40, dq=FAKE, offs=None, B=0):
    return kmip.lib().kmip_backward(FAKE, FAKE, FAKE, N, H, d, topk, offs, B, FAKE, FAKE, FAKE,
                                    dq, FAKE, FAKE, ws, ws_bytes, None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), INVALID), (dict(out=None), INVALID), (dict(idx=None), INVALID),
    (dict(N=0), INVALID), (dict(H=0), INVALID), (dict(B=-1), INVALID),
    (dict(B=3, offs=None), INVALID),
    (dict(q=ctypes.c_void_p((1 << 20) + 8)), INVALID),
    (dict(d=48), UNSUPPORTED), (dict(d=128), UNSUPPORTED), (dict(topk=0), UNSUPPORTED),
    (dict(topk=65), UNSUPPORTED), (dict(N=1 << 30, H=4), UNSUPPORTED),
    (dict(N=2, H=(1 << 15) + 1, d=32), UNSUPPORTED), (dict(N=2, H=1 << 14, d=64), WORKSPACE),
    (dict(B=4, offs=FAKE, ws=None, ws_bytes=0), WORKSPACE),
    (dict(B=4, offs=FAKE, ws=FAKE, ws_bytes=16), WORKSPACE),
    (dict(ws=None, ws_bytes=0), WORKSPACE),
    (dict(ws=FAKE, ws_bytes=1020), WORKSPACE),
])
def test_forward_rejects(kw, status):
    assert _fwd(**kw) == status


@pytest.mark.parametrize("kw,status", [
    (dict(dq=None), INVALID), (dict(N=-5), INVALID), (dict(d=16), UNSUPPORTED),
    (dict(topk=100), UNSUPPORTED), (dict(ws=None), WORKSPACE), (dict(ws_bytes=100), WORKSPACE),
    (dict(ws=ctypes.c_void_p((1 << 20) + 16)), INVALID),
])
def test_backward_rejects(kw, status):
    assert _bwd(**kw) == status


def test_workspace_sizes_are_linear_in_n():
    f = kmip.forward_workspace_bytes
    b = kmip.backward_workspace_bytes
    # One graph: an fp32 threshold, an int32 query-order entry and a 16-bit
    # code per row, plus per-head pivot counters (two int32 tables of 16
    # copies per pivot, one pivot per ~96 nodes: under 1.5 bytes per row).
    # The pruned selection adds per padded key slot a copy of its key (2d
    # bytes), its node id (4 bytes) and a share of its block's bound row
    # (d/16 + 1 bytes); every pivot group (one per ~96 nodes) starts a new 32-slot
    # block, so there are at most N + 32 npiv slots per head.  Plus the live
    # words of one range of query blocks (at most 16 MiB) and the part lists
    # of up to 8192 heavy query blocks (at most 256 MiB).
    rows = 100000 * 4
    parts = 8192 * 8 * 32 * 16 * 8                      # heavy query blocks' part lists
    for N in (100000, 200000, 500000):
        npiv = (N // 96) & ~31
        slots = 4 * (N + 32 * npiv)
        pr = _pruned_bytes(N, 4, 32)
        assert slots * (64 + 4) <= pr <= slots * (64 + 4 + 4 + 1) + parts + (17 << 20)
    for (N, H, d) in [(100000, 4, 32), (200000, 4, 32), (500000, 4, 32), (8192, 4, 64)]:
        without = f(N, H, d, 15, 0) - _pruned_bytes(N, H, d)
        assert 10 * N * H <= without <= 12 * N * H + (1 << 20)
    # lists longer than 16: the pruned buffers without the heavy parts, and
    # the candidate arrays (2 x 256 entries of 8 bytes per row) with counts
    assert rows * 10 <= (f(100000, 4, 32, 45, 0) - _pruned_bytes(100000, 4, 32, parts=False)
                         - 2 * 256 * rows * 8 - rows * 8) <= rows * 10 + (4 << 20)
    assert f(100000, 4, 32, 15, 64) > rows * 4                # thresholds plus the tile plan
    b1, b2 = b(100000, 4, 32, 15), b(200000, 4, 32, 15)
    assert 1.9 < b2 / b1 < 2.1                              # O(N * H * k)
    # pairs (p, ds), two key / id / payload buffers, digit counts: ~50 B per pair
    assert b(500000, 4, 32, 15) < 1.6e9
    assert f(0, 4, 32, 15, 0) == 0 and b(10, 4, 48, 15) == 0   # invalid shapes -> 0


def _fwd32(N=128, H=2, d=32, topk=15, offs=None, B=0, v=FAKE, ws=FAKE, ws_bytes=1 << 40):
    return kmip.lib().kmip_forward_f32(FAKE, FAKE, v, N, H, d, topk, offs, B, FAKE, FAKE, FAKE,
                                       ws, ws_bytes, None)


@pytest.mark.parametrize("kw,status", [
    (dict(v=None), INVALID), (dict(N=0), INVALID), (dict(B=2, offs=None), INVALID),
    (dict(v=ctypes.c_void_p((1 << 20) + 4)), INVALID), (dict(d=96), UNSUPPORTED),
    (dict(topk=65), UNSUPPORTED), (dict(ws=None), WORKSPACE), (dict(ws_bytes=4096), WORKSPACE),
])
def test_forward_f32_rejects(kw, status):
    assert _fwd32(**kw) == status


def test_backward_f32_rejects():
    L = kmip.lib()
    args = [FAKE, FAKE, FAKE, 128, 2, 32, 15, None, 0, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE]
    assert L.kmip_backward_f32(*args, FAKE, 100, None) == WORKSPACE
    assert L.kmip_backward_f32(*args[:5], 16, *args[6:], FAKE, 1 << 40, None) == UNSUPPORTED
    args[12] = None                                   # dq
    assert L.kmip_backward_f32(*args, FAKE, 1 << 40, None) == INVALID


def _pruned_bytes(N, H, d, parts=True):
    """Buffers of the pruned selection (one graph with a query order, bf16
    rows of 32 or 64, or split-precision rows of 96, 2^16 <= N <= 2^19);
    lists longer than 16 have no heavy parts' lists."""
    if not (1 << 16) <= N <= (1 << 19):
        return 0
    a = lambda x: (x + 255) // 256 * 256
    npiv = min(max((N // 96) & ~31, 32), 16384)
    nkb = -(-N // 32)
    nkp = nkb + npiv
    ngr = -(-nkp // 32)
    rows = H * nkb
    fit = (16 << 20) // (ngr * 4)
    shift = 4
    while (2 << shift) <= fit and (1 << shift) < rows:
        shift += 1
    held = min(rows, 1 << shift)
    nrange = -(-rows // (1 << shift))
    heavy = min(held, 8192)
    return (3 * a(H * npiv * 4) + a(H * 4) + a(H * nkp * 4) + a(H * nkp * 32 * 4)
            + a(H * nkp * (d // 16) * 1024) + a(H * ngr * ((32 if d == 96 else d) // 16 + 1) * 1024) + a(held * ngr * 4)
            + a(rows * 4) + 3 * a(nrange * 4) + a(heavy * 4)
            + (a(heavy * 8 * 32 * 16 * 8) if parts else 0))


def test_f32_workspace_adds_split_rows():
    # The fp32 forward also holds q and k as bf16 rows of 3d elements; its
    # pruned selection (d = 32 only) works on those 96-wide rows.
    for (N, H, d, k, B) in [(1000, 2, 32, 15, 0), (100000, 4, 32, 15, 0), (100000, 4, 64, 15, 0),
                            (5000, 4, 64, 45, 7)]:
        extra = kmip.forward_f32_workspace_bytes(N, H, d, k, B) - kmip.forward_workspace_bytes(
            N, H, d, k, B)
        if B == 0:
            extra += _pruned_bytes(N, H, d) - (_pruned_bytes(N, H, 3 * d) if d == 32 else 0)
        assert 12 * N * H * d <= extra <= 12 * N * H * d + 512
    assert kmip.forward_f32_workspace_bytes(10, 4, 48, 15, 0) == 0


def test_no_workspace_forward_rejects_before_any_gpu_call():
    """Sizes beyond the static scratch and invalid arguments are refused on
    the host, before the scratch array's address is looked up."""
    L = kmip.lib()
    # lists longer than 16 need 4 KB of candidate arrays per row: 4e5 rows
    st = L.kmip_forward_no_workspace(FAKE, FAKE, FAKE, 100000, 4, 32, 45, None, 0, FAKE, FAKE,
                                     FAKE, None)
    assert st == 3                                     # KMIP_ERR_WORKSPACE
    st = L.kmip_forward_no_workspace(FAKE, FAKE, FAKE, 4 * 10 ** 6, 4, 32, 15, None, 0, FAKE,
                                     FAKE, FAKE, None)
    assert st == 3
    st = L.kmip_forward_no_workspace(None, FAKE, FAKE, 1000, 4, 32, 15, None, 0, FAKE, FAKE,
                                     FAKE, None)
    assert st == 1                                     # KMIP_ERR_INVALID_VALUE
    st = L.kmip_forward_no_workspace(FAKE, FAKE, FAKE, 1000, 4, 48, 15, None, 0, FAKE, FAKE,
                                     FAKE, None)
    assert st == 2                                     # KMIP_ERR_UNSUPPORTED
    # the entry without a workspace runs without the pruned selection: the
    # rest of the forward workspace fits its static array up to N = 5e5
    assert (kmip.forward_workspace_bytes(500000, 4, 32, 15, 0) - _pruned_bytes(500000, 4, 32)
            <= kmip.NO_WORKSPACE_BYTES)
