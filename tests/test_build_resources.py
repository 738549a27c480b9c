"""Resource limits of the built gfx950 kernels, read from libkmip.so's own
code objects (CPU only).

A kernel whose per-lane scratch (private segment) grows to kilobytes cannot
be dispatched with a full grid (the runtime fails to allocate its scratch and
aborts the queue), and one whose LDS exceeds 160 KB cannot launch at all.
Both are compile-time properties, so they are checked here, before any GPU
run.
"""
import os
import re
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "graph_transformer_sparse_amd", "libkmip.so")
LLVM = "/opt/rocm/llvm/bin"
MAGIC = b"__CLANG_OFFLOAD_BUNDLE__"
MAX_PRIVATE = 4096           # bytes of scratch per lane
MAX_LDS = 160 * 1024         # bytes per workgroup on gfx950


def _kernels():
    tools = [os.path.join(LLVM, t) for t in ("llvm-objcopy", "clang-offload-bundler",
                                            "llvm-readelf")]
    if not os.path.exists(LIB) or not all(os.path.exists(t) for t in tools):
        pytest.skip("libkmip.so or the LLVM tools are missing")
    objcopy, bundler, readelf = tools
    out = []
    with tempfile.TemporaryDirectory() as tmp:
        fat = os.path.join(tmp, "fatbin")
        subprocess.run([objcopy, f"--dump-section=.hip_fatbin={fat}", LIB, os.path.join(tmp, "x")],
                       check=True, capture_output=True)
        data = open(fat, "rb").read()
        starts = [m.start() for m in re.finditer(re.escape(MAGIC), data)]
        for n, (a, b) in enumerate(zip(starts, starts[1:] + [len(data)])):
            part = os.path.join(tmp, f"b{n}")
            open(part, "wb").write(data[a:b])
            co = os.path.join(tmp, f"b{n}.co")
            r = subprocess.run([bundler, "--unbundle", "--type=o", f"--input={part}",
                                "--targets=hipv4-amdgcn-amd-amdhsa--gfx950", f"--output={co}"],
                               capture_output=True)
            if r.returncode != 0 or not os.path.exists(co) or os.path.getsize(co) == 0:
                continue
            notes = subprocess.run([readelf, "--notes", co], check=True, capture_output=True,
                                   text=True).stdout
            for blk in notes.split(".agpr_count")[1:]:
                name = re.search(r"\.name:\s+(\S+)", blk)
                priv = re.search(r"\.private_segment_fixed_size:\s+(\d+)", blk)
                lds = re.search(r"\.group_segment_fixed_size:\s+(\d+)", blk)
                if name and priv and lds:
                    out.append((name.group(1), int(priv.group(1)), int(lds.group(1))))
    return out


def test_kernel_scratch_and_lds_within_limits():
    ks = _kernels()
    names = {k[0] for k in ks}
    assert any("score_topk_kernel" in n for n in names), "no scan kernels found"
    assert any("segreduce_kernel" in n for n in names) and any("gather" in n for n in names)
    bad = [(n, p, l) for n, p, l in ks if p > MAX_PRIVATE or l > MAX_LDS]
    assert not bad, bad
