"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

The HIP sources are compiled host-only with the sanitizers on the host side
(device code is not built: no kernel runs), linked with
`tests/host_asan/abi_check.cpp`, and run: workspace sizes over a grid of
shapes, every class of invalid argument, and valid calls with stand-in
pointers that lay out the workspace and then fail to launch (only on a
machine without a GPU).  CPU only.
"""
import glob
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SAN = ["-Xarch_host", "-fsanitize=address,undefined"]


def _no_gpu():
    try:
        import torch
        return not torch.cuda.is_available()
    except Exception:
        return True


pytestmark = [
    pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not found"),
    pytest.mark.skipif(not _no_gpu(), reason="stand-in pointers: for machines without a GPU"),
]


def test_host_code_under_sanitizers(tmp_path):
    common = ["--offload-arch=gfx950", "-fgpu-rdc", "-O1", "-g", "-std=c++17", *SAN,
              f"-I{os.path.join(ROOT, 'include')}"]
    objs = []
    srcs = sorted(glob.glob(os.path.join(ROOT, "graph_transformer_sparse_amd", "csrc", "*.hip")))
    srcs.append(os.path.join(ROOT, "tests", "host_asan", "abi_check.cpp"))
    procs = []
    for src in srcs:
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        objs.append(obj)
        cmd = [HIPCC, "--offload-host-only", *common, "-fPIC", "-x", "hip", "-c", src, "-o", obj]
        procs.append(subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT))
    for p in procs:
        out = p.communicate()[0].decode()
        assert p.returncode == 0, out
    exe = str(tmp_path / "abi_check")
    r = subprocess.run([HIPCC, "--offload-arch=gfx950", "-fgpu-rdc", "--hip-link", *SAN,
                        "-o", exe, *objs], stdout=subprocess.PIPE, stderr=subprocess.STDOUT)
    assert r.returncode == 0, r.stdout.decode()
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([exe], stdout=subprocess.PIPE, stderr=subprocess.STDOUT, env=env,
                       timeout=300)
    out = r.stdout.decode()
    assert "AddressSanitizer" not in out and "runtime error" not in out, out
    assert r.returncode == 0 and "ok: 0 failures" in out, out
