"""AddressSanitizer and UndefinedBehaviorSanitizer builds of the CPU code: the
fp64 oracle (gcc) and the library's host validation path (every HIP source
compiled for the host only, so no GPU code is built or run). Each driver in
tests/sanitize/ must finish without a sanitizer report and with every status
as expected."""
import glob
import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
HIPCC = "/opt/rocm/bin/hipcc"
ENV = dict(os.environ, ASAN_OPTIONS="abort_on_error=1:detect_leaks=0",
           UBSAN_OPTIONS="halt_on_error=1:abort_on_error=1:print_stacktrace=1")


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr}"
    return r


@pytest.mark.skipif(shutil.which("gcc") is None, reason="no gcc")
def test_oracle_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_san")
    _run(["gcc", "-O1", "-g", "-std=c11", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
          "-fno-omit-frame-pointer", "-ffp-contract=off", "-I", os.path.join(ROOT, "oracle"),
          os.path.join(SAN, "oracle_san.c"), os.path.join(ROOT, "oracle", "zq_oracle.c"), "-lm", "-o", exe])
    r = _run([exe], env=ENV, timeout=300)
    assert "0 failures" in r.stdout


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="no hipcc")
def test_host_validation_under_asan_ubsan(tmp_path):
    # host-only objects: the kernels are not compiled, and nothing here
    # reaches a launch
    flags = ["--offload-host-only", "-O1", "-g", "-std=c++20", "-fPIC", "-fno-omit-frame-pointer",
             "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=all",
             "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROOT, "weight_quantized_amd", "csrc")]
    srcs = sorted(glob.glob(os.path.join(ROOT, "weight_quantized_amd", "csrc", "*.hip")))
    objs = [str(tmp_path / (os.path.basename(s)[:-4] + ".o")) for s in srcs]
    with ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        list(ex.map(lambda so: _run([HIPCC, *flags, "-c", so[0], "-o", so[1]]), zip(srcs, objs)))
    exe = str(tmp_path / "abi_san")
    # the GPU code objects those host objects would register are not built:
    # their symbols stay unresolved, and no call below reaches a kernel
    _run([HIPCC, *flags, "-x", "c++", os.path.join(SAN, "abi_san.c"), "-x", "none", *objs, "-o", exe,
          "-Wl,--unresolved-symbols=ignore-all"])
    r = _run([exe], env=ENV, timeout=300)
    assert "0 failures" in r.stdout
