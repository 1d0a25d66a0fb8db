"""The C ABI's host validation and planning layer under AddressSanitizer and
UndefinedBehaviorSanitizer (host code only, no recovery): hxq_api.cpp is
compiled again with the host sanitizers, linked with the library's other
objects and a driver (host_sanitize_driver.cpp) that makes calls every one of
which is rejected or answered on the host (bad arguments, workspace sizes
and kernel choice over shapes up to 2^31, status strings).  CPU only."""

import os
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
PKG = os.path.join(ROOT, "vq_compressed_linear_amd")
BUILD = os.path.join(PKG, "_build")
CLANG = "/opt/rocm/llvm/bin/clang++"
HIPCC = "/opt/rocm/bin/hipcc"
SAN = ["-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]


def _have_toolchain():
    return os.path.exists(CLANG) and os.path.exists(HIPCC) and os.path.isdir(BUILD)


@pytest.mark.skipif(not _have_toolchain(), reason="needs hipcc, ROCm clang and the library's objects (build())")
def test_host_layer_under_sanitizers(tmp_path):
    import sys

    sys.path.insert(0, ROOT)
    from vq_compressed_linear_amd._digest import source_digest

    objs = [os.path.join(BUILD, f) for f in sorted(os.listdir(BUILD)) if f.endswith(".o") and f != "hxq_api.o"]
    assert objs, "no library objects: run build() first"
    api = str(tmp_path / "hxq_api_san.o")
    # host-side sanitizers only: each -fsanitize flag goes to the host compilation
    host_san = []
    for f in SAN:
        host_san += ["-Xarch_host", f]
    cmd = [HIPCC, "-x", "hip", "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC",
           '-DHXQ_SOURCE_DIGEST="%s"' % source_digest(), "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           *host_san, "-c", os.path.join(PKG, "csrc", "hxq_api.cpp"), "-o", api]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    exe = str(tmp_path / "host_sanitize")
    link = [CLANG, "-O1", "-g", "-std=c++17", *SAN, "-I", os.path.join(ROOT, "include"),
            os.path.join(HERE, "host_sanitize_driver.cpp"), api, *objs,
            "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib", "-o", exe]
    r = subprocess.run(link, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    # the driver is not the first library loaded in every environment, so the link-order check is off
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, (r.stdout[-3000:], r.stderr[-3000:])
    assert "checks ok" in r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr
