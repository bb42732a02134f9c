"""AddressSanitizer + UBSan build of the host code (plan builder, C ABI
argument checks, dispatch tables), driven by tests/host_sanitize_main.cpp.

The host units are rebuilt with g++ and the sanitizers and linked with the
device objects of the normal build (their host stubs unsanitised); the driver
builds plans for natural, wide, ragged, mixed-parity and channel-wise irreps,
reads every table a plan exposes, feeds malformed descriptors and invalid
arguments, and checks that each is rejected on the host.  Leak detection is
on, so a plan or table the library fails to free is an error too.
"""
import glob
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "equivariant_gnn_tensor_receiver_amd", "csrc")
BUILD = os.path.join(ROOT, "_build")
HOST_UNITS = ("api", "plan", "timing", "stream_dispatch")
DEVICE_UNITS = ("gemm", "channelwise", "graph", "scratch", "ragged", "radial", "fixed")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]


def _device_objects():
    objs = [os.path.join(BUILD, u + ".o") for u in DEVICE_UNITS]
    objs += [o for o in sorted(glob.glob(os.path.join(BUILD, "stream_*.o"))) if "dispatch" not in o]
    return objs


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir("/opt/rocm/include"),
                    reason="needs g++ and the ROCm headers")
def test_host_code_under_asan_and_ubsan(tmp_path):
    objs = _device_objects()
    if not all(os.path.exists(o) for o in objs) or not os.path.exists(os.path.join(BUILD, "gen", "cg_tables.inc")):
        pytest.skip("library objects not built")
    inc = ["-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", "-I", CSRC, "-I", os.path.join(ROOT, "include"),
           "-I", os.path.join(BUILD, "gen")]
    host = []
    for u in HOST_UNITS:
        o = str(tmp_path / (u + ".o"))
        subprocess.run(["g++", "-O1", "-g", "-std=c++17"] + SAN + inc + ["-c", os.path.join(CSRC, u + ".cpp"),
                        "-o", o], check=True)
        host.append(o)
    main = str(tmp_path / "main.o")
    subprocess.run(["g++", "-O1", "-g", "-std=c++17"] + SAN + inc +
                   ["-c", os.path.join(ROOT, "tests", "host_sanitize_main.cpp"), "-o", main], check=True)
    exe = str(tmp_path / "host_sanitize")
    subprocess.run(["g++"] + SAN + ["-o", exe, main] + host + objs +
                   ["-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib"], check=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "host sanitizer checks passed" in r.stdout
