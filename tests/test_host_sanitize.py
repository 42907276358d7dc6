"""Host code of libenc under AddressSanitizer + UndefinedBehaviorSanitizer.

Every library source is compiled with both sanitizers on the host
compilation only (the device code is built as usual, never launched, so no
GPU is needed) and errors fatal; tests/sanitize/host_checks.cpp then parses valid stream headers (the
oracle's streams: BF16 at several block sizes, power-of-two widths, RAW,
FP16, FP32) and some 100,000 corrupted ones, checks the invariants of every
header it accepts, and drives the table sizing, batch preparation (up to its
capacity check, before any device copy) and GEMM planning functions with
edge-case arguments. Nothing here launches a kernel.
"""
import os
import shutil
import subprocess

import numpy as np
import pytest

from lossless_weight_compression_amd import build as libbuild
from lossless_weight_compression_amd import synth
from oracle import oracle as orc

HERE = os.path.dirname(os.path.abspath(__file__))
DRIVER = os.path.join(HERE, "sanitize", "host_checks.cpp")
HIPCC = libbuild.HIPCC
CLANGXX = "/opt/rocm/llvm/bin/clang++"
# host-only sanitizer flags (each -fsanitize= applies to the host pass only)
SAN_HOST = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=all"]
SAN_LINK = ["-fsanitize=address", "-fsanitize=undefined"]


def _streams(tmp):
    paths = []
    w = synth.gaussian_bits((64, 1000), 0.02, 7, 1)
    for B, pow2 in ((128, False), (512, False), (4096, False), (512, True)):
        s = orc.encode(w, B, pow2)
        paths.append((s, "bf16_b%d_p%d" % (B, int(pow2))))
    raw = orc.encode(synth.random_bits(5000, 3), 512)     # uniform patterns: RAW
    assert raw[8] == 1
    paths.append((raw, "raw"))
    for dt in (2, 3):
        v = synth.gaussian_values((32, 700), 0.02, 7, 2, dt)
        paths.append((orc.encode(v, 256, dtype=dt), "dt%d" % dt))
    out = []
    for s, name in paths:
        p = os.path.join(tmp, name + ".bin")
        s.tofile(p)
        out.append(p)
    return out


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANGXX)), reason="no ROCm clang")
def test_host_code_under_asan_ubsan(tmp_path):
    tmp = str(tmp_path)
    objs = []
    procs = []
    for src in libbuild.SOURCES:
        obj = os.path.join(tmp, src + ".o")
        cmd = [HIPCC, "-x", "hip", "--offload-arch=" + libbuild.ARCH, "-std=c++17", "-O1", "-g",
               "-fPIC", "-fno-omit-frame-pointer",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"] + SAN_HOST + [
               "-I", libbuild.INCLUDE, "-I", libbuild.CSRC, "-c", os.path.join(libbuild.CSRC, src),
               "-o", obj]
        procs.append((cmd, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT,
                                            text=True)))
        objs.append(obj)
    for cmd, p in procs:
        out, _ = p.communicate()
        assert p.returncode == 0, "compile failed: %s\n%s" % (" ".join(cmd), out)
    drv = os.path.join(tmp, "host_checks.o")
    r = subprocess.run([CLANGXX, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer"] + SAN_LINK +
                       ["-I", libbuild.INCLUDE, "-c", DRIVER, "-o", drv],
                       stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    assert r.returncode == 0, r.stdout
    exe = os.path.join(tmp, "host_checks")
    r = subprocess.run([HIPCC, "--offload-arch=" + libbuild.ARCH] + SAN_HOST + ["-o", exe, drv] + objs +
                       ["-L/opt/rocm/lib", "-Wl,-rpath,/opt/rocm/lib", "-lamdhip64"],
                       stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    assert r.returncode == 0, r.stdout
    files = _streams(tmp)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1",
               HIP_VISIBLE_DEVICES="")
    r = subprocess.run([exe, "12345"] + files, stdout=subprocess.PIPE, stderr=subprocess.STDOUT,
                       text=True, env=env, timeout=600)
    assert r.returncode == 0, r.stdout[-4000:]
    assert "failures 0" in r.stdout, r.stdout[-4000:]
    acc, rej = (int(t) for t in r.stdout.split()[1:4:2])
    assert acc > 0 and rej > 0, r.stdout
