"""Sanitizer builds on the CPU (no GPU needed, nothing is launched).

AddressSanitizer and UndefinedBehaviorSanitizer (no recovery: the first report
ends the run) over
  * the oracle, run by ``tests/sanitize/oracle_checks.cpp`` on small seeded
    inputs and on edge cases (empty inputs, repeated, negative and
    out-of-range coordinates, capacities below the result), checking
    identities that hold for any input: forward, dgrad and wgrad adjoint,
    mirror symmetry of submanifold maps, the transposed relation equal to the
    strided one read backwards, distinct supports;
  * the library's host code -- argument validation and size queries of the C
    ABI -- driven by ``tests/sanitize/abi_checks.cpp``.  The library sources
    are compiled host-only with the sanitizers; each object links against the
    GPU binary that the regular build embedded for the same source (both
    builds name it by the same compilation-unit id), so the program carries
    the real device code but never launches it.
"""
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
from convolution_voxelised_point_amd import build as libbuild  # noqa: E402

SAN_DIR = os.path.join(ROOT, "tests", "sanitize")
LLVM = "/opt/rocm/llvm/bin"
CLANGXX = os.path.join(LLVM, "clang++")
CLANG = os.path.join(LLVM, "clang")
OBJCOPY = shutil.which("objcopy") or os.path.join(LLVM, "llvm-objcopy")
NM = shutil.which("nm") or os.path.join(LLVM, "llvm-nm")
GXX = shutil.which("g++")

# Host-pass sanitizer flags for hipcc: every one is scoped to the host
# compilation, the device code is built exactly as in the library.
HIP_HOST_SAN = ["-Xarch_host", "-fsanitize=address,undefined", "-Xarch_host", "-fno-sanitize-recover=all",
                "-Xarch_host", "-fno-omit-frame-pointer"]
CPU_SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]


def run_checked(exe, leaks):
    env = dict(os.environ,
               ASAN_OPTIONS=f"detect_leaks={1 if leaks else 0}:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    return out


def sh(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return r.stdout


@pytest.mark.skipif(GXX is None, reason="g++ not found")
def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_checks")
    sh([GXX, "-std=c++17", "-O1", "-g", *CPU_SAN, os.path.join(SAN_DIR, "oracle_checks.cpp"), "-o", exe])
    out = run_checked(exe, leaks=True)
    assert "oracle checks: all passed" in out


def _host_object(src, tmp):
    """Sanitized host-only object of one library source, plus an object that
    defines its embedded-GPU-binary symbol from the regular build's object."""
    name = os.path.basename(src)
    host = os.path.join(tmp, name + ".host.o")
    sh([libbuild.HIPCC, *libbuild.CFLAGS, "--cuda-host-only", "-O1", "-g", f"-cuid={libbuild.cuid(src)}",
        *HIP_HOST_SAN, "-c", src, "-o", host])
    wanted = [l.split()[-1] for l in sh([NM, "-u", host]).splitlines() if "__hip_fatbin_" in l]
    if not wanted:
        return [host]
    assert len(wanted) == 1, wanted
    regular = os.path.join(libbuild.BUILD_DIR, name + ".o")
    blob = os.path.join(tmp, name + ".fatbin")
    sh([OBJCOPY, "-O", "binary", "--only-section=.hip_fatbin", regular, blob])
    assert os.path.getsize(blob) > 0, f"{regular} holds no GPU binary"
    asm = os.path.join(tmp, name + ".fatbin.s")
    with open(asm, "w") as f:
        f.write(f'.section .hip_fatbin,"a",@progbits\n.p2align 12\n.globl {wanted[0]}\n{wanted[0]}:\n'
                f'.incbin "{blob}"\n')
    fat = os.path.join(tmp, name + ".fatbin.o")
    sh([CLANG, "-c", asm, "-o", fat])
    return [host, fat]


def test_abi_host_code_under_sanitizers(tmp_path):
    srcs = libbuild.sources()
    if not all(os.path.exists(os.path.join(libbuild.BUILD_DIR, os.path.basename(s) + ".o")) for s in srcs):
        pytest.skip("library objects not built")
    tmp = str(tmp_path)
    with ThreadPoolExecutor(8) as ex:
        objs = [o for group in ex.map(lambda s: _host_object(s, tmp), srcs) for o in group]
    exe = os.path.join(tmp, "abi_checks")
    sh([CLANGXX, "-std=c++17", "-O1", "-g", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
        "-I", libbuild.INCLUDE, *CPU_SAN, os.path.join(SAN_DIR, "abi_checks.cpp"), *objs,
        "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib", "-o", exe])
    out = run_checked(exe, leaks=False)
    assert "abi host checks: all passed" in out
