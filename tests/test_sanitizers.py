"""Host builds under AddressSanitizer and UndefinedBehaviorSanitizer (no GPU).

* The oracle (oracle/oracle.c, built with gcc) runs every entry point on
  small layers held in buffers of exactly their documented sizes
  (tests/sanitize/oracle_drive.c).  A planted one-element-short scratch
  buffer in the oracle must be reported, which shows the instrumented build
  is the one that ran.
* The C ABI's host code (csrc/api.hip, instrumented on the host side only,
  with unsigned wrap-around and implicit integer truncation checks on top)
  runs every refusal path of every entry point and sweeps the size queries
  over the whole supported range (tests/sanitize/abi_validate.cpp).  The
  device kernels are linked from the regular build and never launched.
"""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
ORACLE_SRC = os.path.join(ROOT, "oracle", "oracle.c")
PKG = os.path.join(ROOT, "sparse_mixture_experts_14_amd")
CSRC = os.path.join(PKG, "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

GCC_SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-fno-omit-frame-pointer"]
# host side only: each sanitizer flag right after -Xarch_host
HOST_SAN = ("-Xarch_host -fsanitize=address "
            "-Xarch_host -fsanitize=undefined,unsigned-integer-overflow,implicit-integer-truncation "
            "-Xarch_host -fno-sanitize-recover=all").split()


def _run(cmd, env=None, timeout=300):
    return subprocess.run(cmd, capture_output=True, text=True, env=env, timeout=timeout)


def _oracle_exe(src, tmp, name):
    exe = os.path.join(tmp, name)
    r = _run(["gcc", "-std=c11", "-O1", "-g", "-fopenmp", *GCC_SAN, "-Wall", "-o", exe,
              os.path.join(HERE, "oracle_drive.c"), src, "-lm"])
    assert r.returncode == 0, r.stderr
    return exe


def _env(**kw):
    env = dict(os.environ)
    env.update(kw)
    return env


def test_oracle_clean_under_asan_ubsan(tmp_path):
    exe = _oracle_exe(ORACLE_SRC, str(tmp_path), "oracle_drive")
    r = _run([exe], env=_env(OMP_NUM_THREADS="2"))
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-4000:]
    assert "all entry points clean" in r.stdout


def test_planted_overflow_is_reported(tmp_path):
    """One double short in the forward's per-thread scratch: the token's u
    vector ends one element past the buffer."""
    src = open(ORACLE_SRC).read()
    site = "malloc(sizeof(double) * (size_t)(n + d_ff + 2 * d))"
    assert src.count(site) == 2
    bad = src.replace(site, "malloc(sizeof(double) * (size_t)(n + d_ff + 2 * d - 1))", 1)
    path = tmp_path / "oracle_short.c"
    path.write_text(bad)
    exe = _oracle_exe(str(path), str(tmp_path), "oracle_short")
    r = _run([exe], env=_env(OMP_NUM_THREADS="2"))
    assert r.returncode != 0
    assert "heap-buffer-overflow" in r.stderr


@pytest.fixture(scope="module")
def kernel_objects():
    """The regular build's objects of every source but api.hip."""
    build_dir = os.path.join(PKG, "_build")
    srcs = sorted(f for f in os.listdir(CSRC) if f.endswith(".hip") and f != "api.hip")
    objs = [os.path.join(build_dir, s + ".o") for s in srcs]
    if not all(os.path.exists(o) for o in objs):
        from sparse_mixture_experts_14_amd import build
        build.build()
    return objs


def test_abi_host_validation_clean(tmp_path, kernel_objects):
    api_o = str(tmp_path / "api_san.o")
    exe = str(tmp_path / "abi_validate")
    common = ["--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-I",
              os.path.join(ROOT, "include"), *HOST_SAN, "-Wno-unused-command-line-argument"]
    r = _run([HIPCC, *common, "-I", CSRC, "-Xclang", "-target-feature", "-Xclang",
              "-packed-fp32-ops", "-c", os.path.join(CSRC, "api.hip"), "-o", api_o])
    assert r.returncode == 0, r.stderr
    r = _run([HIPCC, *common, "-x", "c++", os.path.join(HERE, "abi_validate.cpp"), "-x", "none",
              api_o, *kernel_objects, "-o", exe])
    assert r.returncode == 0, r.stderr
    # the HIP runtime keeps allocations until exit: leak reports are its, not ours
    r = _run([exe], env=_env(ASAN_OPTIONS="detect_leaks=0"))
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-4000:]
    assert "validation clean" in r.stdout
