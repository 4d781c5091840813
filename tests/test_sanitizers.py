"""The CPU test suite under AddressSanitizer and UndefinedBehaviorSanitizer.

Builds, into _build/asan/ (never committed):
  * the oracle (oracle/pkv_oracle.c) with clang -fsanitize=address,undefined;
  * libpagedkv with its host C++ -- the C ABI's argument validation
    (csrc/pkv_api.cpp) and the block allocator and table edits
    (csrc/block_allocator.cpp) -- sanitized on the host side only, linked with
    the regular kernel objects (the CPU tests launch no kernel);
  * a canary library with a deliberate heap overflow,
then runs every other CPU test in a child process with clang's ASan runtime
preloaded and PKV_LIBRARY / PKV_ORACLE_LIBRARY pointing at the sanitized
builds.  The canary must abort under the same setup (so a pass means
something), and the suite must pass.  Skipped where hipcc or clang is missing.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OUT = os.path.join(ROOT, "_build", "asan")
CSRC = os.path.join(ROOT, "paged_kv_cache_235_amd", "csrc")
HIPCC = "/opt/rocm/bin/hipcc"
CLANG = "/opt/rocm/llvm/bin/clang"
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer"]
CANARY = r"""
#include <stdlib.h>
int canary_overflow(int n) {
    int* a = (int*)malloc(sizeof(int) * (size_t)n);
    for (int i = 0; i < n; ++i) a[i] = i;
    int r = a[n];                       /* one past the end */
    free(a);
    return r;
}
"""


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr}"
    return r


def _build():
    os.makedirs(OUT, exist_ok=True)
    oracle_so = os.path.join(OUT, "liboracle_asan.so")
    _run([CLANG, "-O1", "-g", "-std=c99", "-fPIC", "-shared", *SAN, "-ffp-contract=off", "-o", oracle_so,
          os.path.join(ROOT, "oracle", "pkv_oracle.c"), "-lm"])
    canary_c = os.path.join(OUT, "canary.c")
    with open(canary_c, "w") as f:
        f.write(CANARY)
    canary_so = os.path.join(OUT, "libcanary_asan.so")
    _run([CLANG, "-O0", "-g", "-fPIC", "-shared", *SAN, "-o", canary_so, canary_c])
    host_san = [x for flag in SAN for x in ("-Xarch_host", flag)]
    common = ["--offload-arch=gfx950", "-std=c++17", "-fPIC", "-I" + os.path.join(ROOT, "include"), "-I" + CSRC]
    objs = []
    for src in ("pkv_api.cpp", "block_allocator.cpp"):
        obj = os.path.join(OUT, src.replace(".cpp", ".o"))
        _run([HIPCC, *common, "-O1", "-g", *host_san, "-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    flags = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
    from paged_kv_cache_235_amd._build import FILE_FLAGS
    for src in ("kv_write.hip", "decode.hip", "prefill.hip", "block_ops.hip"):
        obj = os.path.join(OUT, src.replace(".hip", ".o"))
        _run([HIPCC, *common, "-O3", *flags, *FILE_FLAGS.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    lib_so = os.path.join(OUT, "libpagedkv_asan.so")
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-Xarch_host", "-fsanitize=address",
          "-Xarch_host", "-fsanitize=undefined", "-o", lib_so, *objs])
    return oracle_so, lib_so, canary_so


def _env(oracle_so, lib_so):
    asan_rt = _run([CLANG, "-print-file-name=libclang_rt.asan-x86_64.so"]).stdout.strip()
    env = dict(os.environ)
    env.update(LD_PRELOAD=asan_rt, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1",
               PKV_LIBRARY=lib_so, PKV_ORACLE_LIBRARY=oracle_so)
    return env


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANG)) or shutil.which("gcc") is None,
                    reason="needs hipcc and clang")
def test_cpu_suite_passes_under_address_and_undefined_behaviour_sanitizers():
    oracle_so, lib_so, canary_so = _build()
    env = _env(oracle_so, lib_so)
    # the harness catches a heap overflow
    canary = subprocess.run([sys.executable, "-c", f"import ctypes; ctypes.CDLL({canary_so!r}).canary_overflow(8)"],
                            capture_output=True, text=True, env=env, timeout=120)
    assert canary.returncode != 0 and "heap-buffer-overflow" in canary.stderr, canary.stderr[-2000:]
    # every other CPU test, against the sanitized builds
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests"), "-q", "-x", "-m", "not gpu",
                        "-p", "no:cacheprovider", "--ignore", os.path.abspath(__file__)],
                       capture_output=True, text=True, env=env, cwd=ROOT, timeout=1800)
    tail = (r.stdout + r.stderr)[-3000:]
    assert r.returncode == 0, tail
    assert " passed" in r.stdout and "failed" not in r.stdout, tail
    # the child really loaded the sanitized builds
    probe = subprocess.run([sys.executable, "-c", "import oracle, paged_kv_cache_235_amd as p; "
                            "oracle.lib(); p.load_library(); "
                            "print(open('/proc/self/maps').read())"],
                           capture_output=True, text=True, env=env, cwd=ROOT, timeout=300)
    assert probe.returncode == 0, probe.stderr[-2000:]
    assert lib_so in probe.stdout and oracle_so in probe.stdout
