"""The oracle and the host side of libskv under AddressSanitizer and UndefinedBehaviorSanitizer
(no GPU needed).

- The oracle is compiled by gcc with -fsanitize=address,undefined and the oracle pins run against
  it in a child process (gcc's ASan runtime preloaded, since the Python interpreter is not
  instrumented).
- The host code of libskv (argument validation, workspace planning, the C ABI; abi.cpp and
  noalloc.hip) is compiled by hipcc with the sanitizers on the host side only (-Xarch_host before
  each -fsanitize=), linked with the unchanged objects of the other sources, and the C-ABI tests
  that need no device run against it (clang's ASan runtime preloaded).
Each build is first shown to be instrumented: a canary with a planted heap overflow, built the same
way, must make its child process fail with a sanitizer report.
"""
import glob
import os
import subprocess
import sys

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "sparse_kv_cache_build_amd", "csrc")
SANITIZE_GCC = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer", "-g"]


def _gcc_asan_runtime() -> str:
    return subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True,
                          check=True).stdout.strip()


def _clang_asan_runtime() -> str:
    found = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not found:
        pytest.skip("clang's ASan runtime is not installed")
    return found[-1]


def _run(cmd, preload, extra_env=None, timeout=600):
    env = dict(os.environ, LD_PRELOAD=preload, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", PYTHONDONTWRITEBYTECODE="1", **(extra_env or {}))
    return subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=timeout)


CANARY_C = """
#include <stdlib.h>
int canary(int i) { int *p = (int *)malloc(4 * sizeof(int)); for (int k = 0; k < 4; ++k) p[k] = k; int v = p[i]; free(p); return v; }
"""


CANARY_CPP = """
#include <cstdlib>
extern "C" int canary(int i) {
  int *p = static_cast<int *>(std::malloc(4 * sizeof(int)));
  for (int k = 0; k < 4; ++k) p[k] = k;
  int v = p[i];
  std::free(p);
  return v;
}
"""


def _reported(err: str) -> bool:
    """A sanitizer report: ASan's, or UBSan's (its object-size check can see the overflow first)."""
    return "AddressSanitizer" in err or "runtime error:" in err


def _canary_call(lib, preload):
    code = f"import ctypes; ctypes.CDLL({lib!r}).canary(4)"
    return _run([sys.executable, "-c", code], preload)


def test_oracle_pins_pass_under_asan_and_ubsan(tmp_path):
    rt = _gcc_asan_runtime()
    canary_src = tmp_path / "canary.c"
    canary_src.write_text(CANARY_C)
    canary = oracle.compile_source(str(canary_src), str(tmp_path / "canary.so"), extra=SANITIZE_GCC)
    r = _canary_call(canary, rt)
    assert r.returncode != 0 and _reported(r.stderr), r.stderr[-800:]
    lib = oracle.compile_source(os.path.join(ROOT, "oracle", "skv_oracle.c"), str(tmp_path / "liboracle_san.so"),
                                extra=SANITIZE_GCC)
    r = _run([sys.executable, "-m", "pytest", "tests/test_oracle_pins.py", "-x", "-q", "-p", "no:cacheprovider"], rt,
             dict(SKV_ORACLE_LIB=lib))
    assert r.returncode == 0, (r.stdout[-1500:] + r.stderr[-1500:])
    assert "Sanitizer" not in r.stderr, r.stderr[-1500:]


def _hipcc_host_sanitized(src, out):
    cmd = ["/opt/rocm/bin/hipcc", "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer",
           "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-c", src, "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    return out


def _clang_link(objs, out, rt_dir):
    import torch
    tlib = os.path.join(os.path.dirname(torch.__file__), "lib")
    cmd = ["/opt/rocm/llvm/bin/clang++", "-shared", "-fsanitize=address,undefined", "-shared-libsan", "-o", out,
           *objs, f"-L{tlib}", "-l:libamdhip64.so", f"-Wl,-rpath,{tlib}", f"-Wl,-rpath,{rt_dir}"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    return out


def test_host_abi_passes_under_asan_and_ubsan(tmp_path):
    rt = _clang_asan_runtime()
    rt_dir = os.path.dirname(rt)
    build_dir = os.path.join(ROOT, "_build")
    plain = [os.path.join(build_dir, f) for f in ("meta.o", "score.o", "select.o", "attn.o")]
    if not all(os.path.exists(p) for p in plain):
        pytest.fail("the library's objects are not built (run __graft_entry__.build())")
    canary_src = tmp_path / "canary.cpp"
    canary_src.write_text(CANARY_CPP)
    canary = _clang_link([_hipcc_host_sanitized(str(canary_src), str(tmp_path / "canary.o"))],
                         str(tmp_path / "canary.so"), rt_dir)
    r = _canary_call(canary, rt)
    assert r.returncode != 0 and _reported(r.stderr), r.stderr[-800:]
    san = [_hipcc_host_sanitized(os.path.join(CSRC, f), str(tmp_path / (os.path.splitext(f)[0] + ".o")))
           for f in ("abi.cpp", "noalloc.hip")]
    lib = _clang_link(san + plain, str(tmp_path / "libskv_san.so"), rt_dir)
    # every C-ABI test but the symbol inventory (the sanitizer adds its own padded globals)
    r = _run([sys.executable, "-m", "pytest", "tests/test_abi_cpu.py", "-x", "-q", "-p", "no:cacheprovider",
              "-k", "not keeps_no_host_state"], rt, dict(SKV_LIB=lib))
    assert r.returncode == 0, (r.stdout[-1500:] + r.stderr[-1500:])
    assert "Sanitizer" not in r.stderr and "runtime error" not in r.stderr, r.stderr[-1500:]
