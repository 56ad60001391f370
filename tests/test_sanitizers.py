"""The CPU suite under AddressSanitizer and UndefinedBehaviorSanitizer.

Builds the oracle (C) and the HIP library's host side (argument checks, layouts,
workspace sizing, launch set-up; device code is left as it is) with ASan + UBSan, then
runs every `-m "not gpu"` test against those builds in a child process with the
sanitizer runtime preloaded: any invalid access or undefined behaviour aborts the run.
A canary with a planted heap overflow, run the same way, shows the detector is live.
Both builds use clang (hipcc's, so the two share one sanitizer runtime)."""
import os
import subprocess
import sys
import textwrap

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "hierarchical_kv_approximation_amd", "csrc")
LLVM = "/opt/rocm/llvm"
CLANG = os.path.join(LLVM, "bin", "clang")
HIPCC = "/opt/rocm/bin/hipcc"


def _runtime():
    base = os.path.join(LLVM, "lib", "clang")
    for ver in sorted(os.listdir(base)) if os.path.isdir(base) else []:
        p = os.path.join(base, ver, "lib", "linux", "libclang_rt.asan-x86_64.so")
        if os.path.exists(p):
            return p
    return None


def _env(rt):
    env = dict(os.environ)
    env.update(LD_PRELOAD=rt, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    return env


@pytest.fixture(scope="module")
def builds(tmp_path_factory):
    rt = _runtime()
    if not (os.path.exists(CLANG) and os.path.exists(HIPCC) and rt):
        pytest.skip("clang, hipcc or the clang sanitizer runtime is missing")
    d = tmp_path_factory.mktemp("sanitized")
    san = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer"]
    oracle = str(d / "liblod_oracle.so")
    subprocess.run([CLANG, "-O1", "-g", "-std=c99", "-fPIC", "-shared", "-ffp-contract=off", *san,
                    "-o", oracle, os.path.join(ROOT, "oracle", "lod_oracle.c"),
                    os.path.join(ROOT, "oracle", "video_oracle.c"), "-lm"], check=True)
    host_san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                "-Xarch_host", "-fno-sanitize-recover=undefined"]
    flags = ["--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-ffp-contract=off",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-Wno-unused-command-line-argument",
             *host_san, "-I", os.path.join(ROOT, "include"), "-I", CSRC]
    procs, objs = [], []
    for src in ("lod_host.cpp", "lod_build.hip", "lod_decode.hip", "lod_prefill.hip", "lod_video.hip"):
        obj = str(d / (src + ".o"))
        objs.append(obj)
        procs.append(subprocess.Popen([HIPCC, *flags, "-c", os.path.join(CSRC, src), "-o", obj],
                                      stdout=subprocess.PIPE, stderr=subprocess.STDOUT))
    for p in procs:
        out, _ = p.communicate()
        assert p.returncode == 0, out.decode(errors="replace")[-2000:]
    lib = str(d / "liblod.so")
    subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-Xarch_host", "-fsanitize=address",
                    "-Xarch_host", "-fsanitize=undefined", "-o", lib, *objs], check=True)
    canary = str(d / "libcanary.so")
    src = d / "canary.c"
    src.write_text("#include <stdlib.h>\nint canary(int n) { int* a = malloc(4 * n); int s = a[n]; free(a); return s; }\n")
    subprocess.run([CLANG, "-O0", "-g", "-fPIC", "-shared", *san, "-o", canary, str(src)], check=True)
    return {"runtime": rt, "oracle": oracle, "lib": lib, "canary": canary, "dir": d}


def test_canary_overflow_is_caught(builds):
    code = f"import ctypes; ctypes.CDLL({builds['canary']!r}).canary(8)"
    r = subprocess.run([sys.executable, "-c", code], env=_env(builds["runtime"]), capture_output=True,
                       text=True, timeout=300)
    assert r.returncode != 0 and "heap-buffer-overflow" in r.stderr, r.stderr[-2000:]


def test_cpu_suite_under_asan_and_ubsan(builds):
    runner = builds["dir"] / "run.py"
    runner.write_text(textwrap.dedent(f"""
        import sys
        sys.path.insert(0, {ROOT!r})
        from hierarchical_kv_approximation_amd import lod
        from oracle import oracle as orc
        lod.LIB_PATH = {builds['lib']!r}
        orc._LIB_PATH = {builds['oracle']!r}
        import pytest
        rc = pytest.main(["-q", "-m", "not gpu", "-p", "no:cacheprovider", {os.path.join(ROOT, 'tests')!r},
                          "--ignore", {os.path.join(ROOT, 'tests', 'test_sanitizers.py')!r}])
        maps = open("/proc/self/maps").read()
        assert {builds['lib']!r} in maps and {builds['oracle']!r} in maps, "sanitized builds not loaded"
        sys.exit(rc)
    """))
    r = subprocess.run([sys.executable, str(runner)], env=_env(builds["runtime"]), capture_output=True,
                       text=True, timeout=1200, cwd=str(builds["dir"]))
    tail = (r.stdout[-3000:] + r.stderr[-3000:])
    assert r.returncode == 0, tail
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, tail
