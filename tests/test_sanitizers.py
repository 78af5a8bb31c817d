"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only, no GPU).

* The oracle's C source is built with gcc's sanitizers and its CPU pin tests run against that
  build (every oracle function on small, edge and error cases).
* The library's host code (argument validation, workspace queries and launch planning of every
  C-ABI entry point) is built with clang's sanitizers on the host side only (`-Xarch_host`; the
  gfx950 device code is built as usual) and the C-ABI tests run against it.  They reach every
  host-side refusal without a GPU.

Sanitizer reports go to files (ASAN_OPTIONS log_path); a test fails on a non-zero exit or on
any report.  Leak detection is off: the Python interpreter itself holds memory to exit."""
import glob
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

SAN = ["-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=all"]


def _gcc_runtime(name):
    try:
        path = subprocess.check_output(["gcc", f"-print-file-name={name}"], text=True).strip()
    except (OSError, subprocess.CalledProcessError):
        return None
    return path if os.path.isabs(path) and os.path.exists(path) else None


def _run_pytest(tmp_path, env_extra, files):
    reports = os.path.join(str(tmp_path), "report")
    env = dict(os.environ)
    env.update(env_extra)
    env["ASAN_OPTIONS"] = f"detect_leaks=0:log_path={reports}"
    env["UBSAN_OPTIONS"] = f"print_stacktrace=1:log_path={reports}"
    proc = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", *files],
                          cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    found = sorted(glob.glob(reports + "*"))
    text = "".join(open(f).read()[:4000] for f in found)
    assert proc.returncode == 0 and not found, (proc.stdout[-3000:], proc.stderr[-3000:], text)
    return proc.stdout


def test_oracle_under_asan_ubsan(tmp_path):
    asan, ubsan = _gcc_runtime("libasan.so"), _gcc_runtime("libubsan.so")
    if not (shutil.which("gcc") and asan and ubsan):
        pytest.skip("gcc sanitizer runtimes not available")
    lib = os.path.join(str(tmp_path), "liboracle_san.so")
    subprocess.check_call(["gcc", "-O1", "-g", *SAN, "-fno-omit-frame-pointer", "-fopenmp", "-fPIC", "-shared",
                           "-std=c11", os.path.join(ROOT, "oracle", "dsv_oracle.c"), "-o", lib, "-lm"])
    files = sorted(glob.glob(os.path.join(ROOT, "tests", "test_oracle_*.py")))
    out = _run_pytest(tmp_path, {"LD_PRELOAD": f"{asan} {ubsan}", "DSV_ORACLE_LIBRARY": lib}, files)
    assert "passed" in out


def test_library_host_code_under_asan_ubsan(tmp_path):
    from block_verification_attention_amd import build as B

    hipcc = B.hipcc()
    rt = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not (shutil.which(hipcc) or os.path.exists(hipcc)) or not rt:
        pytest.skip("hipcc or clang's sanitizer runtime not available")
    flags = [f for f in B.HIPCC_FLAGS if f != "-O3"] + ["-O1", "-fno-omit-frame-pointer"]
    for f in SAN:
        flags += ["-Xarch_host", f]
    objs, procs = [], []
    for src in B.SOURCES:
        obj = os.path.join(str(tmp_path), src.replace(".hip", ".o"))
        procs.append(subprocess.Popen([hipcc, *flags, "-I", B.INCLUDE, "-c", os.path.join(B.CSRC, src), "-o", obj],
                                      stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True))
        objs.append(obj)
    for p in procs:
        _, err = p.communicate()
        assert p.returncode == 0, err[-2000:]
    lib = os.path.join(str(tmp_path), "libdsv_san.so")
    link = [hipcc, "--offload-arch=gfx950", "-shared", "-fPIC"]
    for f in SAN[:2]:
        link += ["-Xarch_host", f]
    subprocess.check_call(link + objs + ["-o", lib])
    out = _run_pytest(tmp_path, {"LD_PRELOAD": rt[-1], "DSV_LIBRARY": lib},
                      [os.path.join(ROOT, "tests", "test_abi.py")])
    assert "passed" in out
