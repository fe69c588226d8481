"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

* The oracle (oracle/oracle.c) built with gcc -fsanitize=address,undefined, then its
  field product and Pippenger (threads over windows, every c) against Python integers.
* The library's host code: msm_api.hip (plans, workspace layout, argument checks,
  contexts) compiled with the sanitizers on its host side only (-Xarch_host), linked with
  the other objects of the plain build, then every workspace plan compared with the plain
  library's and every argument error path taken.

Each runs in a subprocess with the matching sanitizer runtime preloaded (gcc's libasan,
clang's asan runtime); the sanitizers abort on the first error. Builds are cached under
the git-ignored build folders, keyed by the sources' hash.
"""
import hashlib
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "elliptic_curve_scalar_amd")
CSRC = os.path.join(PKG, "csrc")
DRIVER = os.path.join(ROOT, "tests", "sanitize_driver.py")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CLANG = "/opt/rocm/llvm/bin/clang"


def _hash(paths):
    h = hashlib.sha256()
    for p in paths:
        with open(p, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def _env(preload):
    env = dict(os.environ)
    env["LD_PRELOAD"] = preload
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    return env


def _run(args, env):
    res = subprocess.run([sys.executable, DRIVER, *args], env=env, capture_output=True,
                         text=True, timeout=600)
    assert res.returncode == 0, res.stdout[-3000:] + res.stderr[-3000:]
    return res.stdout


def test_oracle_under_sanitizers():
    src = os.path.join(ROOT, "oracle", "oracle.c")
    out_dir = os.path.join(ROOT, "oracle", "_build", "asan")
    os.makedirs(out_dir, exist_ok=True)
    lib = os.path.join(out_dir, f"liboracle_asan_{_hash([src])}.so")
    if not os.path.exists(lib):
        cmd = ["gcc", "-O1", "-g", "-std=c11", "-fPIC", "-shared", "-pthread",
               "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
               "-fno-omit-frame-pointer", "-o", lib + ".tmp", src]
        subprocess.run(cmd, check=True)
        os.replace(lib + ".tmp", lib)
    libasan = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True,
                             text=True, check=True).stdout.strip()
    env = _env(libasan)
    env["ORACLE_LIB"] = lib
    assert "ok oracle" in _run(["oracle"], env)


def test_library_host_code_under_sanitizers():
    from elliptic_curve_scalar_amd import build as B
    plain = os.path.join(PKG, "libmsm.so")
    objs = [os.path.join(B.OBJ_DIR, os.path.splitext(s)[0] + ".o") for s in B.SOURCES
            if s != "msm_api.hip"]
    if not os.path.exists(plain) or not all(os.path.exists(o) for o in objs):
        B.build()
    api = os.path.join(CSRC, "msm_api.hip")
    key = _hash([api, os.path.join(CSRC, "msm_internal.hpp"), os.path.join(ROOT, "include", "msm.h")]
                + objs)
    out_dir = os.path.join(B.OBJ_DIR, "asan")
    os.makedirs(out_dir, exist_ok=True)
    lib = os.path.join(out_dir, f"libmsm_asan_{key}.so")
    if not os.path.exists(lib):
        obj = os.path.join(out_dir, "msm_api_asan.o")
        compile_cmd = [HIPCC, *B.FLAGS, "-O1", "-g",
                       "-Xarch_host", "-fsanitize=address",
                       "-Xarch_host", "-fsanitize=undefined",
                       "-Xarch_host", "-fno-sanitize-recover=undefined",
                       "-Xarch_host", "-fno-omit-frame-pointer",
                       "-c", "-o", obj, api]
        subprocess.run(compile_cmd, check=True, capture_output=True)
        link_cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-shared-libsan",
                    "-Xarch_host", "-fsanitize=address",
                    "-Xarch_host", "-fsanitize=undefined",
                    "-o", lib + ".tmp", obj, *objs]
        subprocess.run(link_cmd, check=True, capture_output=True)
        os.replace(lib + ".tmp", lib)
    rt = subprocess.run([CLANG, "-print-file-name=libclang_rt.asan-x86_64.so"],
                        capture_output=True, text=True, check=True).stdout.strip()
    if not os.path.exists(rt):
        pytest.skip("clang's AddressSanitizer runtime is not installed")
    assert "ok libmsm" in _run(["libmsm", lib, plain], _env(rt))
