"""Address and undefined-behaviour sanitizers on the CPU (no GPU).

1. The oracle (plain C) is rebuilt with gcc's AddressSanitizer and UBSan, and its
   pin tests run against that build in a child process (the sanitizer runtime
   preloaded, every report fatal).
2. The library's host translation units (argument validation, option table,
   event hook) are rebuilt with clang's host-side AddressSanitizer and UBSan and
   linked with the ordinary kernel objects; the C-ABI tests, which exercise the
   validation paths without reaching a GPU, run against that build.

Sanitizers apply to host code only: the GPU code objects are built as usual."""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OUT = os.path.join(ROOT, "_build", "sanitize")
HOST_SAN = "-Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined -Xarch_host -fno-sanitize-recover=all -Xarch_host -fno-omit-frame-pointer"
GCC_SAN = "-fsanitize=address,undefined -fno-sanitize-recover=all -fno-omit-frame-pointer"
ENV_SAN = {"ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1:abort_on_error=0",
           "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"}


def _child(code, preload):
    env = dict(os.environ, **ENV_SAN, LD_PRELOAD=preload, PYTHONPATH=ROOT)
    return subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True, text=True,
                          timeout=900)


def _report(r):
    return (r.stdout[-4000:] + "\n" + r.stderr[-4000:])


def test_oracle_pins_under_asan_and_ubsan():
    os.makedirs(OUT, exist_ok=True)
    lib = os.path.join(OUT, "liboracle_san.so")
    cmd = ["gcc", "-O1", "-g", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off", "-fno-fast-math"]
    cmd += GCC_SAN.split() + [os.path.join(ROOT, "oracle", "oracle.c"), "-o", lib, "-lm"]
    subprocess.run(cmd, check=True)
    runtime = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    tests = sorted(glob.glob(os.path.join(ROOT, "tests", "test_oracle_*.py"))) + \
        [os.path.join(ROOT, "tests", "test_codec_rows.py")]
    code = (f"import sys; import oracle.build as b; b.LIB = {lib!r}; import pytest; "
            f"sys.exit(pytest.main(['-q', '-x', '-p', 'no:cacheprovider', '-m', 'not gpu'] + {tests!r}))")
    r = _child(code, runtime)
    assert r.returncode == 0, _report(r)
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, _report(r)


def test_library_host_validation_under_asan_and_ubsan():
    sys.path.insert(0, ROOT)
    from sparse_latent_attention_mla_amd import build as B
    kernels = [os.path.join(B.OBJ, s.replace(".hip", ".o")) for s in B.SOURCES if s.endswith(".hip")]
    if not all(os.path.exists(k) for k in kernels):
        pytest.skip("the library's kernel objects are not built (run __graft_entry__.build())")
    os.makedirs(OUT, exist_ok=True)
    objs = []
    for src in (s for s in B.SOURCES if s.endswith(".cpp")):
        o = os.path.join(OUT, src.replace(".cpp", ".o"))
        subprocess.run([B.HIPCC] + B.FLAGS + HOST_SAN.split() + ["-g", "-x", "hip", "-c",
                                                                  os.path.join(B.CSRC, src), "-o", o],
                       check=True, capture_output=True)
        objs.append(o)
    lib = os.path.join(OUT, "libmla_san.so")
    subprocess.run([B.HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", lib] + objs + kernels, check=True,
                   capture_output=True)
    runtime = glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so")
    if not runtime:
        pytest.skip("clang's AddressSanitizer runtime is not installed")
    code = (f"import sys; import sparse_latent_attention_mla_amd as M; M.LIB_PATH = {lib!r}; import pytest; "
            f"sys.exit(pytest.main(['-q', '-x', '-p', 'no:cacheprovider', '-m', 'not gpu', "
            f"{os.path.join(ROOT, 'tests', 'test_abi.py')!r}]))")
    r = _child(code, runtime[0])
    assert r.returncode == 0, _report(r)
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, _report(r)
