"""Host-side sanitizer runs of the C oracle and of the C-ABI library.

AddressSanitizer and UndefinedBehaviorSanitizer builds (host code only; the
GPU code of the library is built as usual) are made in a temporary folder:
the oracle with gcc, the library with hipcc taking the sanitizer flags on its
host side only.  The oracle's pins (tests/test_oracle_pins.py) then run
against the sanitized oracle, and the C-ABI checks (tests/test_abi.py, which
need no GPU: every call is rejected on the host before any launch) against
the sanitized library, each in a child process with the matching sanitizer
runtime preloaded (gcc's for the oracle, the ROCm clang's for the library).
Any report fails the child.  Building the library takes a few minutes, so
this runs only with DSA_SANITIZE=1."""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

pytestmark = pytest.mark.skipif(os.environ.get("DSA_SANITIZE") != "1",
                                reason="builds sanitized libraries; set DSA_SANITIZE=1")

_SAN = ["address", "undefined"]
_OPTS = {"ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1",
         "UBSAN_OPTIONS": "print_stacktrace=1:halt_on_error=1"}


def _child(env_extra, *test_args):
    env = dict(os.environ, **_OPTS, **env_extra)
    env.pop("DSA_SANITIZE", None)
    # -s: the sanitizers' reports go straight to the child's stderr
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-s", "-p", "no:cacheprovider", "-m", "not gpu",
                        *test_args],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "runtime error" not in out and "ERROR: AddressSanitizer" not in out, out[-4000:]
    return out


def test_oracle_pins_under_asan_ubsan(tmp_path):
    import oracle
    lib = oracle.build(out=str(tmp_path / "liboracle_san.so"),
                       extra=[f"-fsanitize={s}" for s in _SAN] +
                             ["-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer", "-g"])
    libasan = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    out = _child({"LD_PRELOAD": libasan, "DSA_ORACLE_LIB": lib}, "tests/test_oracle_pins.py")
    print(out.strip().splitlines()[-1])


def test_c_abi_validation_under_asan_ubsan(tmp_path):
    from sparse_attention_long_08_amd import _builder
    host = []
    for s in _SAN:
        host += ["-Xarch_host", f"-fsanitize={s}"]
    host += ["-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]
    lib = _builder.build(extra=host, out=str(tmp_path / "libdsa_san.so"), link_extra=["-shared-libsan"] + host)
    rt = glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so")
    assert rt, "ROCm clang's ASan runtime not found"
    out = _child({"LD_PRELOAD": rt[0], "DSA_LIB_PATH": lib}, "tests/test_abi.py")
    print(out.strip().splitlines()[-1])
