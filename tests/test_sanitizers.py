"""The host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU
only, no GPU): the C oracle and the library's host side (argument checks,
workspace sizing, the launch set-up that runs before any kernel) are built
instrumented -- the oracle with clang -fsanitize=address,undefined, the HIP
library with the same flags on its host pass only -- and the oracle's pins
and the C-ABI checks run against those builds in a child process with
clang's sanitizer runtime preloaded.  Any report aborts the child."""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
RUNTIME = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))


@pytest.mark.skipif(not RUNTIME, reason="clang's ASan runtime is not installed")
def test_oracle_and_abi_clean_under_asan_and_ubsan():
    import oracle
    from vertical_slash_sparse_amd import build as vs_build
    oracle.build(force=True, sanitize=True)
    vs_build.build(sanitize=True)
    env = dict(os.environ)
    env.update({
        "VS_SANITIZE": "1",
        "LD_PRELOAD": RUNTIME[-1],
        # Python itself keeps memory to the end; leaks are not what is checked
        "ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1",
        "UBSAN_OPTIONS": "print_stacktrace=1:halt_on_error=1",
    })
    res = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-s", "-p", "no:cacheprovider",
                          "tests/test_oracle.py", "tests/test_oracle_blocks.py", "tests/test_abi.py"],
                         cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    tail = (res.stdout + res.stderr)[-4000:]
    assert res.returncode == 0, tail
    assert "runtime error" not in res.stdout + res.stderr, tail
    assert "AddressSanitizer" not in res.stdout + res.stderr, tail
