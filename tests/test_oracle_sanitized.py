"""The oracle under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

The oracle's C source is compiled with gcc and -fsanitize=address,undefined (no recovery from undefined
behaviour), and every pin the planted-mistake test runs (E4M3, the quantizers, the GEMM and the grouped GEMM,
the dequantization, routing and the gather, FP4, per-channel, E5M6 and SwiGLU) runs against that build in a
child process with the ASan runtime loaded first.  Any out-of-bounds access (heap, stack or the routing's
variable-length arrays), use after free or undefined operation aborts the child with a report, which fails
the test.  The real oracle build is not touched.
"""
import os
import subprocess
import sys

import pytest

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)

SAN_FLAGS = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer", "-g"]

CHILD = r"""
import sys
sys.path.insert(0, {root!r})
sys.path.insert(0, {tests!r})
import oracle
import test_oracle_mutations as tm
lib = oracle.load({lib!r})
n = 0
for fn, kw in tm.pins():
    fn(lib, **kw)
    n += 1
print(f"sanitized oracle: {{n}} pins passed", flush=True)
"""


def _runtime(name):
    p = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    return p if os.path.isabs(p) and os.path.exists(p) else None


@pytest.mark.timeout(900)
def test_pins_pass_under_address_and_undefined_sanitizers(tmp_path):
    asan = _runtime("libasan.so")
    if asan is None:
        pytest.skip("gcc's AddressSanitizer runtime is not installed")
    lib_path = str(tmp_path / "liboracle_fp8q_san.so")
    src = os.path.join(os.path.dirname(oracle.__file__), "fp8q_oracle.c")
    subprocess.run(["gcc", *oracle.CFLAGS, *SAN_FLAGS, src, "-o", lib_path, "-lm"], check=True)
    env = dict(os.environ)
    # the sanitizer runtime must be the first library loaded; anything already preloaded stays after it
    env["LD_PRELOAD"] = asan + (":" + env["LD_PRELOAD"] if env.get("LD_PRELOAD") else "")
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1"   # the interpreter's own allocations are not leaks
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    code = CHILD.format(root=ROOT, tests=HERE, lib=lib_path)
    r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True, timeout=850)
    tail = (r.stdout + r.stderr)[-4000:]
    assert r.returncode == 0, f"sanitized oracle run failed (exit {r.returncode}):\n{tail}"
    assert "pins passed" in r.stdout, tail
    for word in ("AddressSanitizer", "runtime error:"):
        assert word not in r.stderr, tail
