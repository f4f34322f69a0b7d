"""The oracle's C code under AddressSanitizer and UndefinedBehaviorSanitizer
(CPU only): a sanitized build of oracle/ngram_oracle.c runs every oracle pin
test in a subprocess, and any out-of-bounds access, use after free or
undefined operation aborts it."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "ngram_oracle.c")
PINS = ["tests/test_oracle_hash.py", "tests/test_oracle_sum_gate.py", "tests/test_oracle_grad.py",
        "tests/test_oracle_mxfp4.py", "tests/test_oracle_norm_gate.py"]


def _runtime(name):
    r = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True)
    p = r.stdout.strip()
    return p if os.path.isabs(p) and os.path.exists(p) else None


@pytest.mark.skipif(_runtime("libasan.so") is None, reason="gcc's AddressSanitizer runtime is not installed")
def test_oracle_pins_pass_under_asan_and_ubsan(tmp_path):
    lib = tmp_path / "liboracle_san.so"
    subprocess.run(["gcc", "-std=c11", "-O1", "-g", "-ffp-contract=off", "-fno-omit-frame-pointer",
                    "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fPIC", "-shared",
                    "-o", str(lib), SRC, "-lm"], check=True)
    env = dict(os.environ, ORACLE_LIB=str(lib), LD_PRELOAD=_runtime("libasan.so"),
               ASAN_OPTIONS="detect_leaks=0:alloc_dealloc_mismatch=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider", "-p", "no:faulthandler", "--capture=no"] + PINS,
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=1200)
    assert r.returncode == 0, f"sanitized oracle failed:\n{r.stdout[-3000:]}\n{r.stderr[-3000:]}"
    assert "passed" in r.stdout


@pytest.mark.skipif(_runtime("libasan.so") is None, reason="gcc's AddressSanitizer runtime is not installed")
def test_the_sanitized_run_catches_a_planted_out_of_bounds_read(tmp_path):
    """A copy of the oracle whose bf16 sum reads 100000 rows past its row
    aborts the same pin run."""
    before = "acc = acc + oracle_bf16_to_f32(T[r * d + j]);"
    src = open(SRC).read()
    assert src.count(before) == 1
    bad = tmp_path / "bad.c"
    bad.write_text(src.replace(before, "acc = acc + oracle_bf16_to_f32(T[r * d + j + d * 100000]);"))
    lib = tmp_path / "libbad.so"
    subprocess.run(["gcc", "-std=c11", "-O1", "-g", "-ffp-contract=off", "-fno-omit-frame-pointer",
                    "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fPIC", "-shared",
                    "-o", str(lib), str(bad), "-lm"], check=True)
    env = dict(os.environ, ORACLE_LIB=str(lib), LD_PRELOAD=_runtime("libasan.so"),
               ASAN_OPTIONS="detect_leaks=0:alloc_dealloc_mismatch=0:abort_on_error=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider", "-p", "no:faulthandler", "--capture=no",
                        "tests/test_oracle_sum_gate.py"], cwd=ROOT, env=env, capture_output=True, text=True,
                       timeout=600)
    assert r.returncode != 0
    assert "AddressSanitizer" in r.stdout + r.stderr
