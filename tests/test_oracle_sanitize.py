"""The oracle under AddressSanitizer and UndefinedBehaviorSanitizer (host code
only): a C program runs every entry point on small seeded inputs with exactly
sized buffers, including an empty batch, one token, 512 experts with top-16,
alignment larger than every count, out-of-range expert ids, all quant modes
and rows holding NaN and infinities (float-to-integer conversions are checked
too: -fsanitize=float-cast-overflow)."""
import os
import shutil
import subprocess
import tempfile

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


def test_oracle_under_asan_and_ubsan():
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not available")
    with tempfile.TemporaryDirectory() as d:
        exe = os.path.join(d, "oracle_sanitize")
        cmd = [gcc, "-std=c11", "-O1", "-g", "-fno-omit-frame-pointer", "-ffp-contract=off",
               "-fsanitize=address,undefined,float-cast-overflow", "-fno-sanitize-recover=all",
               os.path.join(HERE, "oracle_sanitize_main.c"), os.path.join(ROOT, "oracle", "moe_oracle.c"),
               "-lm", "-o", exe]
        b = subprocess.run(cmd, capture_output=True, text=True)
        if b.returncode != 0 and "asan" in b.stderr.lower() and "cannot find" in b.stderr.lower():
            pytest.skip("sanitizer runtime not installed")
        assert b.returncode == 0, b.stderr
        env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:verify_asan_link_order=0",
                   UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
        r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
        assert r.returncode == 0, r.stdout + r.stderr
        assert "ok" in r.stdout
