"""The host C code the parity checks rest on -- the oracle and the seeded input
generator -- rebuilt with AddressSanitizer and UndefinedBehaviorSanitizer, then
run through the oracle's pins and the input-recipe tests (CPU only).  An
out-of-bounds access, a use after free, a signed overflow or a bad shift in
either library fails this test, where in the normal build it could silently
change an expected value."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
TESTS = os.path.join(ROOT, "tests")


def _runtime(name: str) -> str:
    path = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else ""


def test_oracle_and_generator_clean_under_sanitizers(tmp_path):
    asan = _runtime("libasan.so")
    if not asan:
        pytest.skip("gcc's AddressSanitizer runtime is not installed")
    flags = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
             "-shared", "-fPIC", "-pthread", "-ffp-contract=off", "-fno-fast-math"]
    libs = {}
    for pkg, src, lib in (("oracle", "oracle.c", "liboracle.so"), ("synth", "synth.c", "libsynth.so")):
        out = str(tmp_path / lib)
        subprocess.run(["gcc", *flags, os.path.join(ROOT, pkg, src), "-o", out, "-lm"], check=True,
                       capture_output=True)
        libs[pkg] = out
    code = ("import sys; sys.path.insert(0, %r); sys.path.insert(0, %r); import oracle, synth; "
            "oracle._LIB_PATH = %r; synth._LIB_PATH = %r; import pytest; "
            "sys.exit(pytest.main(['-q', '-x', '-p', 'no:cacheprovider', '-p', 'no:xdist', %r, %r]))"
            % (ROOT, TESTS, libs["oracle"], libs["synth"], os.path.join(TESTS, "test_oracle_pins.py"),
               os.path.join(TESTS, "test_synth_and_constants.py")))
    # the reports go to files of their own (pytest captures stderr inside the run),
    # and a sanitizer stop exits with its own code
    log = str(tmp_path / "sanitizer")
    env = dict(os.environ, LD_PRELOAD=asan,
               ASAN_OPTIONS=f"detect_leaks=0:halt_on_error=1:exitcode=86:log_path={log}",
               UBSAN_OPTIONS=f"halt_on_error=1:print_stacktrace=1:exitcode=86:log_path={log}")
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, cwd=ROOT, env=env, timeout=900)
    reports = "".join(open(tmp_path / f).read() for f in sorted(os.listdir(tmp_path)) if f.startswith("sanitizer"))
    assert not reports and r.returncode != 86, reports[-6000:]
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
