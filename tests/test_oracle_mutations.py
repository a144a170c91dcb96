"""The oracle pins are strong enough: plant one plausible mistake at a time in a
copy of the oracle (CPU only), rebuild it, and check that the pins in
test_oracle_pins.py fail against it.  Each mutation is a mistake someone could
make in that step: an add order, a rounding mode, an exponent bias, a tie-break,
an off-by-one mask, a dropped term."""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ORACLE_C = os.path.join(ROOT, "oracle", "oracle.c")

MUTATIONS = [
    ("O1 add order",
     "float s01 = bf16f(k[d]) + bf16f(k[D + d]);\n                float s23 = bf16f(k[2 * D + d]) + bf16f(k[3 * D + d]);",
     "float s01 = bf16f(k[d]) + bf16f(k[2 * D + d]);\n                float s23 = bf16f(k[D + d]) + bf16f(k[3 * D + d]);"),
    ("O1 partial block by reciprocal", "r = s / 3.0f;", "r = s * (1.0f / 3.0f);"),
    ("O1 partial block over 4", "r = s / 3.0f;", "r = s * 0.25f;"),
    ("O1b truncation", "u = (u + 0x7fffu + keep_odd) & 0xffff0000u;", "u = u & 0xffff0000u;"),
    ("O1b ties away from zero", "u = (u + 0x7fffu + keep_odd) & 0xffff0000u;", "u = (u + 0x8000u) & 0xffff0000u;"),
    ("O1c no saturation", "if (a >= 448.0) return sign | 0x7E;", "if (a >= 480.0) return sign | 0x7F;"),
    ("O1c exponent bias 8", "return sign | (uint8_t)(((E + 7) << 3) | (int)q);",
     "return sign | (uint8_t)(((E + 8) << 3) | (int)q);"),
    ("O1c truncation", "double q = nearbyint((2.0 * m - 1.0) * 8.0);", "double q = floor((2.0 * m - 1.0) * 8.0);"),
    ("O1c subnormal truncation", "const double q = nearbyint(a * 512.0);", "const double q = floor(a * 512.0);"),
    ("O2 a query head dropped", "for (int32_t d = 0; d < D; ++d) qs[d] += (double)bf16f(q[(size_t)j * D + d]);",
     "for (int32_t d = 0; d < D; ++d) qs[d] += j + 1 < g ? (double)bf16f(q[(size_t)j * D + d]) : 0.0;"),
    ("O3 ties to the higher index", "return x->i < y->i ? -1 : (x->i > y->i ? 1 : 0);",
     "return x->i > y->i ? -1 : (x->i < y->i ? 1 : 0);"),
    ("O4 causal mask off by one", "if (pos < L && pos <= t) {", "if (pos < L && pos < t) {"),
    ("O4 scale dropped", "x[i] = scale * acc;", "x[i] = acc;"),
    ("O4 no normalisation", "for (int32_t d = 0; d < D; ++d) oh[d] /= l;", ""),
    ("O4 lse without the max", "lse[h] = m + log(l);", "lse[h] = log(l);"),
    ("O5 weights against the max", "double w = exp(part_lse[(size_t)s * N + r] - lr);",
     "double w = exp(part_lse[(size_t)s * N + r] - M);"),
]


def pins_fail_against(mutated_source: str, workdir: str) -> bool:
    src = os.path.join(workdir, "oracle.c")
    lib = os.path.join(workdir, "liboracle.so")
    with open(src, "w") as f:
        f.write(mutated_source)
    subprocess.run(["gcc", "-O2", "-shared", "-fPIC", "-ffp-contract=off", "-fno-fast-math", src, "-o", lib, "-lm"],
                   check=True, capture_output=True)
    code = ("import sys; sys.path.insert(0, %r); sys.path.insert(0, %r); import oracle; oracle._LIB_PATH = %r; "
            "import pytest; sys.exit(pytest.main(['-q', '-x', '-p', 'no:cacheprovider', %r]))"
            % (ROOT, os.path.join(ROOT, "tests"), lib, os.path.join(ROOT, "tests", "test_oracle_pins.py")))
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, cwd=ROOT, timeout=300)
    return r.returncode == 1  # tests ran and at least one failed


def test_every_planted_mistake_fails_a_pin(tmp_path):
    source = open(ORACLE_C).read()
    jobs = []
    for i, (name, old, new) in enumerate(MUTATIONS):
        assert source.count(old) >= 1, f"mutation site of {name!r} not found"
        d = tmp_path / f"m{i}"
        d.mkdir()
        jobs.append((name, source.replace(old, new, 1), str(d)))
    with ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        caught = list(ex.map(lambda j: pins_fail_against(j[1], j[2]), jobs))
    missed = [name for (name, _, _), c in zip(jobs, caught) if not c]
    assert not missed, f"pins did not catch: {missed}"


def test_unmutated_oracle_passes_the_pins(tmp_path):
    assert not pins_fail_against(open(ORACLE_C).read(), str(tmp_path))
