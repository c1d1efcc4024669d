"""The pins must catch plausible mistakes in the oracle.

Each case plants one mistake in a copy of oracle/zq_oracle.c (a dropped term,
a wrong sign, a transposed index, a wrong field order, a wrong rounding rule),
builds the copy, and runs tests/test_oracle_pins.py against it in a fresh
process: that run must fail. CPU only; nothing here touches the GPU path.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# (name, exact text in zq_oracle.c, replacement)
MUTATIONS = [
    ("nibble order reversed",
     "byte |= ((unsigned)q & mask) << (i * bits);",
     "byte |= ((unsigned)q & mask) << ((per - 1 - i) * bits);"),
    ("codes truncated instead of rounded to nearest even",
     "q = nearbyint(v / s);", "q = trunc(v / s);"),
    ("scale index transposed",
     "return r * (k / group) + c / group;", "return r * (k / group) + (c % (k / group));"),
    ("sign extension off by one",
     "if (f >= (1 << (bits - 1))) f -= (1 << bits);", "if (f > (1 << (bits - 1))) f -= (1 << bits);"),
    ("first term of the dot product dropped",
     "acc += zqo_widen(x, x_dtype, mi * ldx + c) * wdeq;",
     "acc += zqo_widen(x, x_dtype, mi * ldx + c) * wdeq * (c > 0);"),
    ("scale never raised when fp16 rounding would clip",
     "if (zqo_f16_to_f64(s16) * qmax < a) s16 = (uint16_t)(s16 + 1);", ""),
    ("fp16 narrowing rounds half away from zero",
     "double r = nearbyint(ldexp(a, -qexp));", "double r = floor(ldexp(a, -qexp) + 0.5);"),
    ("output sign flipped",
     "y[mi * ldy + r] = acc;", "y[mi * ldy + r] = -acc;"),
    ("activation row and weight row swapped",
     "acc += zqo_widen(x, x_dtype, mi * ldx + c) * wdeq;",
     "acc += zqo_widen(x, x_dtype, (r % (m > 0 ? m : 1)) * ldx + c) * wdeq;"),
    ("bf16 exponent bias off by one",
     "v = ldexp((double)(128 + f), e - 127 - 7);", "v = ldexp((double)(128 + f), e - 126 - 7);"),
    ("asymmetric: zero point dropped from the product",
     "* zqo_f16_to_f64(scales[si]) +\n                      zqo_f16_to_f64(zeros[si]);",
     "* zqo_f16_to_f64(scales[si]);"),
    ("asymmetric: scale divides by 2^b instead of 2^b - 1",
     "uint16_t s16 = zqo_f64_to_f16((hi - lo) / qmax);", "uint16_t s16 = zqo_f64_to_f16((hi - lo) / (qmax + 1));"),
    ("asymmetric: lowest code clamped to 1",
     "if (q < 0.0) q = 0.0;", "if (q < 1.0) q = 1.0;"),
    ("asymmetric: unsigned field masked one bit short",
     "return (byte >> ((c % per) * bits)) & ((1u << bits) - 1u);",
     "return (byte >> ((c % per) * bits)) & ((1u << (bits - 1)) - 1u);"),
]


@pytest.mark.parametrize("name,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_pins_catch_planted_mistake(tmp_path, name, old, new):
    dst = tmp_path / "tree"
    (dst / "oracle").mkdir(parents=True)
    for f in ("zq_oracle.c", "zq_oracle.h", "oracle.py", "__init__.py"):
        src = os.path.join(ROOT, "oracle", f)
        if os.path.exists(src):
            shutil.copy(src, dst / "oracle" / f)
    shutil.copytree(os.path.join(ROOT, "tests"), dst / "tests",
                    ignore=shutil.ignore_patterns("__pycache__", "test_oracle_mutations.py", "test_gpu_*"))
    shutil.copytree(os.path.join(ROOT, "weight_quantized_amd"), dst / "weight_quantized_amd",
                    ignore=shutil.ignore_patterns("__pycache__", "_build", "csrc", "*.so"))
    shutil.copy(os.path.join(ROOT, "pytest.ini"), dst / "pytest.ini")
    c = dst / "oracle" / "zq_oracle.c"
    text = c.read_text()
    assert old in text, f"mutation site not found: {old}"
    c.write_text(text.replace(old, new, 1))  # the first site (the symmetric functions come first)
    env = dict(os.environ, PYTHONPATH=str(dst))
    r = subprocess.run([sys.executable, "-m", "pytest", "tests/test_oracle_pins.py", "-x", "-q",
                        "-p", "no:cacheprovider"], cwd=dst, env=env, capture_output=True, text=True,
                       timeout=600)
    assert r.returncode == 1, f"planted mistake '{name}' was not caught:\n{r.stdout[-2000:]}"
