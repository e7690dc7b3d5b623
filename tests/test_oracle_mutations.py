"""The oracle's pins catch plausible mistakes (CPU only).

Each case copies oracle/zero_oracle.c to a temporary directory, plants ONE
mistake by an exact textual substitution, builds it with the oracle's own
flags, and runs the oracle pin suite (tests/test_oracle_*.py) against that
build through ZERO_ORACLE_LIB.  The suite must fail for every mutant and
pass for the unmodified copy.  The mistakes are of the kinds a reader could
make when writing the oracle from the pages and the textbook: a dropped or
misplaced term, a wrong sign, a wrong index or mask, a wrong rounding rule,
an off-by-one in the layout, a missing clamp.  None of them reads or writes
out of bounds.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "zero_oracle.c")
# cheapest first: with -x a mutant stops at its first failing pin
PIN_FILES = [os.path.join(ROOT, "tests", f) for f in
             ("test_oracle_plan.py", "test_oracle_step.py", "test_oracle_adam.py",
              "test_oracle_cast.py")]
CFLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math"]

MUTATIONS = [
    ("bias correction of m dropped",
     "float c_step = (float)(lr / (1.0 - pow(b1, (double)t)));", "float c_step = (float)lr;"),
    ("bias correction of v dropped",
     "float c_rsbc2 = (float)(1.0 / sqrt(1.0 - pow(b2, (double)t)));", "float c_rsbc2 = 1.0f;"),
    ("bias correction of v without its square root",
     "float c_rsbc2 = (float)(1.0 / sqrt(1.0 - pow(b2, (double)t)));",
     "float c_rsbc2 = (float)(1.0 / (1.0 - pow(b2, (double)t)));"),
    ("bias correction of m one step ahead",
     "float c_step = (float)(lr / (1.0 - pow(b1, (double)t)));",
     "float c_step = (float)(lr / (1.0 - pow(b1, (double)(t + 1))));"),
    ("momentum weighs the gradient by beta1",
     "float c_omb1 = (float)(1.0 - b1);", "float c_omb1 = (float)b1;"),
    ("decoupled decay applied to the updated weight",
     "p = p * c_decay - c_step * u;", "p = (p - c_step * u) * c_decay;"),
    ("eps inside the square root",
     "float d = sqrtf(vk) * c_rsbc2 + c_eps;", "float d = sqrtf(vk + c_eps) * c_rsbc2;"),
    ("decoupled decay with the wrong sign",
     "(float)(1.0 - lr * wd)", "(float)(1.0 + lr * wd)"),
    ("beta2 used for the momentum",
     "float mk = c_b1 * m[k] + c_omb1 * g;", "float mk = c_b2 * m[k] + c_omb2 * g;"),
    ("gradient not squared in the variance",
     "float vk = c_b2 * v[k] + c_omb2 * (g * g);", "float vk = c_b2 * v[k] + c_omb2 * g;"),
    ("loss scale multiplied instead of divided",
     "float c_inv = (float)(1.0 / scale);", "float c_inv = (float)scale;"),
    ("L2 term subtracted",
     "if (!adamw) g = g + c_wd * p;", "if (!adamw) g = g - c_wd * p;"),
    ("update added instead of subtracted",
     "p = p * c_decay - c_step * u;", "p = p * c_decay + c_step * u;"),
    ("rounding down instead of to nearest",
     "if (rem > 0.5) kr = fl + 1.0;", "if (rem > 0.5) kr = fl;"),
    ("ties away from zero instead of to even",
     "else kr = (fmod(fl, 2.0) == 0.0) ? fl : fl + 1.0;", "else kr = fl + 1.0;"),
    ("fp16 exponent mask one bit short",
     "return ((h >> 10) & 0x1F) == 0x1F;", "return ((h >> 10) & 0x1E) == 0x1E;"),
    ("bf16 exponent field misplaced",
     "return ((h >> 7) & 0xFF) == 0xFF;", "return ((h >> 8) & 0x7F) == 0x7F;"),
    ("fp16 subnormal scale off by one binade",
     "mag = ldexpf((float)frac, -24);", "mag = ldexpf((float)frac, -25);"),
    ("padding of the flat shard not zeroed",
     "for (int64_t k = real; k < S; ++k) flat[k] = 0;", ""),
    ("flat length padded one unit too far",
     "int64_t P_pad = ((P + unit - 1) / unit) * unit;", "int64_t P_pad = (P / unit + 1) * unit;"),
    ("real length off by one",
     "if (P > begin) real = (P < end ? P : end) - begin;",
     "if (P > begin) real = (P < end ? P : end) - begin - 1;"),
    ("buckets built from the first tensor",
     "for (int64_t i = n - 1; i >= 0; --i) {", "for (int64_t i = 0; i < n; ++i) {"),
    ("bucket closed only above B",
     "if (fill >= B) {", "if (fill > B) {"),
    ("stage-2 bytes count the gradients twice",
     "scal[8] = 2 * P + 14 * S;", "scal[8] = 2 * P + 16 * S;"),
    ("no floor on the backed-off scale",
     "*scale = s < min_scale ? min_scale : s;", "*scale = s;"),
    ("clean-step count not reset after growth",
     "*scale = *scale * growth;\n        *good = 0;", "*scale = *scale * growth;"),
    ("overflow test skipped",
     "if (oracle_nonfinite(flat, n, gdt)) return 1;", "if (0) return 1;"),
    ("parameters always cast to bf16",
     "param[begin + k - base] = oracle_float_to_half(master[k], pdt);",
     "param[begin + k - base] = oracle_float_to_half(master[k], OR_BF16);"),
    ("fp32 exponent mask one bit short",
     "return ((u >> 23) & 0xFFu) == 0xFFu;", "return ((u >> 23) & 0x7Fu) == 0x7Fu;"),
    ("fp32 gradients read as halves",
     "    if (gdt == OR_F32) {\n        uint32_t u;", "    if (0) {\n        uint32_t u;"),
    ("fp32 gradient read at the wrong offset",
     "memcpy(&u, (const unsigned char*)flat + 4 * k, 4);",
     "memcpy(&u, (const unsigned char*)flat + 2 * k, 4);"),
    ("fp32 flat padding not zeroed",
     "for (int64_t k = real; k < S; ++k) flat[k] = 0u;", ""),
    ("parameter cast of the wrong master element",
     "param[begin + k - base] = oracle_float_to_half(master[k], pdt);",
     "param[begin + k - base] = oracle_float_to_half(master[real - 1 - k], pdt);"),
]


def _build(tmp_path, text, name):
    src = tmp_path / f"{name}.c"
    src.write_text(text)
    out = tmp_path / f"{name}.so"
    subprocess.run(["gcc", *CFLAGS, str(src), "-lm", "-o", str(out)], check=True)
    return str(out)


def _pins_pass(lib):
    env = dict(os.environ, ZERO_ORACLE_LIB=lib)
    # the exhaustive 2^32 cast checks are left out here: the structured sweeps
    # before them catch the rounding mutants in a fraction of the time.  So is
    # the GPT-2-small partitioned-equals-unpartitioned check (about 40 s): the
    # same invariant runs on the tiny model in every run, and no change to
    # the arithmetic can break it.
    r = subprocess.run([sys.executable, "-m", "pytest", *PIN_FILES, "-x", "-q",
                        "-k", "not all_2_32 and not gpt2_small", "-p", "no:cacheprovider"],
                       cwd=ROOT, env=env,
                       capture_output=True, text=True, timeout=900)
    return r.returncode == 0, r.stdout[-2000:]


def test_unmodified_copy_passes_the_pins(tmp_path):
    ok, out = _pins_pass(_build(tmp_path, open(SRC).read(), "control"))
    assert ok, out


def test_every_planted_mistake_fails_a_pin(tmp_path):
    from concurrent.futures import ThreadPoolExecutor
    text = open(SRC).read()
    libs = []
    for i, (name, old, new) in enumerate(MUTATIONS):
        assert text.count(old) == 1, f"mutation site not unique or missing: {old!r}"
        libs.append((name, _build(tmp_path, text.replace(old, new), f"mutant{i}")))
    workers = max(1, min(4, (os.cpu_count() or 1) // 2))
    with ThreadPoolExecutor(workers) as pool:
        results = list(pool.map(lambda nl: (nl[0], _pins_pass(nl[1])[0]), libs))
    survivors = [name for name, ok in results if ok]
    assert not survivors, f"no pin caught: {survivors}"
