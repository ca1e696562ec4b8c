"""The pins are not vacuous: plausible mistakes planted in copies of oracle.c fail them.

Each case below edits one spot of a copy of ``oracle/oracle.c`` (the text after an
anchor that names the function), builds it with the oracle's own gcc line, and runs
the pin tests of that function's family against it in a child pytest process (the
oracle loads the library named by MXFP4_ORACLE_LIB).  The pins must fail (pytest exit
status 1).  A control run with an unmodified copy must pass, so a failure comes from
the planted mistake and not from the way the copy is loaded.  The cases run in
parallel on the host's cores.  CPU only.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")
PINS = os.path.join(ROOT, "tests", "test_oracle_pins.py")

# pin families (pytest -k expressions over test_oracle_pins.py)
MX = "not fp8q and not gemm and not wgrad and not nvfp4 and not sr and not philox and not bf16_round"
FP8Q = "fp8q or e4m3"
GEMM = "fp8_gemm or e4m3_value or bf16_round"
WGRAD = "fp8_wgrad"
NVFP4 = "nvfp4 and not sr"

# (mistake, anchor, original text, planted text, pins)
MUTATIONS = [
    ("MX scale offset -1 instead of -2", "static int ue8m0_scale_for_amax(double amax)",
     "(e2 - 1) - 2 + 127", "(e2 - 1) - 1 + 127", MX),
    ("codes packed high nibble first", "void oracle_quantize_block(",
     "(codes[2 * i] | (codes[2 * i + 1] << 4))", "(codes[2 * i + 1] | (codes[2 * i] << 4))", MX),
    ("codes unpacked high nibble first", "static int code_at(",
     "(k & 1) ? (b >> 4) : (b & 15)", "(k & 1) ? (b & 15) : (b >> 4)", MX),
    ("ties rounded away from zero", "static int minifloat_round_nearest_even(",
     "if (frac > 0.5 || (frac == 0.5 && (q & 1)))", "if (frac >= 0.5)", MX),
    ("E2M1 saturating at 4 instead of 6", "static int e2m1_encode(double y)",
     "minifloat_round_nearest_even(y, 1, 1, 7)", "minifloat_round_nearest_even(y, 1, 1, 6)", MX),
    ("E2M1 subnormal read as 1 instead of 0.5", "static double e2m1_magnitude(int code)",
     "return ldexp((double)m, -1);", "return ldexp((double)m, 0);", MX),
    ("sign of a zero code dropped", "void oracle_quantize_block(",
     "if (bf16_negative(x[i]))\n            c |= 8;", "if (bf16_negative(x[i]) && (c & 7))\n            c |= 8;", MX),
    ("sub-block shift by S - s in the wrong direction", "static uint8_t fp8_of_code(",
     "e2m1_magnitude(c & 7), s - S)", "e2m1_magnitude(c & 7), S - s)", MX),
    ("FP8 row block scale = min of the four MX scales", "void oracle_fp8_rows(",
     "if (srow[4 * b + j] > S)", "if (j == 0 || srow[4 * b + j] < S)", MX),
    ("column output transposed back (row-major index)", "void oracle_fp8_cols(",
     "outT[k * Mg + m] = fp8_of_code", "outT[m * K + k] = fp8_of_code", MX),
    ("column block scale from the block's first row only", "void oracle_fp8_cols(",
     "for (int64_t m = mlo; m < mhi; ++m) {\n                int s = scales",
     "for (int64_t m = mlo; m < mlo + 1; ++m) {\n                int s = scales", MX),
    ("column scales of expert g placed with floor(M_h / 128) blocks", "void oracle_fp8_cols(",
     "Bg += ((int64_t)offs[h + 1] - offs[h] + 127) / 128;", "Bg += ((int64_t)offs[h + 1] - offs[h]) / 128;", MX),
    ("E4M3 block scale with emax 7 instead of 8", "static int ue8m0_scale_for_amax_e4m3(",
     "(e2 - 1) - 8 + 127", "(e2 - 1) - 7 + 127", FP8Q),
    ("E4M3 not saturating at 448", "static int e4m3_encode(double v)",
     "minifloat_round_nearest_even(v, 3, 7, 0x7E)", "minifloat_round_nearest_even(v, 3, 7, 0x7F)", FP8Q),
    ("backward column output transposed back", "void oracle_fp8q_cols(",
     "outT[k * Mg + m] = (uint8_t)e;", "outT[m * K + k] = (uint8_t)e;", FP8Q),
    ("backward column amax from the block's first row only", "void oracle_fp8q_cols(",
     "for (int64_t m = mlo; m < mhi; ++m) {\n                double a", "for (int64_t m = mlo; m < mlo + 1; ++m) {\n                double a",
     FP8Q),
    ("GEMM activation scaled by the weight's scale", "void oracle_fp8_gemm_at(",
     "ldexp(e4m3_value(ar[k]), (int)sar[k / 128] - 127)", "ldexp(e4m3_value(ar[k]), (int)swr[k / 128] - 127)", GEMM),
    ("GEMM row routed to the next expert at its first row", "void oracle_fp8_gemm_at(",
     "(int64_t)offs[g + 1] <= m", "(int64_t)offs[g + 1] < m", GEMM),
    ("BF16 rounding ties away from zero", "static double round_half_even(double q)",
     "if (r > 0.5 || (r == 0.5 && fmod(f, 2.0) != 0.0))", "if (r >= 0.5)", GEMM),
    ("E4M3 subnormal quantum 2^-10", "static double e4m3_value(uint8_t b)",
     "ldexp((double)m, -9)", "ldexp((double)m, -10)", GEMM),
    ("wgrad scale blocks of 256 tokens", "void oracle_fp8_wgrad_at(",
     "int64_t b = m / 128;", "int64_t b = m / 256;", WGRAD),
    ("wgrad block count floor instead of ceiling", "static int64_t blocks_before(",
     "b += ((int64_t)offs[e + 1] - offs[e] + 127) / 128;", "b += ((int64_t)offs[e + 1] - offs[e]) / 128;", WGRAD),
    ("wgrad X row stride dropped", "void oracle_fp8_wgrad_at(",
     "xT + K * m0 + k * Mg;", "xT + K * m0 + k;", WGRAD),
    ("wgrad X scaled by the gradient's scale", "void oracle_fp8_wgrad_at(",
     "(int)xT_scales[K * (Bg + b) + k] - 127", "(int)dyT_scales[N * (Bg + b) + n] - 127", WGRAD),
    ("NVFP4 block scale from amax / 4", "void oracle_nvfp4_block(",
     "float sb = amax / 6.0f;", "float sb = amax / 4.0f;", NVFP4),
    ("NVFP4 tensor scale 2687 / amax", "static float nvfp4_encode_scale(float amax)",
     "float t = 2688.0f / amax;", "float t = 2687.0f / amax;", NVFP4),
    ("NVFP4 element product perturbed", "void oracle_nvfp4_block(",
     "float y = (float)bf16_value(x[i]) * e;", "float y = (float)bf16_value(x[i]) * e * 1.0001f;", NVFP4),
]


def plant(text: str, anchor: str, old: str, new: str) -> str:
    at = text.find(anchor)
    assert at >= 0, f"anchor not in oracle.c: {anchor!r}"
    i = text.find(old, at)
    assert i >= 0, f"text not found after {anchor!r}: {old!r}"
    return text[:i] + new + text[i + len(old):]


def run_pins(tmp_path, name: str, source: str, kexpr: str) -> subprocess.CompletedProcess:
    d = tmp_path / name
    d.mkdir()
    src = d / "oracle.c"
    src.write_text(source)
    lib = oracle.compile_oracle(str(src), str(d / "liboracle.so"))
    env = dict(os.environ, MXFP4_ORACLE_LIB=lib, OMP_NUM_THREADS="1")
    return subprocess.run(
        [sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider", PINS, "-k", kexpr],
        cwd=ROOT, env=env, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, timeout=600)


def workers() -> int:
    try:
        return max(1, min(8, len(os.sched_getaffinity(0))))
    except AttributeError:  # pragma: no cover
        return 4


def test_every_planted_mistake_fails_a_pin(tmp_path):
    text = open(SRC).read()
    jobs = [("control", text, "quantize_matches or fp8q_matches or fp8_gemm_brute or fp8_wgrad_brute")]
    for i, (what, anchor, old, new, kexpr) in enumerate(MUTATIONS):
        jobs.append((f"m{i:02d}", plant(text, anchor, old, new), kexpr))
    with ThreadPoolExecutor(workers()) as pool:
        results = list(pool.map(lambda j: run_pins(tmp_path, *j), jobs))
    control = results[0]
    assert control.returncode == 0, "unmodified copy fails its pins:\n" + control.stdout.decode()[-3000:]
    missed = []
    for (what, *_), r in zip(MUTATIONS, results[1:]):
        if r.returncode != 1:
            missed.append(f"{what}: pytest exit {r.returncode}\n{r.stdout.decode()[-600:]}")
    assert not missed, "mistakes no pin catches:\n" + "\n".join(missed)


@pytest.mark.parametrize("what,anchor,old,new,kexpr", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_each_mistake_still_applies_to_oracle_c(what, anchor, old, new, kexpr):
    """The planted text still exists where the case says (oracle.c edits keep it)."""
    text = open(SRC).read()
    out = plant(text, anchor, old, new)
    assert out != text and len(out) - len(text) == len(new) - len(old)
