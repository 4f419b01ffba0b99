"""The oracle's pins must catch plausible mistakes.

Each case plants one mistake (a dropped term, a wrong sign, index or
operand, a strict comparison for an inclusive one ...) in a copy of
oracle/oracle.c, builds it into a temporary library on the CPU, and runs the
pin suite that covers that part against it with GCQ_ORACLE_LIB. The suite
must fail. The real oracle is untouched.
"""
import concurrent.futures as cf
import os
import pathlib
import subprocess
import sys
import tempfile

ROOT = pathlib.Path(__file__).resolve().parent.parent
SRC = ROOT / "oracle" / "oracle.c"
sys.path.insert(0, str(ROOT))
from oracle import CFLAGS  # noqa: E402

T2 = "tests/test_oracle_2bit.py"
TP = "tests/test_oracle_philox.py"
TQ = "tests/test_oracle_qsgd.py"
TT = "tests/test_oracle_ternary.py"

MUTANTS = [
    # 2-bit quantizer
    ("strict_pos", "if (v >= pos_threshold)", "if (v > pos_threshold)", T2),
    ("strict_neg", "if (v <= neg_threshold)", "if (v < neg_threshold)", T2),
    ("lsb_first", "unsigned shift = 30u - 2u * (unsigned)(i % 16);\n        compr",
     "unsigned shift = 2u * (unsigned)(i % 16);\n        compr", T2),
    ("drop_residual_in", "float v = grad[i] + residual[i];\n        uint32_t c = code_of(v, neg_threshold, pos_threshold);\n        float d = value_of(c, neg_threshold, pos_threshold);\n        residual[i] = v - d;\n        unsigned shift",
     "float v = grad[i];\n        uint32_t c = code_of(v, neg_threshold, pos_threshold);\n        float d = value_of(c, neg_threshold, pos_threshold);\n        residual[i] = v - d;\n        unsigned shift", T2),
    ("residual_sign", "residual[i] = v - d;\n        unsigned shift", "residual[i] = v + d;\n        unsigned shift", T2),
    ("residual_not_reduced", "residual[i] = v - d;\n        unsigned shift", "residual[i] = v;\n        unsigned shift", T2),
    ("header_swapped", "compr[0] = bits_of(neg_threshold);\n    compr[1] = bits_of(pos_threshold);\n    compr[2] = bits_of((float)n);\n    for (size_t j = 0;",
     "compr[0] = bits_of(pos_threshold);\n    compr[1] = bits_of(neg_threshold);\n    compr[2] = bits_of((float)n);\n    for (size_t j = 0;", T2),
    ("deq_wrong_sign", "    if (code == 2u)\n        return neg_threshold;",
     "    if (code == 2u)\n        return -neg_threshold;", T2),
    ("sum_drops_worker0", "for (int w = 1; w < W; ++w) {\n            const uint32_t* b = compr[w];\n            float d = value_of(code_at(",
     "acc = 0.0f;\n        for (int w = 1; w < W; ++w) {\n            const uint32_t* b = compr[w];\n            float d = value_of(code_at(", T2),
    ("word_index", "compr[3 + i / 16] |= c << shift;", "compr[2 + i / 16] |= c << shift;", T2),
    # ternary packing
    ("ternary_lsb_first", "bytes[i / 5] = (unsigned char)(bytes[i / 5] + c * pow3[4 - i % 5]);",
     "bytes[i / 5] = (unsigned char)(bytes[i / 5] + c * pow3[i % 5]);", TT),
    ("ternary_decode_order", "unsigned k = 4u - (unsigned)(i % 5);", "unsigned k = (unsigned)(i % 5);", TT),
    ("ternary_digits_unreduced", "return k == 4u ? d : d % 3u;", "return d;", TT),
    ("ternary_no_residual", "        residual[i] = v - d;\n        bytes[i / 5]",
     "        residual[i] = v;\n        bytes[i / 5]", TT),
    ("ternary_header_swapped", "compr[0] = bits_of(neg_threshold);\n    compr[1] = bits_of(pos_threshold);\n    compr[2] = bits_of((float)n);\n    for (size_t j = 3;",
     "compr[0] = bits_of(pos_threshold);\n    compr[1] = bits_of(neg_threshold);\n    compr[2] = bits_of((float)n);\n    for (size_t j = 3;", TT),
    ("ternary_sum_drops_worker0", "for (int w = 1; w < W; ++w) {\n            const uint32_t* b = compr[w];\n            float d = value_of(ternary_digit_at(",
     "acc = 0.0f;\n        for (int w = 1; w < W; ++w) {\n            const uint32_t* b = compr[w];\n            float d = value_of(ternary_digit_at(", TT),
    # Philox
    ("philox_mult_swap", "uint64_t prod_a = (uint64_t)mult_a * (uint64_t)x0;",
     "uint64_t prod_a = (uint64_t)mult_b * (uint64_t)x0;", TP),
    ("philox_no_bump", "k0 += weyl_a;", "k0 += 0u;", TP),
    ("philox_wrong_xor", "uint32_t y0 = hi_b ^ x1 ^ k0;", "uint32_t y0 = hi_a ^ x1 ^ k0;", TP),
    ("philox_9_rounds", "for (int round = 0; round < 10; ++round)",
     "for (int round = 0; round < 9; ++round)", TP),
    # QSGD
    ("u_wrong_shift", "return (float)(r >> 8) * 0x1p-24f;", "return (float)(r >> 9) * 0x1p-24f;", TQ),
    ("level_drops_u", "return (int)floor((double)x + (double)u);", "return (int)floor((double)x);", TQ),
    ("level_rounds_in_fp32", "return (int)floor((double)x + (double)u);",
     "return (int)floorf(x + u);", TQ),
    ("scale_off_by_one", "float x = q * (float)s;", "float x = q * (float)(s + 1);", TQ),
    ("block_index", "philox_word(seed, index / 4, worker, 0u, (unsigned)(index % 4));",
     "philox_word(seed, index, worker, 0u, (unsigned)(index % 4));", TQ),
    ("worker_ignored", "philox_word(seed, index / 4, worker, 0u, (unsigned)(index % 4));",
     "philox_word(seed, index / 4, 0u, 0u, (unsigned)(index % 4));", TQ),
    ("sign_dropped", "return (int8_t)(g < 0.0f ? -m : m);", "return (int8_t)m;", TQ),
    ("maxnorm_no_abs", "m = fmaxf(m, fabsf(grads[w][i]));", "m = fmaxf(m, grads[w][i]);", TQ),
    ("sum_drops_term", "for (int w = 0; w < W; ++w)\n            acc += (int32_t)levels[w][i];",
     "for (int w = 1; w < W; ++w)\n            acc += (int32_t)levels[w][i];", TQ),
    ("deq_times_s", "out[i] = t / (float)s;", "out[i] = t * (float)s;", TQ),
    ("deq_other_order", "float t = norm * (float)sums[i];\n        out[i] = t / (float)s;",
     "float t = (float)sums[i] / (float)s;\n        out[i] = norm * t;", TQ),
    ("deq_in_fp64", "float t = norm * (float)sums[i];\n        out[i] = t / (float)s;",
     "double t = (double)norm * (double)sums[i];\n        out[i] = (float)(t / (double)s);", TQ),
    ("randk_range_n", "uint64_t range = (uint64_t)(n - i);", "uint64_t range = (uint64_t)n;", TQ),
    ("randk_takes_j", "idx[i] = perm[i];", "idx[i] = perm[j];", TQ),
    ("randk_low_word_only", "uint64_t R = ((uint64_t)r[1] << 32) | (uint64_t)r[0];",
     "uint64_t R = (uint64_t)r[0];", TQ),
]


def _run_mutant(name, old, new, target, tmpdir):
    text = SRC.read_text()
    assert text.count(old) == 1, f"mutant {name}: anchor not unique"
    mutated = text.replace(old, new)
    csrc = pathlib.Path(tmpdir) / f"{name}.c"
    lib = pathlib.Path(tmpdir) / f"lib{name}.so"
    csrc.write_text(mutated)
    # keep the oracle's include of its own header working
    flags = [f for f in CFLAGS if f != "-Werror"]
    subprocess.run(["gcc", *flags, f"-I{SRC.parent}", str(csrc), "-o", str(lib), "-lm"],
                   check=True, capture_output=True)
    env = dict(os.environ, GCQ_ORACLE_LIB=str(lib))
    res = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                          "-m", "not gpu", target],
                         cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    return name, res.returncode


def test_every_planted_mistake_fails_a_pin():
    with tempfile.TemporaryDirectory() as tmp:
        with cf.ThreadPoolExecutor(max_workers=4) as ex:
            futs = [ex.submit(_run_mutant, *m, tmp) for m in MUTANTS]
            results = dict(f.result() for f in futs)
    survivors = [n for n, rc in results.items() if rc == 0]
    assert not survivors, f"pins did not catch: {survivors}"
    # rc 1 = tests failed; anything else would be a crash of the harness
    assert all(rc == 1 for rc in results.values()), results

