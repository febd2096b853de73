"""The oracle's pins catch plausible mistakes (CPU only).

Each case below plants one mistake in a copy of ``oracle/oracle.c`` (a dropped
term, a wrong sign, index or stride, a transposed operand, a wrong rounding
rule, a wrong codec constant), builds that copy into a temporary library, and
runs the oracle pin suite (tests/test_oracle_gemm.py, tests/test_oracle_codecs.py,
tests/test_oracle_epilogue.py, tests/test_oracle_attention.py, tests/test_oracle_fp8.py)
against it in a child process.  The suite must fail for every mutant; a mutant
that survives is a mistake the pins would not see.
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")

# (name, exact text in oracle.c, replacement)
MUTANTS = [
    ("A transposed", "load_fp(j->A, j->in_type, oa + at(j->layout_a, i, k, j->lda))",
     "load_fp(j->A, j->in_type, oa + at(j->layout_a, k, i, j->lda))"),
    ("B transposed", "accf[c] += a * load_fp(j->B, j->in_type, ob + at(j->layout_b, k, c, j->ldb))",
     "accf[c] += a * load_fp(j->B, j->in_type, ob + at(j->layout_b, c, k, j->ldb))"),
    ("int B transposed", "load_int(j->B, OR_I8, ob + at(j->layout_b, k, c, j->ldb))",
     "load_int(j->B, OR_I8, ob + at(j->layout_b, c, k, j->ldb))"),
    ("selected elements: A transposed", "load_fp(A, in_type, oa + at(layout_a, i, k, lda))",
     "load_fp(A, in_type, oa + at(layout_a, k, i, lda))"),
    ("selected elements: batch stride of B ignored", "ob = b * stride_b,", "ob = 0 * stride_b,"),
    ("selected elements: C dropped", "addend += load_fp(C, out_type", "addend += 0.0 * load_fp(C, out_type"),
    ("selected elements: epilogue skipped", "store_out(out, out_type, s, epilogue(&j, b, i, c, acc, addend));",
     "store_out(out, out_type, s, acc + addend);"),
    ("selected elements: int k dropped", "for (int64_t k = 0; k < K; ++k)\n                acc += load_int",
     "for (int64_t k = 1; k < K; ++k)\n                acc += load_int"),
    ("column-major ignored", "r * ld + c : r + c * ld", "r * ld + c : r * ld + c"),
    ("C dropped", "epilogue(j, b, i, c, accf[c], addend)", "epilogue(j, b, i, c, accf[c], 0.0)"),
    ("int C subtracted", "v += load_int(j->C", "v -= load_int(j->C"),
    ("last k dropped", "for (int64_t k = 0; k < j->K; ++k) {\n                const double",
     "for (int64_t k = 0; k + 1 < j->K; ++k) {\n                const double"),
    ("first int k dropped", "for (int64_t k = 0; k < j->K; ++k) {\n                const int64_t",
     "for (int64_t k = 1; k < j->K; ++k) {\n                const int64_t"),
    ("product sign", "accf[c] += a * load_fp", "accf[c] -= a * load_fp"),
    ("fp32 accumulator", "accf[c] += a * load_fp(j->B, j->in_type, ob + at(j->layout_b, k, c, j->ldb));",
     "accf[c] = (float)(accf[c] + a * load_fp(j->B, j->in_type, ob + at(j->layout_b, k, c, j->ldb)));"),
    ("fp32 intermediate before 16-bit output", "od + i * j->ldd + c, epilogue(j, b, i, c, accf[c], addend));",
     "od + i * j->ldd + c, (double)(float)epilogue(j, b, i, c, accf[c], addend));"),
    ("ties away from zero", "(frac == 0.5 && fmod(r, 2.0) != 0.0)", "(frac == 0.5)"),
    ("truncation", "if (frac > 0.5 || (frac == 0.5 && fmod(r, 2.0) != 0.0))", "if (0)"),
    ("subnormal outputs flushed", "return sign_bit | n;", "return sign_bit;"),
    ("overflow limit off by one", "if (e > emax)", "if (e > emax + 1)"),
    ("fp16 subnormal scale", "ldexp((double)m, -24)", "ldexp((double)m, -25)"),
    ("fp16 exponent bias", "e - 25); /* (1024+m)", "e - 24); /* (1024+m)"),
    ("bf16 exponent bias", "e - 134); /* (128+m)", "e - 133); /* (128+m)"),
    ("bf16 mantissa width", "m = h & 0x7f;", "m = h & 0x3f;"),
    ("batch stride of A ignored", "const int64_t oa = b * j->stride_a", "const int64_t oa = 0 * j->stride_a"),
    ("batch stride of B ignored", "ob = b * j->stride_b;", "ob = 0 * j->stride_b;"),
    ("batch stride of C ignored", "const int64_t oc = b * j->stride_c", "const int64_t oc = 0 * j->stride_c"),
    ("ldc taken as N", "oc + i * j->ldc + c) : 0.0;\n                store_out(j->D, j->out_type, od + i * j->ldd + c, epilogue(j, b, i, c, accf[c]",
     "oc + i * j->N + c) : 0.0;\n                store_out(j->D, j->out_type, od + i * j->ldd + c, epilogue(j, b, i, c, accf[c]"),
    ("int8 read unsigned", "(int64_t)((const int8_t *)p)[idx]", "(int64_t)((const uint8_t *)p)[idx]"),
    ("row scale indexed by column", "v *= (double)j->rs[b * j->stride_rs + i];",
     "v *= (double)j->rs[b * j->stride_rs + c];"),
    ("column scale indexed by row", "v *= (double)j->cs[b * j->stride_cs + c];",
     "v *= (double)j->cs[b * j->stride_cs + i];"),
    ("bias indexed by row", "v += (double)j->bias[b * j->stride_bias + c];",
     "v += (double)j->bias[b * j->stride_bias + i];"),
    ("batch stride of the column scale ignored", "j->cs[b * j->stride_cs + c]", "j->cs[0 * j->stride_cs + c]"),
    ("bias subtracted", "v += (double)j->bias[", "v -= (double)j->bias["),
    ("ReLU keeps negatives", "v = v > 0.0 ? v : 0.0;", "v = v > 0.0 ? v : 0.1 * v;"),
    ("GELU cubic coefficient", "(v + 0.044715 * v * v * v)", "(v + 0.0447 * v * v * v)"),
    ("GELU without the sqrt(2/pi) factor", "sqrt(2.0 / acos(-1.0)) * (v", "(v"),
    ("GELU logistic of u instead of 2u", "v = v / (1.0 + exp(-2.0 * u));", "v = v / (1.0 + exp(-u));"),
    ("dequantisation without wrap-around", "epilogue(j, b, i, c, (double)wrap_i32(acci[c]), addend)",
     "epilogue(j, b, i, c, (double)acci[c], addend)"),
    ("int32 saturates", "static int32_t wrap_i32(int64_t v) { return (int32_t)(uint32_t)(uint64_t)v; }",
     "static int32_t wrap_i32(int64_t v) { return v > INT32_MAX ? INT32_MAX : "
     "(v < INT32_MIN ? INT32_MIN : (int32_t)v); }"),
    ("e4m3 exponent bias", "ldexp((double)(m | 0x8), e - 10);", "ldexp((double)(m | 0x8), e - 11);"),
    ("e4m3 subnormal scale", "ldexp((double)m, -9);", "ldexp((double)m, -10);"),
    ("e4m3 all-ones exponent taken as infinity", "if (e == 0xf && m == 0x7)\n        return NAN;",
     "if (e == 0xf)\n        return m ? NAN : INFINITY;"),
    ("e4m3 sign ignored", "    return s ? -v : v;\n}\n\n/*\n * Round x", "    return v;\n}\n\n/*\n * Round x"),
    ("e4m3 read as a 16-bit type", "case OR_E4M3: return oracle_decode_e4m3(((const uint8_t *)p)[idx]);",
     "case OR_E4M3: return oracle_decode_e4m3((uint8_t)((const uint16_t *)p)[idx]);"),
    ("attention: K indexed (d, key)", "b * a->stride_k + j * a->ldk + t", "b * a->stride_k + t * a->ldk + j"),
    ("attention: batch stride of V ignored", "b * a->stride_v + j * a->ldv + c", "0 * a->stride_v + j * a->ldv + c"),
    ("attention: last key dropped", "for (int64_t j = 0; j < a->sk; ++j) {\n        const double w",
     "for (int64_t j = 0; j + 1 < a->sk; ++j) {\n        const double w"),
    ("attention: last score term dropped", "for (int64_t t = 0; t < a->d; ++t)", "for (int64_t t = 0; t + 1 < a->d; ++t)"),
    ("attention: not normalised", "acc[c] / l);", "acc[c]);"),
    ("attention: scale applied twice", "s[j] = a->scale * dot;", "s[j] = a->scale * a->scale * dot;"),
    ("attention: row maximum not subtracted", "const double w = exp(s[j] - m);", "const double w = exp(s[j]);"),
    ("attention: first score as the maximum", "if (s[j] > m)\n            m = s[j];",
     "if (j == 0)\n            m = s[j];"),
    ("attention: ldo taken as dv", "out_row = b * a->stride_o + i * a->ldo;", "out_row = b * a->stride_o + i * a->dv;"),
    ("attention: selected rows map to the wrong query", "i = a->rows[2 * r + 1];", "i = a->rows[2 * r];"),
]

RUNNER = (
    "import sys, pytest, oracle\n"
    "oracle.LIB_PATH = sys.argv[1]\n"
    "sys.exit(pytest.main(['-x', '-q', '-p', 'no:cacheprovider', '--no-header',\n"
    "                      'tests/test_oracle_gemm.py', 'tests/test_oracle_codecs.py',\n"
    "                      'tests/test_oracle_epilogue.py', 'tests/test_oracle_attention.py',\n"
    "                      'tests/test_oracle_fp8.py']))\n"
)


def _build_mutant(tmp, idx, old, new):
    src = open(SRC).read()
    if old is not None:
        assert src.count(old) == 1, f"mutation site not unique or missing: {old!r}"
        src = src.replace(old, new)
    path_c = os.path.join(tmp, f"mutant{idx}.c")
    path_so = os.path.join(tmp, f"mutant{idx}.so")
    open(path_c, "w").write(src)
    subprocess.run(["gcc", "-std=c11", "-O2", "-fno-fast-math", "-ffp-contract=off", "-fPIC",
                    "-shared", "-pthread", "-o", path_so, path_c, "-lm"], check=True)
    return path_so


def _run_pins(lib):
    r = subprocess.run([sys.executable, "-c", RUNNER, lib], cwd=ROOT, capture_output=True,
                       text=True, timeout=600)
    return r.returncode, r.stdout[-2000:] + r.stderr[-2000:]


@pytest.fixture(scope="module")
def outcomes(tmp_path_factory):
    tmp = str(tmp_path_factory.mktemp("mutants"))
    libs = [_build_mutant(tmp, i, old, new) for i, (_, old, new) in enumerate(MUTANTS)]
    libs.append(_build_mutant(tmp, len(MUTANTS), None, None))  # unmutated control
    with ThreadPoolExecutor(max_workers=4) as ex:
        return list(ex.map(_run_pins, libs))


def test_unmutated_copy_passes(outcomes):
    rc, out = outcomes[-1]
    assert rc == 0, out


@pytest.mark.parametrize("idx", range(len(MUTANTS)), ids=[m[0] for m in MUTANTS])
def test_pins_fail_on_mutant(outcomes, idx):
    rc, out = outcomes[idx]
    assert rc == 1, f"mutant '{MUTANTS[idx][0]}' survived the pins (exit {rc}):\n{out}"
