"""The pins have teeth: each plausible mistake planted in a copy of the oracle (on the CPU) makes
at least one pin of test_oracle_pins.py fail.  The planted copies are built into a temporary
directory and never touch oracle/liboracle.so."""
import inspect
import os
import subprocess

import pytest

import oracle
from tests import test_oracle_pins as pins

ORACLE_C = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle",
                        "oracle.c")

# (name, text to replace, replacement) -- each is one plausible slip
MUTATIONS = [
    ("nibble order swapped in pack", "(uint8_t)(code[0] | (code[1] << 4))",
     "(uint8_t)(code[1] | (code[0] << 4))"),
    ("nibble order swapped in unpack", "codes[j * k_pad + 2 * i] = low;",
     "codes[j * k_pad + 2 * i] = high;"),
    ("symmetric scale max/8", "s32 = amax / 7.0f;", "s32 = amax / 8.0f;"),
    ("asymmetric scale /16", "s32 = range / 15.0f;", "s32 = range / 16.0f;"),
    ("zero point sign", "const float neg_mn = -mn;", "const float neg_mn = mn;"),
    ("zero point not added", "v = v + zf;", "v = v;"),
    ("truncation instead of round", "v = v + zf;\n                        v = rintf(v);",
     "v = v + zf;\n                        v = truncf(v);"),
    ("act truncation instead of round", "v = rintf(v);\n                if (v < -127.0f)",
     "v = truncf(v);\n                if (v < -127.0f)"),
    ("pads excluded from stats", "const float r = k < d_in ? w[j * ldw + k] : 0.0f;\n"
     "                const float a = fabsf(r);",
     "const float r = k < d_in ? w[j * ldw + k] : w[j * ldw + d_in - 1];\n"
     "                const float a = fabsf(r);"),
    ("clip at 14", "if (v > 15.0f) v = 15.0f;", "if (v > 14.0f) v = 14.0f;"),
    ("bf16 truncation", "if (lower > 0x8000u || (lower == 0x8000u && (upper & 1u))) upper += 1u;",
     "(void)lower;"),
    ("dequant symmetric offset 7",
     "const double z = zeros ? (double)oracle_bf16_to_f32(zeros[j * n_groups + G]) : 8.0;\n"
     "            const double q = (double)code_at(qweight, k_pad, j, k);\n"
     "            w_hat[j * k_pad + k]",
     "const double z = zeros ? (double)oracle_bf16_to_f32(zeros[j * n_groups + G]) : 7.0;\n"
     "            const double q = (double)code_at(qweight, k_pad, j, k);\n"
     "            w_hat[j * k_pad + k]"),
    ("w4a16 wrong group index", "                const int64_t G = k / g;\n"
     "                const double s = (double)oracle_bf16_to_f32(scales[j * n_groups + G]);\n"
     "                const double z =\n",
     "                const int64_t G = (k / g + 1) % n_groups;\n"
     "                const double s = (double)oracle_bf16_to_f32(scales[j * n_groups + G]);\n"
     "                const double z =\n"),
    ("w4a16 bias dropped", "if (bias) acc += (double)oracle_bf16_to_f32(bias[j]);\n"
     "            y[m * d_out + j] = acc;", "y[m * d_out + j] = acc;"),
    ("act scale /128", "const float s = a / 127.0f;", "const float s = a / 128.0f;"),
    ("act clip 126", "if (v > 127.0f) v = 127.0f;", "if (v > 126.0f) v = 126.0f;"),
    ("w4a8 offset 7", "const int64_t wq = (int64_t)code_at(qweight, k_pad, j, k) - 8;",
     "const int64_t wq = (int64_t)code_at(qweight, k_pad, j, k) - 7;"),
    ("w4a8 scale dropped", "double r = (double)oracle_bf16_to_f32(s_w[j]) * (double)s_x[m]",
     "double r = (double)s_x[m]"),
    ("qat step max/8", "const float s_m = amax / (float)m;", "const float s_m = amax / 8.0f;"),
    ("qat search from 8 down", "for (int m = 1; m <= 8 && !found; ++m) {",
     "for (int m = 8; m >= 1 && !found; --m) {"),
    ("qat tolerance 1/2", "dev > 0.0625f", "dev > 0.5f"),
    ("qat least squares dropped", "const float s32 = den > 0.0 ? (float)(num / den) : 0.0f;",
     "const float s32 = amax / (float)found;"),
    ("qat level +8 allowed", "l > 7.0f ||", "l > 8.0f ||"),
]


def _pin_tests():
    out = []
    for name, fn in inspect.getmembers(pins, inspect.isfunction):
        if not name.startswith("test_"):
            continue
        params = getattr(fn, "pytestmark", [])
        cases = [{}]
        for mark in params:
            if mark.name == "parametrize":
                argnames = [a.strip() for a in mark.args[0].split(",")] if isinstance(
                    mark.args[0], str) else list(mark.args[0])
                new = []
                for c in cases:
                    for v in mark.args[1]:
                        vals = v if len(argnames) > 1 else (v,)
                        d = dict(c)
                        d.update(zip(argnames, vals))
                        new.append(d)
                cases = new
        out.append((name, fn, cases))
    return out


def _any_pin_fails(golden_dir):
    for name, fn, cases in _pin_tests():
        for kw in cases:
            if "golden_dir" in inspect.signature(fn).parameters:
                kw = dict(kw, golden_dir=golden_dir)
            try:
                fn(**kw)
            except Exception:
                return name
    return None


@pytest.mark.parametrize("name,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_planted_mistake_is_caught(tmp_path, golden_dir, name, old, new):
    src = open(ORACLE_C).read()
    assert src.count(old) == 1, f"mutation anchor not unique/found: {name}"
    mutated = tmp_path / "oracle_mut.c"
    mutated.write_text(src.replace(old, new))
    lib = tmp_path / "liboracle_mut.so"
    subprocess.run(["gcc", "-std=c11", "-O2", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
                    "-o", str(lib), str(mutated), "-lm"], check=True)
    with oracle.use_library(str(lib)):
        caught = _any_pin_fails(golden_dir)
    assert caught is not None, f"no pin catches: {name}"


# The GPTQ reference (oracle/gptq.py, numpy): each slip planted in a copy of the module makes at
# least one GPTQ pin fail.
GPTQ_PY = os.path.join(os.path.dirname(ORACLE_C), "gptq.py")
GPTQ_MUTATIONS = [
    ("gptq update sign", "W[:, i:] -= np.outer(e, U[i, i:])", "W[:, i:] += np.outer(e, U[i, i:])"),
    ("gptq column of U", "W[:, i:] -= np.outer(e, U[i, i:])", "W[:, i:] -= np.outer(e, U[i:, i])"),
    ("gptq error not normalised", "e = err / U[i, i]", "e = err"),
    ("gptq no damping", "h[np.diag_indices_from(h)] += lam", "pass"),
    ("gptq dead weights kept", "w[:, dead] = 0.0", "pass"),
    ("gptq hessian 1/N", "(2.0 / x.shape[0])", "(1.0 / x.shape[0])"),
    ("gptq loss without U_ii", "L += 0.5 * float(np.sum(err * err)) / (U[i, i] * U[i, i])",
     "L += 0.5 * float(np.sum(err * err))"),
]


@pytest.mark.parametrize("name,old,new", GPTQ_MUTATIONS, ids=[m[0] for m in GPTQ_MUTATIONS])
def test_planted_gptq_mistake_is_caught(monkeypatch, name, old, new):
    import types
    src = open(GPTQ_PY).read()
    assert src.count(old) == 1, f"mutation anchor not unique/found: {name}"
    mod = types.ModuleType("oracle.gptq_mut")
    mod.__package__ = "oracle"
    exec(compile(src.replace(old, new), GPTQ_PY, "exec"), mod.__dict__)
    monkeypatch.setattr(pins, "gq", mod)
    caught = None
    for pname, fn, cases in _pin_tests():
        if "gptq" not in pname:
            continue
        for kw in cases:
            try:
                fn(**kw)
            except Exception:
                caught = pname
                break
        if caught:
            break
    assert caught is not None, f"no pin catches: {name}"
