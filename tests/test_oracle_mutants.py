"""The pins must catch plausible mistakes in the oracle.

Each case plants one mistake in a temporary copy of ``oracle/gdn_oracle.c`` (on
the CPU), builds it, and runs the pins of ``test_oracle_pins`` against that
mutant: at least one pin has to fail.  The real oracle is never modified.
"""
import importlib.util
import os
import subprocess

import pytest

import test_oracle_pins as pins

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "gdn_oracle.c")
PKG = os.path.join(ROOT, "oracle", "__init__.py")

MUTANTS = {
    "sign_of_erase_term": ("- alpha * beta * sk * k[j]", "+ alpha * beta * sk * k[j]"),
    "dropped_erase_term": ("- alpha * beta * sk * k[j]", ""),
    "dropped_write_term": ("+ beta * v[i] * k[j]", ""),
    "transposed_state": ("sk += row[j] * k[j];", "sk += S[(int64_t)j * Dk + i] * k[j];"),
    "interleaved_pairing": ("int g = h % NK;                                           /* tiled",
                            "int g = h / (NV / NK);                                    /* tiled"),
    "no_output_scale": ("double scale = 1.0 / sqrt((double)Dk);", "double scale = 1.0;"),
    "output_decayed_twice": ("acc += row[j] * q[j];", "acc += row[j] * q[j] * alpha;"),
    "eps_outside_root": ("sqrt(ss / (double)Dv + eps)", "(sqrt(ss / (double)Dv) + eps)"),
    "sigmoid_sign": ("z[i] / (1.0 + exp(-z[i]))", "z[i] / (1.0 + exp(z[i]))"),
    "norm_weight_dropped": ("(gn[i] * o[i] / r)", "(o[i] / r)"),
    "f16_truncates": ("double m = nearbyint(ldexp(a, 10 - e));", "double m = floor(ldexp(a, 10 - e));"),
    "bf16_truncates": ("double m = nearbyint(ldexp(a, 7 - e));", "double m = floor(ldexp(a, 7 - e));"),
    "bf16_subnormal_flush": ("double m = nearbyint(ldexp(a, 133));", "double m = 0.0;"),
    "f16_subnormal_flush": ("double m = nearbyint(ldexp(a, 24));", "double m = 0.0;"),
    "no_per_step_rounding": ("if (state_kind == ORC_STATE_F32) S[e] = (double)(float)S[e];",
                             "if (state_kind == ORC_STATE_F32) S[e] = S[e];"),
    "v_row_index": ("v[r * v_stride + (int64_t)h * Dv + i]", "v[r * v_stride + (int64_t)g * Dv + i]"),
    "conv_input_at_oldest_row": ("ring[(int64_t)(taps - 1) * C + c] = x[c];", "ring[c] = x[c];"),
    "conv_drops_a_tap": ("for (int t = 0; t < taps; ++t)\n            acc +=",
                         "for (int t = 1; t < taps; ++t)\n            acc +="),
    "conv_no_silu": ("y[c] = acc / (1.0 + exp(-acc));", "y[c] = acc;"),
    "l2_eps_outside_root": ("sqrt(ss + l2_eps)", "(sqrt(ss) + l2_eps)"),
    "l2_over_all_of_q": ("for (int j = 0; j < D; ++j) ss += src[j] * src[j];",
                         "for (int j = 0; j < D; ++j) ss += y[j] * y[j];"),
    "v_takes_k_channels": ("v[i] = y[(int64_t)2 * NK * D + i]", "v[i] = y[(int64_t)NK * D + i]"),
    "beta_sign": ("exp(-(double)br[h])", "exp((double)br[h])"),
    "decay_sign": ("exp((double)ar[h] + (double)dt[h])", "exp(-(double)ar[h] - (double)dt[h])"),
    "decay_without_dt": ("exp((double)ar[h] + (double)dt[h])", "exp((double)ar[h])"),
    "fused_interleaved_pairing": ("int g = h % NK;\n            float *slot",
                                  "int g = h / (NV / NK);\n            float *slot"),
    "quant_scale_128": ("a / 127.0f", "a / 128.0f"),
    "quant_truncates": ("nearbyintf(y[g0 + i] / s)", "truncf(y[g0 + i] / s)"),
    "quant_ties_away": ("nearbyintf(y[g0 + i] / s)", "roundf(y[g0 + i] / s)"),
}

PINS = [name for name in dir(pins) if name.startswith("test_p") or name.startswith("test_f16")]


def _mutant(tmp_path, name):
    old, new = MUTANTS[name]
    text = open(SRC).read()
    assert text.count(old) == 1, f"mutation site for {name} not unique"
    src = tmp_path / f"{name}.c"
    src.write_text(text.replace(old, new))
    spec = importlib.util.spec_from_file_location(f"oracle_mutant_{name}", PKG)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    mod._SRC = str(src)
    mod._LIB = str(tmp_path / f"lib{name}.so")
    mod._lib = None
    subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off", "-o",
                    mod._LIB, mod._SRC, "-lm"], check=True)
    mod._load()
    return mod


def _call(fn, mod):
    import inspect
    params = inspect.signature(fn).parameters
    marks = getattr(fn, "pytestmark", [])
    combos = [{}]
    for m in marks:
        if m.name == "parametrize":
            names = [n.strip() for n in m.args[0].split(",")]
            combos = [dict(c, **dict(zip(names, vals if isinstance(vals, tuple) else (vals,))))
                      for c in combos for vals in m.args[1]]
    for extra in combos:
        kwargs = {k: v for k, v in extra.items() if k in params}
        fn(mod, **kwargs) if "orc" in params else fn(**kwargs)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(tmp_path, name):
    mod = _mutant(tmp_path, name)
    failed = []
    for pin in PINS:
        fn = getattr(pins, pin)
        try:
            _call(fn, mod)
        except (AssertionError, RuntimeError, ValueError, FloatingPointError):
            failed.append(pin)
    assert failed, f"no pin caught the planted mistake {name}"
