"""Plant plausible mistakes in copies of the oracle (on the CPU) and check
that the pins catch every one: a dropped term, a wrong sign, index or
offset, a wrong head mapping, a missing normalisation."""

import os

import pytest

import oracle
import pins

MUTANTS = {
    "no_scale": ("s[j] = J->scale * dot;", "s[j] = dot;"),
    "exp_sign": ("s[j] = exp(s[j] - m);", "s[j] = exp(m - s[j]);"),
    "no_normalise": ("const double w = s[j] / l;", "const double w = s[j];"),
    "lse_drops_max": ("*lout = m + log(l);", "*lout = log(l);"),
    "lse_base2": ("*lout = m + log(l);", "*lout = m + log2(l);"),
    "causal_strict": ("(int64_t)i + (skv - sq) + 1;", "(int64_t)i + (skv - sq);"),
    "causal_top_left": ("(int64_t)i + (skv - sq) + 1;", "(int64_t)i + 1;"),
    "gqa_modulo": ("int hk = h / group;", "int hk = h % J->Hkv;"),
    "v_uses_k": ("const float* vrow = vbase + (jlo + j) * d;", "const float* vrow = kbase + (jlo + j) * d;"),
    "last_key_dropped": ("for (int64_t j = 0; j < n; ++j) {\n        s[j] = exp",
                         "for (int64_t j = 0; j + 1 < n; ++j) {\n        s[j] = exp"),
    "empty_row_lse_zero": ("if (lout) *lout = -INFINITY;", "if (lout) *lout = 0.0;"),
    "tail_key_dropped": ("int64_t nvis = skv;", "int64_t nvis = skv - 1;"),
    "varlen_kv_offset": ("kbase = J->k + ((int64_t)hk * T + start) * d;", "kbase = J->k + ((int64_t)hk * T) * d;"),
    "window_off_by_one": ("jlo = (int64_t)i + (skv - sq) - J->window + 1;", "jlo = (int64_t)i + (skv - sq) - J->window;"),
    "window_not_causal": ("if (J->causal || J->window > 0) {", "if (J->causal) {"),
    "window_from_top_left": ("jlo = (int64_t)i + (skv - sq) - J->window + 1;", "jlo = (int64_t)i - J->window + 1;"),
    "sink_sign": ("if (J->sinks) l += exp(sink - m);", "if (J->sinks) l += exp(m - sink);"),
    "sink_dropped": ("if (J->sinks) l += exp(sink - m);", ";"),
    "sink_no_max": ("if (J->sinks && sink > m) m = sink;", ";"),
    "sink_empty_row_lse": ("if (lout && J->sinks) *lout = sink;", ";"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name, tmp_path):
    src = open(os.path.join(os.path.dirname(oracle.__file__), "attn_ref.c")).read()
    old, new = MUTANTS[name]
    assert src.count(old) == 1, f"mutation site for {name} not unique"
    mpath = tmp_path / f"attn_{name}.c"
    mpath.write_text(src.replace(old, new))
    lib = oracle.load(oracle.build(out=str(tmp_path / f"lib_{name}.so"), src=str(mpath)))
    caught = []
    for pin in pins.ALL_PINS:
        try:
            pin(lib)
        except (AssertionError, ValueError, FloatingPointError):
            caught.append(pin.__name__)
    assert caught, f"no pin catches mutant {name}"
