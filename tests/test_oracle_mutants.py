"""Each plausible mistake planted in a copy of the oracle must fail a pin.

The copies are made on the CPU, in a temporary directory: the oracle source is
read, one passage is replaced by a broken one, and both builds are compiled
and run through every pin. A mutant that passes all pins would mean the pins
cannot see that mistake.
"""
import os
import subprocess

import pytest

import oracle
from oracle_pins import ALL_PINS

SRC = os.path.join(os.path.dirname(oracle.__file__), "gdn_oracle.c")

MUTANTS = {
    # recurrence
    "pred_sign": ("(v[vec + j] - pred) * b", "(pred - v[vec + j]) * b"),
    "no_decay": ("r[i] = r[i] * d;", "r[i] = r[i];"),
    "decay_neg_g": ("const real d = R_EXP(g[tok * n_v_heads + h]);",
                    "const real d = R_EXP(-g[tok * n_v_heads + h]);"),
    "no_beta": ("const real delta = (v[vec + j] - pred) * b;",
                "const real delta = (v[vec + j] - pred);"),
    "update_uses_q": ("r[i] = r[i] + kt[i] * delta;", "r[i] = r[i] + qt[i] * delta;"),
    "no_scale": ("y[vec + j] = scale * o;", "y[vec + j] = o;"),
    "v_wrong_index": ("(v[vec + j] - pred)", "(v[vec + (S - 1 - j)] - pred)"),
    "read_before_write": (
        """            for (int i = 0; i < S; i++)
                r[i] = r[i] + kt[i] * delta;

            real o = 0;
            for (int i = 0; i < S; i++)
                o = o + r[i] * qt[i];""",
        """            real o = 0;
            for (int i = 0; i < S; i++)
                o = o + r[i] * qt[i];
            for (int i = 0; i < S; i++)
                r[i] = r[i] + kt[i] * delta;"""),
    "pred_before_decay": (
        """            for (int i = 0; i < S; i++)
                r[i] = r[i] * d;

            real pred = 0;
            for (int i = 0; i < S; i++)
                pred = pred + r[i] * kt[i];""",
        """            real pred = 0;
            for (int i = 0; i < S; i++)
                pred = pred + r[i] * kt[i];
            for (int i = 0; i < S; i++)
                r[i] = r[i] * d;"""),
    "transposed_state": (
        "real *r = state + (size_t)row * S;",
        "real rr[512]; real *r = rr; real *base = state + ((size_t)n * n_v_heads + h) * S * S;"
        " for (int i = 0; i < S; i++) r[i] = base[(size_t)i * S + j];"),
    # gate / sigmoid
    "gate_sign": ("real ssm_a = -R_EXP(A_log[h]);", "real ssm_a = R_EXP(A_log[h]);"),
    "gate_no_dt": ("real u = a[r * n_heads + h] + dt_bias[h];", "real u = a[r * n_heads + h];"),
    "softplus_guard": ("if (u > (real)20)", "if (u > (real)2)"),
    "softplus_plain_log": ("return R_LOG1P(R_EXP(u));", "return R_EXP(u);"),
    "sigmoid_sign": ("return (real)1 / ((real)1 + R_EXP(-x));", "return (real)1 / ((real)1 + R_EXP(x));"),
    # conv
    "conv_newest_weight": ("real acc = xv * wc[taps];", "real acc = xv * wc[0];"),
    "conv_appends_output": ("hist[taps - 1] = xv;", "hist[taps - 1] = acc;"),
    "conv_no_roll": ("hist[u] = hist[u + 1];", "hist[u] = hist[u];"),
    "conv_reversed_history": ("acc = acc + hist[u] * wc[u];", "acc = acc + hist[taps - 1 - u] * wc[u];"),
    "silu_sign": ("return x / ((real)1 + R_EXP(-x));", "return x / ((real)1 + R_EXP(x));"),
    # norm
    "norm_eps_outside": ("R_SQRT(ss / (real)D + eps)", "(R_SQRT(ss / (real)D) + eps)"),
    "norm_sum_not_mean": ("R_SQRT(ss / (real)D + eps)", "R_SQRT(ss + eps)"),
    "norm_no_gate": ("o[d] = yr[d] * inv * w[d] * silu(zr[d]);", "o[d] = yr[d] * inv * w[d];"),
    # l2 norm / repeat / block glue
    "l2_eps_added": ("real inv = (real)1 / (norm > eps ? norm : eps);", "real inv = (real)1 / (norm + eps);"),
    "l2_no_sqrt": ("real norm = R_SQRT(ss);", "real norm = ss;"),
    "gqa_interleaved": (
        "for (int vh = kh; vh < n_v_heads; vh += n_k_heads) {",
        "for (int vh = kh * (n_v_heads / n_k_heads); vh < (kh + 1) * (n_v_heads / n_k_heads); vh++) {"),
    "block_v_offset": ("co + 2 * key_dim, gt, bt, yt", "co + key_dim, gt, bt, yt"),
    "block_k_from_q": ("oracle_l2norm_gqa(co + key_dim, kr,", "oracle_l2norm_gqa(co, kr,"),
    "prefill_k_split": ("ks[t * key_dim + e] = co[t * C + key_dim + e];",
                        "ks[t * key_dim + e] = co[t * C + e];"),
    "prefill_gate_rows": ("gt,\n                          n_v_heads, n_tokens);",
                          "gt,\n                          n_v_heads, 1);"),
}


def _build(src_text, tmp_path, prec):
    c = tmp_path / "mut.c"
    c.write_text(src_text)
    out = tmp_path / f"libmut_{prec}.so"
    defs = ["-DORACLE_F64"] if prec == "f64" else []
    subprocess.run(["gcc", *oracle.CFLAGS, *defs, str(c), "-o", str(out), "-lm"], check=True)
    return oracle.bind(str(out), prec)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation site for {name} not found exactly once"
    mutated = src.replace(old, new)
    L32 = _build(mutated, tmp_path, "f32")
    L64 = _build(mutated, tmp_path, "f64")
    caught = []
    for pin_name, pin in ALL_PINS.items():
        try:
            pin(L32, L64)
        except AssertionError:
            caught.append(pin_name)
    assert caught, f"mutant {name} passed every pin"
