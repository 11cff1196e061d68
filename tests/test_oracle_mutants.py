"""Mutation test of the oracle's pins.

Each case plants one plausible mistake in a copy of ``oracle/oracle.c`` (on the
CPU, in a temporary directory), builds it, and checks that at least one pin in
``oracle_pins`` fails on the broken copy.  The real oracle passes every pin
(``test_oracle.py``), so the pins are sensitive to each mistake listed here.
"""
import os
import tempfile

import pytest

import oracle
import oracle_pins
from oracle.build import DEFAULT_SRC, build

# (name, text in oracle.c, replacement)
MUTANTS = [
    ("sum_without_max_shift", "d += exp(x[j] - m);", "d += exp(x[j]);"),
    ("normalise_sign_flip", "y[j] = exp(x[j] - m) / d;", "y[j] = exp(m - x[j]) / d;"),
    ("normalise_without_divide", "y[j] = exp(x[j] - m) / d;", "y[j] = exp(x[j] - m);"),
    ("max_skips_last_element", "for (int64_t j = 0; j < n; ++j)\n        if (x[j] > m)",
     "for (int64_t j = 0; j + 1 < n; ++j)\n        if (x[j] > m)"),
    ("rescale_with_updated_max",  # the lesson's pitfall: rescale after overwriting m
     "        double d_new = d_prev * exp(m_prev - m_new) + exp(x[j] - m_new);\n        m_prev = m_new;",
     "        m_prev = m_new;\n        double d_new = d_prev * exp(m_prev - m_new) + exp(x[j] - m_new);"),
    ("recurrence_drops_rescale", "d_prev * exp(m_prev - m_new) + exp(x[j] - m_new)",
     "d_prev + exp(x[j] - m_new)"),
    ("combine_wrong_exponent_sign", "d1 * exp(m1 - m) + d2 * exp(m2 - m)",
     "d1 * exp(m - m1) + d2 * exp(m2 - m)"),
    ("combine_drops_second_term", "d1 * exp(m1 - m) + d2 * exp(m2 - m)", "d1 * exp(m1 - m)"),
    ("combine_takes_min", "double m = fmax(m1, m2);", "double m = fmin(m1, m2);"),
    ("identity_not_neutral", "        *m_out = m2;\n        *d_out = d2;",
     "        *m_out = m2;\n        *d_out = d2 + d1 + 1.0;"),
    ("topk_ties_to_highest_index", "if (a->index < b->index)\n        return -1;",
     "if (a->index < b->index)\n        return 1;"),
    ("topk_ascending", "if (a->value > b->value)\n        return -1;",
     "if (a->value > b->value)\n        return 1;"),
    ("topk_prob_unshifted", "probs[k] = exp(order[k].value - m) / d;",
     "probs[k] = exp(order[k].value) / d;"),
    ("bf16_wrong_shift", "((uint32_t)bits) << 16", "((uint32_t)bits) << 15"),
    ("logsumexp_drops_max", "return (d == 0.0) ? -INFINITY : m + log(d);",
     "return (d == 0.0) ? -INFINITY : log(d);"),
    ("naive_subtracts_a_maximum",  # the safe form: no longer overflows as the page says
     "        d += exp(x[j]);\n    for (int64_t j = 0; j < n; ++j)\n        y[j] = exp(x[j]) / d;",
     "        d += exp(x[j] - row_max(x, n));\n    for (int64_t j = 0; j < n; ++j)\n"
     "        y[j] = exp(x[j] - row_max(x, n)) / d;"),
    ("naive_sum_skips_first", "    double d = 0.0;\n    for (int64_t j = 0; j < n; ++j)\n        d += exp(x[j]);",
     "    double d = 0.0;\n    for (int64_t j = 1; j < n; ++j)\n        d += exp(x[j]);"),
    ("attention_drops_scale", "s[j] = scale * dot;", "s[j] = dot;"),
    ("attention_causal_hides_diagonal", "const int64_t nvis = causal ? q_off + i + 1 : nk; /* keys",
     "const int64_t nvis = causal ? q_off + i : nk; /* keys"),
    ("attention_weights_unnormalised", "a[j] = exp(s[j] - m) / l;", "a[j] = exp(s[j] - m);"),
    ("attention_lse_drops_max", "            if (lse)\n                lse[h * nq + i] = m + log(l);\n        }\n    }\n    free(qr);\n    free(kv);\n    free(vv);\n    free(s);\n    free(a);",
     "            if (lse)\n                lse[h * nq + i] = log(l);\n        }\n    }\n    free(qr);\n    free(kv);\n    free(vv);\n    free(s);\n    free(a);"),
    ("attention_multiplies_k_not_v", "orow[c] += a[j] * vv[j * d + c];", "orow[c] += a[j] * kv[j * d + c];"),
    ("attention_logits_use_key_zero", "dot += qr[c] * kv[j * d + c];", "dot += qr[c] * kv[c];"),
    ("attention_scale_applied_twice", "s[j] = scale * dot;", "s[j] = scale * scale * dot;"),
    ("tiled_forgets_rescale", "acc[c] *= alpha;", "acc[c] *= 1.0;"),
    ("tiled_sum_not_rescaled", "l = alpha * l + rowsum;", "l = l + rowsum;"),
    ("select_returns_reversed", "        vals[k] = order[k].value;", "        vals[k] = order[K - 1 - k].value;"),
    ("select_returns_probability_like", "        vals[k] = order[k].value;", "        vals[k] = exp(order[k].value);"),
]


@pytest.fixture(scope="module")
def source():
    with open(DEFAULT_SRC) as f:
        return f.read()


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_mutant(source, name, old, new):
    assert source.count(old) == 1, f"mutation site for {name} not found exactly once"
    with tempfile.TemporaryDirectory() as tmp:
        src = os.path.join(tmp, "oracle_mutant.c")
        with open(src, "w") as f:
            f.write(source.replace(old, new))
        lib = build(src, os.path.join(tmp, "liboracle_mutant.so"), werror=False)
        failed = oracle_pins.run_all(oracle.Oracle(lib))
    assert failed, f"no pin caught the mutant {name}"
