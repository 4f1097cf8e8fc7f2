"""Plant plausible mistakes in a private copy of the oracle (on the CPU) and check that the
pins catch every one: a dropped term, a wrong exponent, a transposed operand, a missing decay.

Each mutant is a textual substitution of la_oracle.c compiled with gcc into a temporary
library; the real oracle is never modified."""
import os

import pytest

import oracle
import oracle_pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "la_oracle.c")

# (name, original text, replacement, occurrence index or None for all)
MUTANTS = [
    ("quadratic_exponent_doubled", "    w *= lam;\n  }\n  if (S0 != NULL)",
     "    w *= lam * lam;\n  }\n  if (S0 != NULL)", 0),
    ("quadratic_drops_diagonal", "for (int64_t s = t; s >= beg; --s)",
     "for (int64_t s = t - 1; s >= beg; --s)", 0),
    ("quadratic_drops_first_token", "for (int64_t s = t; s >= beg; --s)",
     "for (int64_t s = t; s > beg; --s)", 0),
    ("quadratic_sign", "o[b] += a * vs[b];", "o[b] -= a * vs[b];", 0),
    ("quadratic_initial_state_undecayed", "o[b] += w * acc;", "o[b] += acc;", 0),
    ("recurrent_outer_transposed",
     "St[(size_t)a * D + b] = lam * St[(size_t)a * D + b] + kt[a] * vt[b];",
     "St[(size_t)a * D + b] = lam * St[(size_t)a * D + b] + kt[b] * vt[a];", 0),
    ("recurrent_state_read_transposed",
     "acc += qt[a] * St[(size_t)a * D + b];\n            ot[b] = acc;",
     "acc += qt[a] * St[(size_t)b * D + a];\n            ot[b] = acc;", 0),
    ("recurrent_no_decay",
     "St[(size_t)a * D + b] = lam * St[(size_t)a * D + b] + kt[a] * vt[b];",
     "St[(size_t)a * D + b] = St[(size_t)a * D + b] + kt[a] * vt[b];", 0),
    ("final_state_exponent_off_by_one",
     "double w = 1.0; /* lambda^(end-1-t), starting at the last token */",
     "double w = lam; /* lambda^(end-1-t), starting at the last token */", 0),
    ("final_state_outer_transposed", "St[(size_t)a * D + b] += w * kt[a] * vt[b];",
     "St[(size_t)a * D + b] += w * kt[b] * vt[a];", 0),
    ("decode_no_decay",
     "St[(size_t)a * D + c] = lam * St[(size_t)a * D + c] + kt[a] * vt[c];",
     "St[(size_t)a * D + c] = St[(size_t)a * D + c] + kt[a] * vt[c];", 0),
    ("decode_drops_outer_product",
     "St[(size_t)a * D + c] = lam * St[(size_t)a * D + c] + kt[a] * vt[c];\n      for (int32_t c = 0; c < D; ++c) {",
     "St[(size_t)a * D + c] = lam * St[(size_t)a * D + c] + 0.0 * kt[a] * vt[c];\n      for (int32_t c = 0; c < D; ++c) {", 0),
    ("unmasked_right_transposed",
     "M[(size_t)a * D + b] += k[(size_t)s * D + a] * v[(size_t)s * D + b];",
     "M[(size_t)a * D + b] += k[(size_t)s * D + b] * v[(size_t)s * D + a];", 0),
    ("unmasked_left_transposed_scores",
     "A[(size_t)t * n + s] = dot(q + (size_t)t * D, k + (size_t)s * D, D);",
     "A[(size_t)s * n + t] = dot(q + (size_t)t * D, k + (size_t)s * D, D);", 0),
    ("varlen_rows_wrong_sequence_start", "if (t >= beg && t < end) break;",
     "if (t >= beg && t < end) { beg = 0; break; }", 0),
    # backward, term-by-term form
    ("bwd_dq_initial_state_undecayed", "g[a] += w * acc;", "g[a] += acc;", 0),
    ("bwd_dq_initial_state_transposed", "acc += S0[(size_t)a * D + b] * dout_t[b];",
     "acc += S0[(size_t)b * D + a] * dout_t[b];", 0),
    ("bwd_dq_drops_diagonal", "for (int64_t s = t; s >= beg; --s) {\n            const double c",
     "for (int64_t s = t - 1; s >= beg; --s) {\n            const double c", 0),
    ("bwd_dk_drops_diagonal", "for (int64_t tp = t; tp < end; ++tp)",
     "for (int64_t tp = t + 1; tp < end; ++tp)", 0),
    ("bwd_dv_uses_dk_coefficient", "gv[a] += cv * dp[a];", "gv[a] += ck * dp[a];", 0),
    ("bwd_dv_final_grad_not_transposed", "accv += dSn[(size_t)b * D + a] * kt[b];",
     "accv += dSn[(size_t)a * D + b] * kt[b];", 0),
    ("bwd_dk_final_grad_exponent", "for (int64_t m = t; m < end - 1; ++m) wn *= lam;",
     "for (int64_t m = t; m < end; ++m) wn *= lam;", 0),
    ("bwd_dinit_exponent_off_by_one", "double w = lam; /* lambda^(t+1) at t = beg */",
     "double w = 1.0; /* lambda^(t+1) at t = beg */", 0),
    ("bwd_dinit_final_grad_undecayed", "g[e] += wn * dSn[e];", "g[e] += dSn[e];", 0),
    # backward, scan form
    ("bwdrec_dq_state_transposed", "acc += St[(size_t)a * D + b] * dt[b];",
     "acc += St[(size_t)b * D + a] * dt[b];", 0),
    ("bwdrec_decays_before_last_token", "const double w = t == end - 1 ? 1.0 : lam;",
     "const double w = lam;", 0),
    ("bwdrec_dv_not_transposed", "accv += G[(size_t)b * D + a] * kt[b];",
     "accv += G[(size_t)a * D + b] * kt[b];", 0),
    ("bwdrec_dk_from_k", "acck += G[(size_t)a * D + b] * vt[b];",
     "acck += G[(size_t)a * D + b] * kt[b];", 0),
    ("bwdrec_dinit_missing_lambda", "const double w = end > beg ? lam : 1.0;",
     "const double w = 1.0;", 0),
]


def _mutate(text, old, new, idx):
    parts = text.split(old)
    assert len(parts) > idx + 1, "mutation anchor not found: %r" % old
    return old.join(parts[: idx + 1]) + new + old.join(parts[idx + 1:])


@pytest.mark.parametrize("name,old,new,idx", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_mutant(tmp_path, name, old, new, idx):
    text = open(SRC).read()
    mutated = _mutate(text, old, new, idx)
    assert mutated != text
    src = tmp_path / ("mut_%s.c" % name)
    src.write_text(mutated)
    # the header sits next to the real source
    import shutil

    shutil.copy(os.path.join(os.path.dirname(SRC), "la_oracle.h"), tmp_path / "la_oracle.h")
    lib = oracle.build(force=True, src=str(src), out=str(tmp_path / ("lib_%s.so" % name)))
    mut = oracle.Oracle(lib)
    caught = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(mut)
        except (AssertionError, ValueError):
            caught.append(pin.__name__)
    assert caught, "no pin caught mutant %s" % name
