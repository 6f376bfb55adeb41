"""Planted mistakes in the oracle must be caught by its pins.

Each case copies ``oracle/gdr_oracle.c``, makes one plausible slip (a dropped term, a
flipped sign, a wrong index, a swapped operand, a reordered step), builds it with gcc in
a temporary directory and runs the pin suite against the broken build.  At least one pin
must fail, which shows the pins constrain every part of the oracle they are meant to.
The real oracle is never modified.
"""
import os
import re

import pytest

import oracle
from oracle_pins import ALL_PINS, TOL

SRC = os.path.join(os.path.dirname(oracle.__file__), "gdr_oracle.c")
# The tree route, at the end of the file, repeats the token step; these slips target the
# sequential and chunked routes before it (test_oracle_tree.py plants its own).
TREE_MARK = "/* Token recurrence over a tree"


def _split(src):
    i = src.index(TREE_MARK)
    return src[:i], src[i:]

# (name, route, old, new); route: which oracle route the pins exercise for this slip
MUTANTS = [
    ("decay_sign", "sequential", "Si[j] *= e;", "Si[j] *= 1.0 / e;"),
    ("delta_sign", "sequential", "d[j] = bt * (vt[j] - pred[j]);", "d[j] = bt * (vt[j] + pred[j]);"),
    ("beta_dropped", "sequential", "d[j] = bt * (vt[j] - pred[j]);", "d[j] = (vt[j] - pred[j]);"),
    ("gqa_modulo", "sequential",
     "h = bh % HV, kh = h / G;\n        double* S = (double*)malloc",
     "h = bh % HV, kh = h % HK;\n        double* S = (double*)malloc"),
    ("query_is_key", "sequential", "const double qi = qt[i];", "const double qi = kt[i];"),
    ("h0_ignored", "sequential",
     "if (h0)\n            memcpy(S, h0 + bh * dk * dv", "if (0)\n            memcpy(S, h0 + bh * dk * dv"),
    ("gate_per_key_head", "sequential",
     "const double* gt = g + ((b * T + t) * HV + h) * dk;",
     "const double* gt = g + ((b * T + t) * HV + kh) * dk;"),
    ("beta_per_key_head", "sequential",
     "const double bt = beta[(b * T + t) * HV + h];", "const double bt = beta[(b * T + t) * HV + kh];"),
    ("value_per_key_head", "sequential",
     "const double* vt = v + ((b * T + t) * HV + h) * dv;",
     "const double* vt = v + ((b * T + t) * HV + kh) * dv;"),
    ("output_before_update", "sequential", None, None),   # block swap, see _mutate
    ("predict_before_decay", "sequential", None, None),   # block swap, see _mutate
    ("prefix_exclusive", "chunked",
     "acc += GROW(r)[c];\n                    gam[r * dk + c] = acc;",
     "gam[r * dk + c] = acc;\n                    acc += GROW(r)[c];"),
    ("gram_diagonal_kept", "chunked", "A[r * C + s] = (s < r) ?", "A[r * C + s] = (s <= r) ?"),
    ("causal_diagonal_dropped", "chunked", "P[r * C + s] = (s <= r) ? p", "P[r * C + s] = (s < r) ? p"),
    ("rhs_beta_dropped", "chunked", "X[r * RW + c] = br * exp(", "X[r * RW + c] = exp("),
    ("query_decay_dropped", "chunked",
     "const double qd = exp(gam[r * dk + c]) * QROW(r)[c];", "const double qd = QROW(r)[c];"),
    ("carry_decay_dropped", "chunked", "const double el = exp(gl);", "const double el = 1.0;"),
    ("carry_key_decay_flipped", "chunked",
     "exp(gl - gam[r * dk + c]) * KROW(r)[c]", "exp(gam[r * dk + c] - gl) * KROW(r)[c]"),
    ("substitution_sign", "chunked", "X[r * RW + x] -= a * X[s * RW + x];", "X[r * RW + x] += a * X[s * RW + x];"),
    ("pseudo_value_sign", "chunked", "U[r * dv + j] -= w * S[c * dv + j];", "U[r * dv + j] += w * S[c * dv + j];"),
]


def _swap_blocks(src, first, second, end):
    """Swap the code blocks that start at comment ``first`` and ``second`` (ending at ``end``)."""
    i, j, e = src.index(first), src.index(second), src.index(end, src.index(second))
    a, b = src[i:j], src[j:e]
    return src[:i] + b + a + src[e:]


def _mutate(name, old, new):
    with open(SRC) as f:
        head, tail = _split(f.read())
    if name == "output_before_update":
        return _swap_blocks(head, "/* 3. rank-one delta update */", "/* 4. output from the updated state */",
                            "        }\n        if (ht) memcpy") + tail
    if name == "predict_before_decay":
        return _swap_blocks(head, "/* 1. decay */", "/* 2. predict */", "/* 3. rank-one delta update */") + tail
    assert head.count(old) == 1, f"mutation anchor for {name} not unique/present"
    return head.replace(old, new) + tail


@pytest.mark.parametrize("name,route,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_planted_mistake(tmp_path, name, route, old, new):
    src = _mutate(name, old, new)
    path = tmp_path / "mutant.c"
    path.write_text(src)
    lib = oracle.load(oracle.build(str(path), str(tmp_path / "libmutant.so")))
    errors = {}
    for pin_name, pin in ALL_PINS.items():
        kw = {"route": route} if route == "sequential" else {"route": route, "chunk": 3}
        try:
            errors[pin_name] = pin(lib, **kw)
        except Exception as exc:  # a crash or a shape error also counts as caught
            errors[pin_name] = float("inf")
            errors[pin_name + "_exc"] = repr(exc)
    caught = [p for p, e in errors.items() if isinstance(e, float) and not (e < TOL)]
    assert caught, f"mutant {name} passed every pin: {errors}"


def test_mutation_anchors_are_live():
    # guard against the mutants silently going stale when the oracle is edited
    with open(SRC) as f:
        src, _ = _split(f.read())
    for name, _, old, _ in MUTANTS:
        if old is not None:
            assert src.count(old) == 1, name
    assert re.search(r"/\* 4\. output from the updated state \*/", src)
