"""The oracle against its pins, and planted mistakes against the same pins.

Every pin in ``oracle_pins`` must hold for the oracle. Each planted mistake is
a copy of ``oracle/sgla_oracle.c`` with one plausible error (a swapped step, a
dropped term, a wrong index, sign or base), compiled on the CPU; at least one
pin must reject each of them, which shows the pins can see that kind of error.
"""
import os

import numpy as np
import pytest

import oracle
from tests import oracle_pins


@pytest.fixture(scope="module")
def orc():
    oracle.build(force=False)
    return oracle.Oracle(oracle.LIBRARY)


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda p: p.__name__)
def test_pin(orc, pin):
    pin(orc)


MUTANTS = {
    "update_before_decay": ("    decay(S, g, Dk, Dv);\n    update(S, k, v, Dk, Dv);",
                            "    update(S, k, v, Dk, Dv);\n    decay(S, g, Dk, Dv);"),
    "query_before_update": ("    update(S, k, v, Dk, Dv);\n    query(S, q, scale, Dk, Dv, o_out);",
                            "    query(S, q, scale, Dk, Dv, o_out);\n    update(S, k, v, Dk, Dv);"),
    "decay_base_two": ("const double alpha = exp(g);", "const double alpha = exp2(g);"),
    "decay_sign": ("const double alpha = exp(g);", "const double alpha = exp(-g);"),
    "scale_dropped": ("o[j] *= scale;", "o[j] *= 1.0;"),
    "key_index_reversed": ("const double ki = (double)k[i];",
                           "const double ki = (double)k[Dk - 1 - i];"),
    "query_index_frozen": ("const double qi = (double)q[i];", "const double qi = (double)q[0];"),
    "state_transposed_read": ("o[j] += qi * S[(size_t)i * Dv + j];",
                              "o[j] += qi * S[(size_t)j * Dk + i];"),
    "initial_state_dropped": ("S[e] = S0 ? S0[sbase + e] : 0.0;", "S[e] = 0.0;"),
    "varlen_short_by_one": ("len = cu[n + 1] - cu[n];",
                            "len = cu[n + 1] - cu[n] - (cu[n + 1] > cu[n]);"),
    "time_reversed": ("for (int64_t t = tok0; t < tok0 + len; ++t) {",
                      "for (int64_t t = tok0 + len - 1; t >= tok0; --t) {"),
    "slot_map_ignored": ("const int64_t slot = idx ? (int64_t)idx[r] : (int64_t)r;",
                         "const int64_t slot = (int64_t)r;"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(tmp_path, name):
    old, new = MUTANTS[name]
    with open(oracle.SOURCE) as f:
        src = f.read()
    assert src.count(old) == 1, "mutation anchor not found: %s" % name
    path = tmp_path / ("mutant_%s.c" % name)
    path.write_text(src.replace(old, new))
    lib = oracle.compile_source(str(path), str(tmp_path / ("libmutant_%s.so" % name)))
    mutant = oracle.Oracle(lib)
    caught = []
    with np.errstate(all="ignore"):
        for pin in oracle_pins.ALL_PINS:
            try:
                pin(mutant)
            except (AssertionError, ValueError, RuntimeError):
                caught.append(pin.__name__)
    assert caught, "no pin rejects the planted mistake %s" % name
