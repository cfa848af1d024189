"""Plant plausible mistakes into copies of the oracle (on the CPU) and check
that the pins catch every one of them: a dropped decay, erase reading the
undecayed state, swapped gates, read-out before the write, a sign flip, the
decay applied along the value axis, and reverse-mode slips."""
import ctypes
import os
import subprocess

import numpy as np
import pytest

import oracle
from tests import test_oracle_pins as pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "gdr_oracle.c")

FWD_MUTANTS = {
    "no_decay": ("S[i * dv + j] *= a;", "S[i * dv + j] *= 1.0;"),
    "erase_sign": ("S[i * dv + j] += k[i] * (w[j] * v[j] - r[j]);",
                   "S[i * dv + j] += k[i] * (w[j] * v[j] + r[j]);"),
    "swap_gate_roles": ("double e = b[i] * k[i];\n        for (int j = 0; j < dv; ++j) r[j] += S[i * dv + j] * e;",
                        "double e = k[i];\n        for (int j = 0; j < dv; ++j) r[j] += S[i * dv + j] * e * w[j];"),
    "write_gate_dropped": ("(w[j] * v[j] - r[j])", "(v[j] - r[j])"),
    "erase_gate_dropped": ("double e = b[i] * k[i];\n        for (int j = 0; j < dv; ++j) r[j] += S[i * dv + j] * e;",
                           "double e = k[i];\n        for (int j = 0; j < dv; ++j) r[j] += S[i * dv + j] * e;"),
    "readout_index": ("o[j] += S[i * dv + j] * q[i];", "o[j] += S[i * dv + j] * k[i];"),
}

BWD_MUTANTS = {
    "dla_missing_a": ("dla[xk + i] = acc * a;", "dla[xk + i] = acc;"),
    "db_sign": ("db[xk + i] = de[i] * kt[i];", "db[xk + i] = -de[i] * kt[i];"),
    "G_not_decayed": ("G[i * dv + j] = a * g;", "G[i * dv + j] = g;"),
    "dw_uses_w": ("dw[xv + j] = ddl[j] * vt[j];", "dw[xv + j] = ddl[j] * wt[j];"),
}


def _build_mutant(tmp_path, name, old, new):
    src = open(SRC).read()
    assert src.count(old) >= 1, name
    msrc = src.replace(old, new)
    c = tmp_path / f"{name}.c"
    so = tmp_path / f"{name}.so"
    c.write_text(msrc)
    subprocess.run(["gcc", "-O1", "-fopenmp", "-fPIC", "-shared", "-o", str(so), str(c), "-lm"],
                   check=True)
    return str(so)


def _swap_lib(path):
    lib = ctypes.CDLL(path)
    P, I = ctypes.c_void_p, ctypes.c_int
    lib.oracle_fwd.argtypes = [I, I, I, I] + [P] * 9 + [I]
    lib.oracle_decode.argtypes = [I, I, I] + [P] * 8 + [I]
    lib.oracle_bwd.argtypes = [I, I, I, I] + [P] * 16 + [I]
    lib.oracle_num_threads.restype = I
    return lib


FWD_PINS = [pins.test_hand_worked_two_tokens, pins.test_pure_decay_closed_form,
            pins.test_overwrite_with_decay_and_write_gate,
            pins.test_tied_gates_with_channel_decay_give_kda,
            lambda: pins.test_brute_force_transition_products(9, 3, 7, 2.0)]
BWD_PINS = [pins.test_hand_worked_scalar_backward,
            lambda: pins.test_backward_finite_differences(True)]


def _caught(pinset):
    for p in pinset:
        try:
            p()
        except AssertionError:
            return True
    return False


@pytest.mark.parametrize("name", sorted(FWD_MUTANTS) + sorted(BWD_MUTANTS))
def test_pins_catch_mutant(tmp_path, monkeypatch, name):
    old, new = {**FWD_MUTANTS, **BWD_MUTANTS}[name]
    so = _build_mutant(tmp_path, name, old, new)
    oracle._load()
    monkeypatch.setattr(oracle, "_lib", _swap_lib(so))
    pinset = FWD_PINS if name in FWD_MUTANTS else BWD_PINS
    assert _caught(pinset), f"mutant {name} survived every pin"
