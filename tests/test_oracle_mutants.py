"""Plausible mistakes planted in the oracle must fail at least one pin (CPU only).

Each mutant replaces the oracle's one-token update with a subtly wrong variant
(operation order, a dropped factor, a sign, the floor) and the pin battery of
test_oracle_pins.py is run against it.  This shows the pins would catch such a
mistake in the oracle itself.
"""
import numpy as np
import pytest

import oracle.sequential as R
from test_oracle_pins import PINS

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def _decay(g):
    return np.exp(R.clamp_decay(g))


def m_read_before_write(S, q, k, v, g, b):
    Sp = _decay(g)[..., :, None] * S
    u = b[..., None] * (v - np.einsum("bhi,bhij->bhj", k, Sp))
    o = np.einsum("bhi,bhij->bhj", q, Sp)
    return o, Sp + k[..., :, None] * u[..., None, :]


def m_decay_after_write(S, q, k, v, g, b):
    u = b[..., None] * (v - np.einsum("bhi,bhij->bhj", k, S))
    S = _decay(g)[..., :, None] * (S + k[..., :, None] * u[..., None, :])
    return np.einsum("bhi,bhij->bhj", q, S), S


def m_no_beta(S, q, k, v, g, b):
    Sp = _decay(g)[..., :, None] * S
    u = v - np.einsum("bhi,bhij->bhj", k, Sp)
    S = Sp + k[..., :, None] * u[..., None, :]
    return np.einsum("bhi,bhij->bhj", q, S), S


def m_erase_sign(S, q, k, v, g, b):
    Sp = _decay(g)[..., :, None] * S
    u = b[..., None] * (v + np.einsum("bhi,bhij->bhj", k, Sp))
    S = Sp + k[..., :, None] * u[..., None, :]
    return np.einsum("bhi,bhij->bhj", q, S), S


def m_beta_on_erase_only(S, q, k, v, g, b):
    Sp = _decay(g)[..., :, None] * S
    u = v - b[..., None] * np.einsum("bhi,bhij->bhj", k, Sp)
    S = Sp + k[..., :, None] * u[..., None, :]
    return np.einsum("bhi,bhij->bhj", q, S), S


def m_erase_undecayed(S, q, k, v, g, b):
    Sp = _decay(g)[..., :, None] * S
    u = b[..., None] * (v - np.einsum("bhi,bhij->bhj", k, S))
    S = Sp + k[..., :, None] * u[..., None, :]
    return np.einsum("bhi,bhij->bhj", q, S), S


def m_read_with_key(S, q, k, v, g, b):
    Sp = _decay(g)[..., :, None] * S
    u = b[..., None] * (v - np.einsum("bhi,bhij->bhj", k, Sp))
    S = Sp + k[..., :, None] * u[..., None, :]
    return np.einsum("bhi,bhij->bhj", k, S), S


def _with_decay(fn):
    def step(S, q, k, v, g, b):
        Sp = fn(g)[..., :, None] * S
        u = b[..., None] * (v - np.einsum("bhi,bhij->bhj", k, Sp))
        S = Sp + k[..., :, None] * u[..., None, :]
        return np.einsum("bhi,bhij->bhj", q, S), S
    return step


MUTANTS = {
    "read_before_write": m_read_before_write,
    "decay_after_write": m_decay_after_write,
    "no_beta": m_no_beta,
    "erase_sign": m_erase_sign,
    "beta_on_erase_only": m_beta_on_erase_only,
    "erase_undecayed": m_erase_undecayed,
    "read_with_key": m_read_with_key,
    "no_floor": _with_decay(lambda g: np.exp(np.minimum(0.0, g))),
    "floor_at_minus_4": _with_decay(lambda g: np.exp(np.clip(g, -4.0, 0.0))),
    "no_upper_clamp": _with_decay(lambda g: np.exp(np.maximum(-5.0, g))),
    "decay_base_2": _with_decay(lambda g: np.exp2(R.clamp_decay(g))),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, monkeypatch):
    monkeypatch.setattr(R, "_step", MUTANTS[name])
    failed = []
    for pin, (fn, tol) in PINS.items():
        try:
            err = fn()
        except Exception:  # a crash also counts as a caught mistake
            failed.append(pin)
            continue
        if not (err <= tol):
            failed.append(pin)
    assert failed, f"mutant {name} passed every pin"


def test_unmutated_passes_every_pin():
    for pin, (fn, tol) in PINS.items():
        assert fn() <= tol, pin
