"""Planted mistakes in the oracle (on the CPU) must each trip at least one pin.

Each mutant replaces the oracle's per-row kernel ``_rows_plain`` or its
per-sequence driver with a copy carrying one plausible mistake: a dropped
term, a wrong sign, an off-by-one or reversed mask, a transposed operand, a
missing scale, the wrong logarithm.  The pins of ``oracle_pins`` are then
run against the broken oracle; a mutant that passes them all means the pins
have a blind spot.
"""
import numpy as np
import pytest

import oracle.exact as oa
from oracle_pins import PINS

_orig_rows = oa._rows_plain
_orig_seq = oa._sequence


def _rows_factory(mistake):
    def rows(q_rows, k, v, scale, row_ids, causal):
        n = k.shape[0]
        sc = 1.0 if mistake == "no_scale" else float(scale)
        s = sc * (q_rows @ k.T)
        if causal:
            if mistake == "mask_offbyone":
                mask = np.arange(n)[None, :] >= row_ids[:, None]
            elif mistake == "mask_reversed":
                mask = np.arange(n)[None, :] < row_ids[:, None]
            else:
                mask = np.arange(n)[None, :] > row_ids[:, None]
            s = np.where(mask, -np.inf, s)
        m = s.max(axis=1)
        empty = ~np.isfinite(m)
        m_safe = np.where(empty, 0.0, m)
        if mistake == "wrong_sign":
            p = np.exp(m_safe[:, None] - s)
            p = np.where(np.isfinite(s), p, 0.0)
        else:
            p = np.exp(s - m_safe[:, None])
        l = p.sum(axis=1)
        if mistake == "no_normalise":
            o = p @ v
        elif mistake == "values_reversed":
            o = (p @ v[::-1]) / l[:, None]
        else:
            o = (p @ v) / l[:, None]
        if mistake == "lse_no_max":
            lse = np.log(l)
        elif mistake == "lse_log2":
            lse = m_safe + np.log2(l)
        else:
            lse = m_safe + np.log(l)
        return o, lse
    return rows


def _seq_transposed(q, k, v, scale, causal, rows=None):
    # scores built with the roles of queries and keys swapped
    return _orig_seq(k, q, v, scale, causal, rows)


MUTANTS = ["no_scale", "mask_offbyone", "mask_reversed", "wrong_sign", "no_normalise",
           "values_reversed", "lse_no_max", "lse_log2", "transposed"]


@pytest.mark.parametrize("mistake", MUTANTS)
def test_mutant_is_caught(monkeypatch, mistake):
    if mistake == "transposed":
        monkeypatch.setattr(oa, "_sequence", _seq_transposed)
    else:
        monkeypatch.setattr(oa, "_rows_plain", _rows_factory(mistake))
    caught = []
    for pin in PINS:
        try:
            pin()
        except (AssertionError, ValueError, FloatingPointError, IndexError):
            caught.append(pin.__name__)
    assert caught, f"planted mistake '{mistake}' passed every pin"


def test_unmutated_factory_passes_all_pins(monkeypatch):
    """The mutant factory without a mistake is the oracle itself: all pins pass,
    so each mutant's failure is due to its one planted change."""
    monkeypatch.setattr(oa, "_rows_plain", _rows_factory("none"))
    for pin in PINS:
        pin()
