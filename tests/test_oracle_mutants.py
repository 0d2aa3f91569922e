"""Plant plausible mistakes in the decode oracle and check that its pins catch each one.

The mistakes are planted by swapping one helper of ``oracle.attention`` (or the
layout view it reads through) for a wrong version; every mutant must make at
least one pin fail.
"""
import numpy as np
import pytest

import oracle
import oracle.attention as att
import oracle.layout as lay
from oracle_pins import ALL_PINS


def _wrong_group(h, group):                      # q head -> kv head modulo instead of div
    return h % max(1, 2 if group == 1 else group)


def _off_by_one_gather(orig):
    def g(k, v, row, length, bs, n):
        return orig(k, v, row, length + 1, bs, n)    # reads one slot past the context
    return g


def _short_gather(orig):
    def g(k, v, row, length, bs, n):
        return orig(k, v, row, max(length - 1, 1), bs, n)   # drops the appended token
    return g


def _wrong_offset_gather(k_log, v_log, row, length, bs, n):
    t = np.arange(length)
    phys = np.asarray(row, dtype=np.int64)[t // bs]
    off = (t + 1) % bs
    return k_log[phys, :, off, :], v_log[phys, :, off, :]


def _swapped_kv_gather(orig):
    def g(k, v, row, length, bs, n):
        a, b = orig(k, v, row, length, bs, n)
        return b, a
    return g


def _no_max_attend(q_heads, k_ctx, v_ctx, scale64):
    s = scale64 * (q_heads @ k_ctx.T)
    w = np.exp(s)
    return (w @ v_ctx) / w.sum(axis=1, keepdims=True)


def _token_major_k_view(k_flat, N, Hkv, bs, D):
    return k_flat.reshape(N, bs, Hkv, D).transpose(0, 2, 1, 3)   # tokens outside kv heads


MUTANTS = {
    "gqa-modulo": lambda mp: mp.setattr(att, "kv_head_of", _wrong_group),
    "no-scale": lambda mp: mp.setattr(att, "scale_as_passed", lambda s: 1.0),
    "gather-one-extra": lambda mp: mp.setattr(att, "gather_context", _off_by_one_gather(att.gather_context)),
    "gather-one-short": lambda mp: mp.setattr(att, "gather_context", _short_gather(att.gather_context)),
    "gather-wrong-offset": lambda mp: mp.setattr(att, "gather_context", _wrong_offset_gather),
    "k-v-swapped": lambda mp: mp.setattr(att, "gather_context", _swapped_kv_gather(att.gather_context)),
    "softmax-without-max": lambda mp: mp.setattr(att, "attend", _no_max_attend),
    "k-layout-heads-and-tokens-swapped": lambda mp: mp.setattr(att, "k_logical", _token_major_k_view),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, monkeypatch):
    MUTANTS[name](monkeypatch)
    caught = []
    with np.errstate(all="ignore"):
        for pin in ALL_PINS:
            try:
                pin(oracle.decode)
            except (AssertionError, FloatingPointError, ValueError, IndexError):
                caught.append(pin.__name__)
    assert caught, f"mutant {name} passed every pin"
