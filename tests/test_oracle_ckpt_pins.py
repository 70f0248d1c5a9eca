"""Pins for the oracle's prefix-reuse checkpoints (CPU only).

Source: "Kimi K3's architecture" (orkas.ai), section "The bill comes due in the
serving stack": a prefix-cache hit needs the recurrent state restorable at the
same boundary as the cached token pages, so the state is checkpointed at a
sparse subset of the 512-token hash endpoints.

Pins, each able to catch a plausible slip in ``prefill_ckpt`` (a checkpoint
taken one piece early or late, pieces that restart from S0 instead of handing
the state on, outputs of the wrong piece):

* checkpoint i equals the final state of one uninterrupted run over the first
  (i + 1) * every tokens;
* the outputs and final state equal those of one uninterrupted run;
* resuming from a checkpoint reproduces the remaining outputs and the final
  state (the point of prefix reuse);
* fewer tokens than one interval give no checkpoint.
"""
import numpy as np
import pytest

import oracle


def _inputs(rng, B, T, H, dk, dv):
    q = rng.standard_normal((B, T, H, dk))
    k = rng.standard_normal((B, T, H, dk))
    q /= np.linalg.norm(q, axis=-1, keepdims=True)
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((B, T, H, dv))
    la = -0.1 * rng.random((B, T, H, dk))
    bt = rng.random((B, T, H))
    S0 = rng.standard_normal((B, H, dk, dv))
    return q, k, v, la, bt, S0


def _rel(x, y):
    return np.linalg.norm(x - y) / max(np.linalg.norm(y), 1e-300)


@pytest.mark.parametrize("T,every", [(40, 8), (37, 8), (16, 16)])
def test_checkpoints_are_prefix_states(T, every):
    rng = np.random.default_rng(T + every)
    q, k, v, la, bt, S0 = _inputs(rng, 2, T, 2, 6, 5)
    o, st, ck = oracle.prefill_ckpt(q, k, v, la, bt, S0, every)
    assert ck.shape == (2, T // every, 2, 6, 5)
    for i in range(T // every):
        p = (i + 1) * every
        _, sp = oracle.prefill(q[:, :p], k[:, :p], v[:, :p], la[:, :p], bt[:, :p], S0)
        assert _rel(ck[:, i], sp) < 1e-13, i
    o_full, st_full = oracle.prefill(q, k, v, la, bt, S0)
    assert _rel(o, o_full) < 1e-13 and _rel(st, st_full) < 1e-13


def test_resume_from_checkpoint():
    rng = np.random.default_rng(7)
    T, every = 48, 16
    q, k, v, la, bt, S0 = _inputs(rng, 2, T, 3, 8, 8)
    o, st, ck = oracle.prefill_ckpt(q, k, v, la, bt, S0, every)
    for i in range(T // every):
        p = (i + 1) * every
        o_r, st_r = oracle.prefill(q[:, p:], k[:, p:], v[:, p:], la[:, p:], bt[:, p:], ck[:, i])
        assert _rel(o_r, o[:, p:]) < 1e-12 and _rel(st_r, st) < 1e-12


def test_short_sequence_has_no_checkpoint():
    rng = np.random.default_rng(8)
    q, k, v, la, bt, S0 = _inputs(rng, 1, 7, 1, 4, 4)
    _, _, ck = oracle.prefill_ckpt(q, k, v, la, bt, S0, 8)
    assert ck.shape == (1, 0, 1, 4, 4)


# ------------------------------------------------------------- planted mistakes
def _ckpt_early(q, k, v, la, bt, S0, every, nthreads=None):
    o, st, ck = _REAL(q, k, v, la, bt, S0, every)
    ck2 = ck.copy()
    ck2[:, 1:] = ck[:, :-1]
    ck2[:, :1] = S0[:, None] if S0 is not None else 0.0
    return o, st, ck2


def _ckpt_no_handoff(q, k, v, la, bt, S0, every, nthreads=None):
    B, T = q.shape[:2]
    n = T // every
    o, st, ck = _REAL(q, k, v, la, bt, S0, every)
    for i in range(n):
        a, e = i * every, (i + 1) * every
        _, ck[:, i] = oracle.prefill(q[:, a:e], k[:, a:e], v[:, a:e], la[:, a:e], bt[:, a:e], S0)
    return o, st, ck


_REAL = oracle.prefill_ckpt
MUTANTS = {"checkpoint_one_piece_early": _ckpt_early, "pieces_restart_from_S0": _ckpt_no_handoff}
PINS = [lambda: test_checkpoints_are_prefix_states(40, 8), lambda: test_checkpoints_are_prefix_states(37, 8),
        test_resume_from_checkpoint]


@pytest.mark.parametrize("mutant", sorted(MUTANTS))
def test_ckpt_mutant_is_caught(mutant, monkeypatch):
    monkeypatch.setattr(oracle, "prefill_ckpt", MUTANTS[mutant])
    caught = 0
    for pin in PINS:
        try:
            pin()
        except AssertionError:
            caught += 1
    assert caught, f"no pin catches the mutant {mutant}"
