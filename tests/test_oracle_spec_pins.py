"""Pins for the oracle's speculative-decoding functions (CPU only).

Source: "Kimi K3's architecture" (orkas.ai), section "The bill comes due in the
serving stack": the state is updated in place, so a rejected draft cannot be
undone; the projected inputs of the drafted tokens are kept instead and the
state is rebuilt from them.  ``spec_verify`` is the recurrence over the m
drafted tokens from S with its final state discarded; ``spec_commit`` is the
state after the first accepted[n] of them.

Pins, chosen so that a plausible slip (committing every drafted token, ignoring
the clamp, verifying from an already-advanced state, mutating S in verify,
dropping the first or last accepted token) fails at least one of them:

* exact retrieval with unit decay, unit beta and orthonormal keys: after the
  commit, every accepted key retrieves its value and every rejected key still
  retrieves what the old state stored under it (closed form);
* verify outputs are the outputs of m successive one-token steps from S, and S
  is left untouched;
* commit of 0 tokens is the identity, of m tokens the full run, and counts
  outside [0, m] are clamped;
* rebuilding: the state after a accepted tokens, continued over the remaining
  drafted tokens, reproduces the verify outputs of those tokens.
"""
import numpy as np
import pytest

import oracle


def _inputs(rng, N, m, H, dk, dv, la_scale=1.0):
    q = rng.standard_normal((N, m, H, dk))
    k = rng.standard_normal((N, m, H, dk))
    q /= np.linalg.norm(q, axis=-1, keepdims=True)
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((N, m, H, dv))
    la = -la_scale * 5.0 * rng.random((N, m, H, dk))
    bt = rng.random((N, m, H))
    S = rng.standard_normal((N, H, dk, dv))
    return q, k, v, la, bt, S


def _rel(x, y):
    return np.linalg.norm(x - y) / max(np.linalg.norm(y), 1e-300)


def test_commit_retrieves_accepted_and_keeps_rejected():
    """alpha = 1, beta = 1, orthonormal keys: accepted keys retrieve their values exactly,
    rejected keys retrieve what S held before the block."""
    rng = np.random.default_rng(101)
    N, m, H, d = 5, 6, 2, 16
    q, k, v, la, bt, S = _inputs(rng, N, m, H, d, d)
    la[:] = 0.0
    bt[:] = 1.0
    for n in range(N):
        for h in range(H):
            Qm, _ = np.linalg.qr(rng.standard_normal((d, d)))
            k[n, :, h] = Qm[:, :m].T
    accepted = np.array([0, 1, 3, 6, 4])
    S_new = oracle.spec_commit(q, k, v, la, bt, S, accepted)
    for n in range(N):
        for h in range(H):
            for t in range(m):
                got = S_new[n, h].T @ k[n, t, h]
                want = v[n, t, h] if t < accepted[n] else S[n, h].T @ k[n, t, h]
                assert np.allclose(got, want, atol=1e-12), (n, h, t)


def test_verify_is_stepwise_and_leaves_state():
    rng = np.random.default_rng(102)
    N, m, H, dk, dv = 3, 5, 2, 12, 10
    q, k, v, la, bt, S = _inputs(rng, N, m, H, dk, dv)
    S_copy = S.copy()
    o = oracle.spec_verify(q, k, v, la, bt, S)
    assert np.array_equal(S, S_copy)
    s = S.copy()
    for t in range(m):
        o_t, s = oracle.decode_step(q[:, t], k[:, t], v[:, t], la[:, t], bt[:, t], s)
        assert _rel(o[:, t], o_t) < 1e-12, t


def test_commit_limits_and_clamp():
    rng = np.random.default_rng(103)
    N, m, H, dk, dv = 4, 7, 2, 8, 8
    q, k, v, la, bt, S = _inputs(rng, N, m, H, dk, dv)
    S_copy = S.copy()
    _, S_full = oracle.prefill(q, k, v, la, bt, S)
    assert np.array_equal(oracle.spec_commit(q, k, v, la, bt, S, np.zeros(N, dtype=int)), S)
    assert _rel(oracle.spec_commit(q, k, v, la, bt, S, np.full(N, m)), S_full) < 1e-13
    clamped = oracle.spec_commit(q, k, v, la, bt, S, np.array([-3, m + 5, 0, m]))
    assert np.array_equal(clamped[0], S[0]) and np.array_equal(clamped[2], S[2])
    assert _rel(clamped[1], S_full[1]) < 1e-13 and _rel(clamped[3], S_full[3]) < 1e-13
    assert np.array_equal(S, S_copy)


@pytest.mark.parametrize("a", [1, 2, 4])
def test_commit_then_continue_reproduces_verify(a):
    rng = np.random.default_rng(104 + a)
    N, m, H, dk, dv = 3, 5, 2, 10, 12
    q, k, v, la, bt, S = _inputs(rng, N, m, H, dk, dv, la_scale=0.2)
    o_all = oracle.spec_verify(q, k, v, la, bt, S)
    S_a = oracle.spec_commit(q, k, v, la, bt, S, np.full(N, a))
    o_rest = oracle.spec_verify(q[:, a:], k[:, a:], v[:, a:], la[:, a:], bt[:, a:], S_a)
    assert _rel(o_rest, o_all[:, a:]) < 1e-12


# ------------------------------------------------------------- planted mistakes
def _commit_all(q, k, v, la, bt, S, accepted, nthreads=None):
    return oracle.prefill(q, k, v, la, bt, S)[1]


def _commit_no_clamp(q, k, v, la, bt, S, accepted, nthreads=None):
    acc = np.asarray(accepted)
    return _REAL_COMMIT(q, k, v, la, bt, S, np.where(acc < 0, 1, acc))


def _commit_off_by_one(q, k, v, la, bt, S, accepted, nthreads=None):
    return _REAL_COMMIT(q, k, v, la, bt, S, np.maximum(np.asarray(accepted) - 1, 0))


def _verify_from_advanced_state(q, k, v, la, bt, S, nthreads=None):
    S1 = oracle.prefill(q[:, :1], k[:, :1], v[:, :1], la[:, :1], bt[:, :1], S)[1]
    return oracle.prefill(q, k, v, la, bt, S1)[0]


def _verify_mutates_state(q, k, v, la, bt, S, nthreads=None):
    o, st = oracle.prefill(q, k, v, la, bt, S)
    S[...] = st
    return o


_REAL_COMMIT = oracle.spec_commit
_REAL_VERIFY = oracle.spec_verify
MUTANTS = {
    "commit_every_drafted_token": ("spec_commit", _commit_all),
    "commit_without_lower_clamp": ("spec_commit", _commit_no_clamp),
    "commit_drops_last_accepted": ("spec_commit", _commit_off_by_one),
    "verify_from_advanced_state": ("spec_verify", _verify_from_advanced_state),
    "verify_mutates_state": ("spec_verify", _verify_mutates_state),
}
PINS = [test_commit_retrieves_accepted_and_keeps_rejected, test_verify_is_stepwise_and_leaves_state,
        test_commit_limits_and_clamp] + [lambda a=a: test_commit_then_continue_reproduces_verify(a)
                                         for a in (1, 2, 4)]


@pytest.mark.parametrize("mutant", sorted(MUTANTS))
def test_spec_mutant_is_caught(mutant, monkeypatch):
    attr, fn = MUTANTS[mutant]
    monkeypatch.setattr(oracle, attr, fn)
    caught = 0
    for pin in PINS:
        try:
            pin()
        except AssertionError:
            caught += 1
    assert caught, f"no pin catches the mutant {mutant}"
