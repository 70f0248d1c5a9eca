"""Pins for the float64 oracle (CPU only).

No page prints a worked KDA example, so the oracle is pinned to what the
definition and the mathematics fix, each chosen so that a plausible slip in the
oracle (decay after the write, error taken on the undecayed state, read before
the write, gate on the value axis, a transposed read, a wrong sign or beta
factor, a wrong clamp, a batch/head indexing error) fails at least one test:

* brute-force unrolled sums of explicit transition matrices (T <= 8);
* one step is one LMS / Widrow-Hoff gradient step on the decayed state, with the
  gradient taken by central finite differences;
* beta = 1 retrieves the value just written under a unit key, for any decay;
* orthonormal keys with alpha = 1, beta = 1 retrieve every stored value;
* beta = 0 is pure per-key-channel decay (closed form with the cumulative sum);
* the clamp of log alpha to [-5, 0] and the pages' constants;
* chunk-size independence and segment composition against the independent
  block form in ``chunk_algebra``;
* linearity in (V, S0), state-column independence, padding tokens, splitting
  a prefill at any token, batch/head independence and the contraction bound.
"""
import math
import os

import numpy as np
import pytest

import oracle
from tests import chunk_algebra as ca

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand_inputs(rng, B, T, H, dk, dv, unit_keys=True, la_scale=1.0, beta_hi=1.0):
    q = rng.standard_normal((B, T, H, dk))
    k = rng.standard_normal((B, T, H, dk))
    if unit_keys:
        q /= np.linalg.norm(q, axis=-1, keepdims=True)
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((B, T, H, dv))
    la = -la_scale * rng.random((B, T, H, dk)) * 5.0
    bt = beta_hi * rng.random((B, T, H))
    S0 = rng.standard_normal((B, H, dk, dv))
    return q, k, v, la, bt, S0


def _rel(x, y):
    return np.linalg.norm(x - y) / max(np.linalg.norm(y), 1e-300)


# ---------------------------------------------------------------- brute force
def _bruteforce_head(q, k, v, la, bt, S0):
    """S_t = Phi_{t,0} S0 + sum_i Phi_{t,i} beta_i k_i v_i^T with
    Phi_{t,i} = M_t M_{t-1} ... M_{i+1},  M_j = (I - beta_j k_j k_j^T) Diag(alpha_j).
    Every product is formed as an explicit d_k x d_k matrix."""
    T, dk = k.shape
    Ms = []
    for j in range(T):
        a = np.exp(np.clip(la[j], -5.0, 0.0))
        Ms.append((np.eye(dk) - bt[j] * np.outer(k[j], k[j])) @ np.diag(a))

    def phi(t, i):  # product M_t ... M_{i+1} (1-based t, i)
        P = np.eye(dk)
        for j in range(i + 1, t + 1):
            P = Ms[j - 1] @ P
        return P

    o = np.zeros((T, v.shape[1]))
    St = None
    for t in range(1, T + 1):
        St = phi(t, 0) @ S0
        for i in range(1, t + 1):
            St = St + phi(t, i) @ (bt[i - 1] * np.outer(k[i - 1], v[i - 1]))
        o[t - 1] = St.T @ q[t - 1]
    return o, St


@pytest.mark.parametrize("T,dk,dv", [(1, 3, 2), (4, 5, 3), (8, 4, 6), (7, 6, 6)])
def test_bruteforce_unrolled_sums(T, dk, dv):
    rng = np.random.default_rng(100 + T * 10 + dk)
    q, k, v, la, bt, S0 = _rand_inputs(rng, 2, T, 3, dk, dv, unit_keys=False)
    la[0, 0, 0, :2] = [-7.0, 0.5]             # out-of-range values exercise the clamp
    o, st = oracle.prefill(q, k, v, la, bt, S0)
    for b in range(2):
        for h in range(3):
            ob, sb = _bruteforce_head(q[b, :, h], k[b, :, h], v[b, :, h], la[b, :, h],
                                      bt[b, :, h], S0[b, h])
            np.testing.assert_allclose(o[b, :, h], ob, rtol=1e-11, atol=1e-12)
            np.testing.assert_allclose(st[b, h], sb, rtol=1e-11, atol=1e-12)


# ------------------------------------------------------------- LMS / textbook
def test_one_step_is_lms_gradient_step_on_decayed_state():
    """Delta rule = one gradient step of L(S) = 1/2 ||S^T k - v||^2 with step beta, taken
    on the decayed state S' = Diag(alpha) S.  Gradient by central differences."""
    rng = np.random.default_rng(7)
    dk, dv = 5, 4
    S = rng.standard_normal((dk, dv))
    k = rng.standard_normal(dk)
    v = rng.standard_normal(dv)
    q = rng.standard_normal(dk)
    la = -rng.random(dk) * 3.0
    beta = 0.37
    Sd = np.exp(la)[:, None] * S

    def loss(X):
        r = X.T @ k - v
        return 0.5 * float(r @ r)

    eps = 1e-5
    grad = np.zeros_like(Sd)
    for i in range(dk):
        for j in range(dv):
            E = np.zeros_like(Sd)
            E[i, j] = eps
            grad[i, j] = (loss(Sd + E) - loss(Sd - E)) / (2 * eps)
    expect = Sd - beta * grad
    o, st = oracle.decode_step(q[None, None], k[None, None], v[None, None], la[None, None],
                               np.array([[beta]]), S[None, None])
    np.testing.assert_allclose(st[0, 0], expect, rtol=1e-8, atol=1e-9)
    np.testing.assert_allclose(o[0, 0], expect.T @ q, rtol=1e-8, atol=1e-9)


def test_beta_one_retrieves_last_written_value_any_decay():
    """beta = 1, ||k_t|| = 1: the write fully corrects the decayed state, so S_t^T k_t = v_t,
    and reading with q_t = k_t returns v_t (read happens after the write)."""
    rng = np.random.default_rng(11)
    B, T, H, dk, dv = 1, 9, 2, 6, 5
    q, k, v, la, bt, S0 = _rand_inputs(rng, B, T, H, dk, dv)
    bt[:] = 1.0
    q = k.copy()
    o, st = oracle.prefill(q, k, v, la, bt, S0)
    np.testing.assert_allclose(o, v, rtol=1e-12, atol=1e-12)
    for h in range(H):
        np.testing.assert_allclose(st[0, h].T @ k[0, -1, h], v[0, -1, h], atol=1e-12)


def test_orthonormal_keys_exact_retrieval():
    """alpha = 1, beta = 1 and orthonormal keys: every stored value is retrieved exactly,
    whatever S0 held (the textbook delta rule with unit step)."""
    rng = np.random.default_rng(3)
    dk, dv, T = 8, 5, 6
    Qm, _ = np.linalg.qr(rng.standard_normal((dk, dk)))
    k = Qm[:, :T].T.reshape(1, T, 1, dk)
    v = rng.standard_normal((1, T, 1, dv))
    la = np.zeros((1, T, 1, dk))
    bt = np.ones((1, T, 1))
    S0 = rng.standard_normal((1, 1, dk, dv))
    q = rng.standard_normal((1, T, 1, dk))
    _, st = oracle.prefill(q, k, v, la, bt, S0)
    for i in range(T):
        np.testing.assert_allclose(st[0, 0].T @ k[0, i, 0], v[0, i, 0], atol=1e-12)
    # directions orthogonal to every key keep S0's content untouched
    P = np.eye(dk) - k[0, :, 0].T @ k[0, :, 0]
    np.testing.assert_allclose(P @ st[0, 0], P @ S0[0, 0], atol=1e-12)


def test_beta_zero_is_pure_channel_decay():
    rng = np.random.default_rng(5)
    B, T, H, dk, dv = 2, 11, 2, 6, 4
    q, k, v, la, bt, S0 = _rand_inputs(rng, B, T, H, dk, dv, unit_keys=False)
    bt[:] = 0.0
    o, st = oracle.prefill(q, k, v, la, bt, S0)
    g = np.cumsum(np.clip(la, -5, 0), axis=1)                       # [B, T, H, dk]
    np.testing.assert_allclose(st, np.exp(g[:, -1])[..., None] * S0, rtol=1e-12)
    expect_o = np.einsum("bhij,bthi->bthj", S0, np.exp(g) * q)
    np.testing.assert_allclose(o, expect_o, rtol=1e-11, atol=1e-13)


# ---------------------------------------------------------------- the bound
def _golden_constants():
    vals = {}
    with open(os.path.join(GOLDEN, "decay_bound.txt")) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                name, val = line.split()
                vals[name] = float(val)
    return vals


def test_pages_decay_constants():
    c = _golden_constants()
    assert round(100 * math.exp(c["log_alpha_min"]), 2) == c["min_retention_percent"]
    assert c["tile_tokens"] * c["log_alpha_min"] == c["tile_log_decay_min"]
    recip = math.exp(-c["tile_log_decay_min"])
    assert abs(recip / c["reciprocal_bound"] - 1) < 0.01
    bf16_max = (2 - 2 ** -7) * 2.0 ** 127
    assert abs(bf16_max / c["bf16_range"] - 1) < 0.01 and recip < bf16_max
    fp16_max = 65504.0
    assert math.log(fp16_max) < -c["tile_log_decay_min"]   # fp16 cannot hold e^80


def test_clamp_of_log_alpha():
    """Out-of-range log alpha acts as the nearest bound: one beta = 0 step keeps exactly
    e^-5 (0.67%) of S for log alpha = -100 and all of it for log alpha = +2."""
    c = _golden_constants()
    S = np.ones((1, 1, 2, 3))
    la = np.array([[[-100.0, 2.0]]])
    o, st = oracle.decode_step(np.zeros((1, 1, 2)), np.zeros((1, 1, 2)), np.zeros((1, 1, 3)),
                               la, np.zeros((1, 1)), S)
    assert np.allclose(st[0, 0, 0], math.exp(c["log_alpha_min"]), rtol=1e-15)
    assert np.allclose(st[0, 0, 1], 1.0, rtol=0, atol=0)
    rng = np.random.default_rng(9)
    q, k, v, la, bt, S0 = _rand_inputs(rng, 1, 6, 1, 4, 3)
    la2 = la.copy()
    la2[0, 1] = -50.0
    la2[0, 3] = 7.0
    la3 = la.copy()
    la3[0, 1] = -5.0
    la3[0, 3] = 0.0
    a = oracle.prefill(q, k, v, la2, bt, S0)
    b = oracle.prefill(q, k, v, la3, bt, S0)
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_array_equal(a[1], b[1])


# ---------------------------------------------------- chunk form, segments
@pytest.mark.parametrize("chunk", [1, 2, 4, 8, 16, 32, 64])
def test_chunk_size_independence(chunk):
    rng = np.random.default_rng(21)
    q, k, v, la, bt, S0 = _rand_inputs(rng, 1, 150, 2, 16, 8)
    o_ref, s_ref = oracle.prefill(q, k, v, la, bt, S0)
    o, s = ca.prefill(q, k, v, la, bt, S0, chunk=chunk, tile=16)
    assert _rel(o, o_ref) < 1e-12 and _rel(s, s_ref) < 1e-12


@pytest.mark.parametrize("chunk", [16, 64])
def test_chunk_form_at_the_decay_bound(chunk):
    """Every log alpha = -5: the diagonal tile's column factor reaches exactly e^80."""
    rng = np.random.default_rng(22)
    q, k, v, la, bt, S0 = _rand_inputs(rng, 1, 130, 1, 16, 8)
    la[:] = -5.0
    o_ref, s_ref = oracle.prefill(q, k, v, la, bt, S0)
    o, s = ca.prefill(q, k, v, la, bt, S0, chunk=chunk, tile=16)
    assert _rel(o, o_ref) < 1e-12 and _rel(s, s_ref) < 1e-12


def test_slow_decay_hand_off():
    """Long memory (log alpha ~ -0.05 sigmoid): S0 and early chunks still matter at the end."""
    rng = np.random.default_rng(23)
    q, k, v, la, bt, S0 = _rand_inputs(rng, 1, 300, 1, 16, 8, la_scale=0.001, beta_hi=0.1)
    o_ref, s_ref = oracle.prefill(q, k, v, la, bt, S0)
    o, s = ca.prefill(q, k, v, la, bt, S0, chunk=64, tile=16)
    assert _rel(o, o_ref) < 1e-12 and _rel(s, s_ref) < 1e-12
    _, s_zero = oracle.prefill(q, k, v, la, bt, None)
    assert _rel(s_ref, s_zero) > 0.1             # S0 is still visible after 300 tokens


def test_segment_composition():
    """S_out = M S_in + H per segment, with M = run on identity columns and zero values and
    H = run from zero; the scan over segments reproduces the sequential states."""
    rng = np.random.default_rng(24)
    T, seg, dk, dv = 300, 64, 8, 6
    q, k, v, la, bt, S0 = _rand_inputs(rng, 1, T, 1, dk, dv, la_scale=0.02)
    o_ref, s_ref = oracle.prefill(q, k, v, la, bt, S0)
    K, V, L, Bt = k[0, :, 0], v[0, :, 0], la[0, :, 0], bt[0, :, 0]
    Ms, Hs, bounds = [], [], []
    for s0 in range(0, T, seg):
        s1 = min(T, s0 + seg)
        bounds.append((s0, s1))
        Ms.append(ca.segment_transition(K[s0:s1], L[s0:s1], Bt[s0:s1], chunk=16))
        Hs.append(ca.segment_increment(K[s0:s1], V[s0:s1], L[s0:s1], Bt[s0:s1], chunk=16))
    entries = ca.scan_entry_states(Ms, Hs, S0[0, 0])
    assert _rel(entries[-1], s_ref[0, 0]) < 1e-12
    for (s0, s1), Sin in zip(bounds, entries):
        o_seg, _ = oracle.prefill(q[:, s0:s1], k[:, s0:s1], v[:, s0:s1], la[:, s0:s1],
                                  bt[:, s0:s1], Sin[None, None])
        assert _rel(o_seg, o_ref[:, s0:s1]) < 1e-12
    # the oracle itself is affine in S0 with exactly this transition
    zeros_v = np.zeros((1, seg, 1, dk))
    _, M_or = oracle.prefill(np.zeros((1, seg, 1, dk)), k[:, :seg], zeros_v, la[:, :seg],
                             bt[:, :seg], np.eye(dk)[None, None])
    assert _rel(M_or[0, 0], Ms[0]) < 1e-12


# --------------------------------------------------------------- structure
def test_linearity_in_values_and_state():
    rng = np.random.default_rng(31)
    q, k, v1, la, bt, S1 = _rand_inputs(rng, 1, 40, 2, 6, 5)
    v2 = rng.standard_normal(v1.shape)
    S2 = rng.standard_normal(S1.shape)
    a, b = 0.7, -1.9
    o1, s1 = oracle.prefill(q, k, v1, la, bt, S1)
    o2, s2 = oracle.prefill(q, k, v2, la, bt, S2)
    o3, s3 = oracle.prefill(q, k, a * v1 + b * v2, la, bt, a * S1 + b * S2)
    np.testing.assert_allclose(o3, a * o1 + b * o2, atol=1e-12)
    np.testing.assert_allclose(s3, a * s1 + b * s2, atol=1e-12)


def test_state_columns_independent():
    rng = np.random.default_rng(32)
    q, k, v, la, bt, S0 = _rand_inputs(rng, 1, 50, 1, 6, 7)
    o, s = oracle.prefill(q, k, v, la, bt, S0, col_block=3)
    cols = [1, 4, 6]
    o2, s2 = oracle.prefill(q, k, v[..., cols], la, bt, S0[..., cols], col_block=32)
    np.testing.assert_allclose(o[..., cols], o2, atol=1e-13)
    np.testing.assert_allclose(s[..., cols], s2, atol=1e-13)


def test_batch_and_heads_independent():
    rng = np.random.default_rng(33)
    q, k, v, la, bt, S0 = _rand_inputs(rng, 2, 20, 3, 5, 4)
    o, s = oracle.prefill(q, k, v, la, bt, S0)
    for b in range(2):
        for h in range(3):
            sl = (slice(b, b + 1), slice(None), slice(h, h + 1))
            ob, sb = oracle.prefill(q[sl], k[sl], v[sl], la[sl], bt[b:b + 1, :, h:h + 1],
                                    S0[b:b + 1, h:h + 1])
            np.testing.assert_array_equal(o[b, :, h], ob[0, :, 0])
            np.testing.assert_array_equal(s[b, h], sb[0, 0])


def test_padding_tokens_are_identity():
    """k = 0, beta = 0, log alpha = 0 leaves S unchanged (how a tail chunk may be padded)."""
    rng = np.random.default_rng(34)
    q, k, v, la, bt, S0 = _rand_inputs(rng, 1, 13, 1, 6, 5)
    k[:, 5:9] = 0.0
    bt[:, 5:9] = 0.0
    la[:, 5:9] = 0.0
    o, s = oracle.prefill(q, k, v, la, bt, S0)
    keep = [i for i in range(13) if not 5 <= i < 9]
    o2, s2 = oracle.prefill(q[:, keep], k[:, keep], v[:, keep], la[:, keep], bt[:, keep], S0)
    np.testing.assert_allclose(s, s2, atol=1e-13)
    np.testing.assert_allclose(o[:, keep], o2, atol=1e-13)


@pytest.mark.parametrize("split", [1, 37, 64, 99])
def test_split_prefill_equals_whole(split):
    rng = np.random.default_rng(35)
    q, k, v, la, bt, S0 = _rand_inputs(rng, 1, 100, 2, 6, 5)
    o, s = oracle.prefill(q, k, v, la, bt, S0)
    a = slice(0, split)
    b = slice(split, None)
    o1, s1 = oracle.prefill(q[:, a], k[:, a], v[:, a], la[:, a], bt[:, a], S0)
    o2, s2 = oracle.prefill(q[:, b], k[:, b], v[:, b], la[:, b], bt[:, b], s1)
    np.testing.assert_allclose(np.concatenate([o1, o2], axis=1), o, atol=1e-12)
    np.testing.assert_allclose(s2, s, atol=1e-12)


def test_contraction_bound():
    """Unit keys and beta in [0, 2]: each transition has spectral norm <= 1, so
    ||S_T||_F <= ||S0||_F + sum_t |beta_t| ||v_t||."""
    rng = np.random.default_rng(36)
    q, k, v, la, bt, S0 = _rand_inputs(rng, 1, 200, 1, 8, 8, beta_hi=2.0)
    _, s = oracle.prefill(q, k, v, la, bt, S0)
    bound = np.linalg.norm(S0) + np.sum(np.abs(bt[0, :, 0]) * np.linalg.norm(v[0, :, 0], axis=-1))
    assert np.linalg.norm(s) <= bound


def test_empty_sequence_returns_initial_state():
    rng = np.random.default_rng(37)
    q, k, v, la, bt, S0 = _rand_inputs(rng, 1, 0, 2, 4, 3)
    o, s = oracle.prefill(q, k, v, la, bt, S0)
    assert o.shape == (1, 0, 2, 3)
    np.testing.assert_array_equal(s, S0)


def test_chunk_algebra_blocked_inverse():
    rng = np.random.default_rng(38)
    n = 64
    A = np.tril(rng.standard_normal((n, n)) * 0.1, -1)
    Tm = ca.unit_lower_inverse_blocked(A, 16)
    np.testing.assert_allclose(Tm @ (np.eye(n) + A), np.eye(n), atol=1e-12)
