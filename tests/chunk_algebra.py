"""Chunked (UT/WY) form of the KDA recurrence in float64 NumPy — test helper only.

This is an independent derivation of the same result the token-by-token oracle
computes, written as block linear algebra: a pin for the oracle (chunk-size
independence, segment composition) and a model of the factorisation that the
device kernels use.  It shares no code with either.

Derivation, for one chunk of n tokens entering with state S (d_k x d_v), with
g_r = sum_{j<=r} log alpha_j (inclusive, per key channel) and u_i the
beta-scaled error written at token i:

    S_r   = Diag(e^{g_r}) S + sum_{i<=r} Diag(e^{g_r - g_i}) k_i u_i^T
    u_i   = beta_i (v_i - S'_i^T k_i),   S'_i = Diag(e^{g_i - g_{i-1}}) S_{i-1}
  =>  (I + A) U = Diag(beta) (V - K~ S),   A_ri = beta_r <k_r e^{g_r - g_i}, k_i>  (i < r)
      O = Q~ S + Bqk U,                    Bqk_ri = <q_r e^{g_r - g_i}, k_i>      (i <= r)
      S_next = Diag(e^{g_n}) S + K'^T U,   K'_i = k_i e^{g_n - g_i}
  with K~ = k e^{g}, Q~ = q e^{g}.

The pair-wise decay e^{g_r - g_i} is factored per row tile a of ``tile`` tokens
around the reference rho_a = g at the token before the tile: the row factor
e^{g_r - rho_a} is at most 1 and the column factor e^{rho_a - g_i} is at most
e^{5 * tile} on the diagonal tile and at most 1 on earlier tiles.  With the
decay bound log alpha >= -5 and 16-token tiles this is the (-80, 0) range of
"Kimi K3's architecture" (orkas.ai), section "A lower bound that deleted a GPU
code path", which lets diagonal and off-diagonal tiles share one dense product.

(I + A)^{-1} is formed blockwise: forward substitution inside each diagonal
tile, then T_ab = -T_aa sum_{c=b}^{a-1} A_ac T_cb below the diagonal.
"""
from __future__ import annotations

import numpy as np

LOG_ALPHA_MIN = -5.0


def _clamp(la):
    return np.clip(la, LOG_ALPHA_MIN, 0.0)


def unit_lower_inverse_blocked(A: np.ndarray, tile: int) -> np.ndarray:
    """(I + A)^{-1} for strictly lower-triangular A, blockwise by ``tile``."""
    n = A.shape[0]
    nt = (n + tile - 1) // tile
    Tm = np.zeros((n, n))
    blk = [(a * tile, min((a + 1) * tile, n)) for a in range(nt)]
    for a, (r0, r1) in enumerate(blk):          # diagonal tiles: forward substitution
        m = r1 - r0
        Ta = np.zeros((m, m))
        for r in range(m):
            Ta[r, r] = 1.0
            for i in range(r):
                Ta[r, :] -= A[r0 + r, r0 + i] * Ta[i, :]
        Tm[r0:r1, r0:r1] = Ta
    for d in range(1, nt):                      # then below the diagonal, band by band
        for a in range(d, nt):
            b = a - d
            (ra0, ra1), (rb0, rb1) = blk[a], blk[b]
            acc = np.zeros((ra1 - ra0, rb1 - rb0))
            for c in range(b, a):
                rc0, rc1 = blk[c]
                acc += A[ra0:ra1, rc0:rc1] @ Tm[rc0:rc1, rb0:rb1]
            Tm[ra0:ra1, rb0:rb1] = -Tm[ra0:ra1, ra0:ra1] @ acc
    return Tm


def chunk_step(Q, K, V, lam, bt, S, tile=16):
    """One chunk of n tokens: returns (O [n, dv], S_next [dk, dv])."""
    n = K.shape[0]
    lam = _clamp(lam)
    tau = min(tile, n)
    g = np.cumsum(lam, axis=0)
    nt = (n + tau - 1) // tau
    A = np.zeros((n, n))
    Bqk = np.zeros((n, n))
    for a in range(nt):
        r0, r1 = a * tau, min((a + 1) * tau, n)
        rho = g[r0 - 1] if r0 > 0 else np.zeros(K.shape[1])
        x = np.exp(g[r0:r1] - rho)              # row factors, <= 1
        R = K[:r1] * np.exp(rho - g[:r1])       # column factors, <= e^{5 tau} on the diagonal tile
        Ablk = (K[r0:r1] * x) @ R.T
        Bblk = (Q[r0:r1] * x) @ R.T
        for rr in range(r1 - r0):
            r = r0 + rr
            A[r, :r] = bt[r] * Ablk[rr, :r]
            Bqk[r, :r + 1] = Bblk[rr, :r + 1]
    Tm = unit_lower_inverse_blocked(A, tau)
    Kt = K * np.exp(g)
    Qt = Q * np.exp(g)
    Kp = K * np.exp(g[-1] - g)
    X = Kt @ S
    U = Tm @ (bt[:, None] * (V - X))
    O = Qt @ S + Bqk @ U
    S_next = np.exp(g[-1])[:, None] * S + Kp.T @ U
    return O, S_next


def prefill_head(q, k, v, la, bt, S0, chunk, tile=16):
    """One (b, h): q, k, la [T, dk]; v [T, dv]; bt [T]; S0 [dk, dv]."""
    T = q.shape[0]
    S = np.array(S0, dtype=np.float64, copy=True)
    O = np.zeros((T, v.shape[1]))
    for c0 in range(0, T, chunk):
        c1 = min(T, c0 + chunk)
        O[c0:c1], S = chunk_step(q[c0:c1], k[c0:c1], v[c0:c1], la[c0:c1], bt[c0:c1], S, tile)
    return O, S


def prefill(q, k, v, la, bt, S0, chunk, tile=16):
    """Batched wrapper with the library layouts ([B, T, H, d], S0 [B, H, dk, dv])."""
    q, k, v, la, bt = (np.asarray(x, dtype=np.float64) for x in (q, k, v, la, bt))
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    o = np.zeros((B, T, H, dv))
    st = np.zeros((B, H, dk, dv))
    for b in range(B):
        for h in range(H):
            s0 = np.zeros((dk, dv)) if S0 is None else np.asarray(S0[b, h], dtype=np.float64)
            o[b, :, h], st[b, h] = prefill_head(q[b, :, h], k[b, :, h], v[b, :, h],
                                                la[b, :, h], bt[b, :, h], s0, chunk, tile)
    return o, st


def segment_transition(k, la, bt, chunk, tile=16):
    """M with S_out = M S_in + H over a segment: the recurrence run on identity columns with
    zero values."""
    dk = k.shape[1]
    zeros_v = np.zeros((k.shape[0], dk))
    _, M = prefill_head(np.zeros_like(k), k, zeros_v, la, bt, np.eye(dk), chunk, tile)
    return M


def segment_increment(k, v, la, bt, chunk, tile=16):
    """H: the segment's end state from a zero start."""
    _, Hs = prefill_head(np.zeros_like(k), k, v, la, bt, np.zeros((k.shape[1], v.shape[1])),
                         chunk, tile)
    return Hs


def scan_entry_states(Ms, Hs, S0):
    """Entry state of every segment: S_in(0) = S0, S_in(s+1) = M_s S_in(s) + H_s."""
    out = [np.array(S0, dtype=np.float64)]
    for M, Hs_ in zip(Ms, Hs):
        out.append(M @ out[-1] + Hs_)
    return out
