"""Float64 NumPy reference of the block-parallel (chunked) form.

TEST INFRASTRUCTURE ONLY (same import rules as the rest of ``oracle/``).

The page "Inside Qwen3.8-27B: Hybrid DeltaNet Architecture, 256k Context, and
24GB Local Serving" (note under "The Role of Periodic Gated Attention") says
that prefill rewrites the token-sequential update into a block-parallel matrix
form.  The page does not spell the rewrite out.  This module writes down the
plainest such rewrite, derived directly from the recurrence

    S_t = alpha_t S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,  o_t = S_t q_t

and exists so that the tests can show, in float64, that it reaches the same
result as the sequential oracle (to rounding) before any GPU kernel relies on
it.  It is not the oracle: the oracle is the sequential definition.

Derivation (one chunk of L tokens, local index i = 0..L-1, incoming state S0):

    one step:  S_i = alpha_i S_{i-1} + d_i k_i^T,
               d_i = beta_i (v_i - alpha_i S_{i-1} k_i)
    gates:     G_i = sum_{j<=i} ln alpha_j,  gamma_i = exp(G_i),
               Gam_ij = exp(G_i - G_j) for j <= i, else 0 (masked before exp)
    unrolled:  S_i = gamma_i S0 + sum_{j<=i} Gam_ij d_j k_j^T
    so         d_i + sum_{j<i} beta_i Gam_ij (k_i.k_j) d_j
                   = beta_i v_i - beta_i gamma_i S0 k_i
    matrix form (rows are tokens):
               A   = strict_lower(diag(beta) (K K^T * Gam))
               Tm  = (I + A)^-1                 (unit lower triangular)
               U   = Tm diag(beta) V,   W = Tm diag(beta*gamma) K
               Dl  = U - W S0^T                 (row i = d_i^T)
               O   = diag(gamma) Q S0^T + (Q K^T * Gam_incl) Dl
               S_L = gamma_{L-1} S0 + Dl^T diag(Gam_{L-1, .}) K

Value head h reads query/key head h // (Hv // Hqk).

Backward of one chunk (for the training pass; same page and note: training
uses the block-parallel form too).  With N = (I + A)^-1 (so Tm diag(beta) =
N diag(beta)), X = V - diag(gamma) K S0^T, Dl = N diag(beta) X,
M = Q K^T * Gam_incl and dec_i = Gam_{L-1, i}, and given dO = dL/dO and
dS_L = dL/dS_L:

    dDl = M^T dO + diag(dec) K dS_L^T
    Y   = N^T dDl,          dX = diag(beta) Y = dV
    dS0 = gamma_{L-1} dS_L + dO^T diag(gamma) Q - dX^T diag(gamma) K
    dM  = tril(dO Dl^T)                        (diagonal included)
    dA  = -strict_lower(Y Dl^T)
    dQ  = diag(gamma) dO S0 + (dM * Gam) K
    dK  = -diag(gamma) dX S0 + diag(dec) Dl dS_L + (dM * Gam)^T Q
          + Wa K + Wa^T K,          Wa = diag(beta) (dA * Gam)
    dbeta_i = Y_i . X_i + sum_j dA_ij Gam_ij (k_i . k_j)
    gates (every gate enters through G = cumsum ln alpha):
      dG_i = gamma_i dO_i.(S0 q_i) - gamma_i dX_i.(S0 k_i)
             + rowsum_i(P) - colsum_i(P)     for P = dM * M and P = dA * A
             - w_i,   w_i = dec_i Dl_i.(dS_L k_i)
      dG_{L-1} += sum_i w_i + gamma_{L-1} <dS_L, S0>
      d ln alpha_j = sum_{i >= j} dG_i,   dalpha_j = d ln alpha_j / alpha_j
"""
from __future__ import annotations

import numpy as np


def _f64(x):
    if hasattr(x, "detach"):
        x = x.detach().cpu().float().numpy()
    return np.asarray(x, dtype=np.float64)


def chunk_step(Qc, Kc, Vc, ac, bc, S0, stages=None):
    """One chunk for one value head.  Qc, Kc, Vc ``[L, D]``; ac, bc ``[L]``;
    S0 ``[Dv, Dk]``.  Returns ``(O [L, Dv], S_L [Dv, Dk])``.  When ``stages``
    is a dict, the intermediate quantities are stored in it."""
    L = Qc.shape[0]
    Gc = np.cumsum(np.log(ac))
    gamma = np.exp(Gc)
    diff = Gc[:, None] - Gc[None, :]
    incl = np.tril(np.ones((L, L), dtype=bool))
    Gam = np.where(incl, np.exp(np.where(incl, diff, 0.0)), 0.0)
    A = np.tril(bc[:, None] * (Kc @ Kc.T) * Gam, k=-1)
    Tm = np.linalg.solve(np.eye(L) + A, np.eye(L))
    U = Tm @ (bc[:, None] * Vc)
    W = Tm @ ((bc * gamma)[:, None] * Kc)
    Dl = U - W @ S0.T
    O = gamma[:, None] * (Qc @ S0.T) + ((Qc @ Kc.T) * Gam) @ Dl
    S_L = gamma[-1] * S0 + Dl.T @ (Gam[-1][:, None] * Kc)
    if stages is not None:
        stages.update(G=Gc, gamma=gamma, Gam=Gam, A=A, T=Tm, U=U, W=W,
                      Delta=Dl, O=O, S=S_L)
    return O, S_L


def chunk_backward(Qc, Kc, Vc, ac, bc, S0, dOc, dSL):
    """Backward of :func:`chunk_step` for one value head.  Returns
    ``(dQ, dK, dV, dalpha, dbeta, dS0)`` given ``dOc = dL/dO`` ``[L, Dv]``
    and ``dSL = dL/dS_L`` ``[Dv, Dk]`` (formulas in the module docstring)."""
    L = Qc.shape[0]
    Gc = np.cumsum(np.log(ac))
    gamma = np.exp(Gc)
    diff = Gc[:, None] - Gc[None, :]
    incl = np.tril(np.ones((L, L), dtype=bool))
    Gam = np.where(incl, np.exp(np.where(incl, diff, 0.0)), 0.0)
    KK = Kc @ Kc.T
    A = np.tril(bc[:, None] * KK * Gam, k=-1)
    N = np.linalg.solve(np.eye(L) + A, np.eye(L))
    KS = Kc @ S0.T
    X = Vc - gamma[:, None] * KS
    Dl = N @ (bc[:, None] * X)
    Mm = (Qc @ Kc.T) * Gam
    dec = Gam[-1]
    KdS = Kc @ dSL.T
    dDl = Mm.T @ dOc + dec[:, None] * KdS
    Y = N.T @ dDl
    dX = bc[:, None] * Y
    dS0 = gamma[-1] * dSL + dOc.T @ (gamma[:, None] * Qc) - dX.T @ (gamma[:, None] * Kc)
    dM = np.tril(dOc @ Dl.T)
    dA = -np.tril(Y @ Dl.T, k=-1)
    dQ = gamma[:, None] * (dOc @ S0) + (dM * Gam) @ Kc
    Wa = bc[:, None] * dA * Gam
    dK = (-gamma[:, None] * (dX @ S0) + dec[:, None] * (Dl @ dSL)
          + (dM * Gam).T @ Qc + Wa @ Kc + Wa.T @ Kc)
    dbeta = np.sum(Y * X, axis=1) + np.sum(dA * Gam * KK, axis=1)
    dG = (gamma * np.sum(dOc * (Qc @ S0.T), axis=1)
          - gamma * np.sum(dX * KS, axis=1))
    for P in (dM * Mm, dA * A):
        dG += P.sum(axis=1) - P.sum(axis=0)
    w = dec * np.sum(Dl * KdS, axis=1)
    dG -= w
    dG[-1] += w.sum() + gamma[-1] * np.sum(dSL * S0)
    dlog = np.cumsum(dG[::-1])[::-1]
    return dQ, dK, dX, dlog / ac, dbeta, dS0


def chunked_backward(q, k, v, alpha, beta, do, h0=None, dht=None, C=64):
    """Chunked evaluation of the prefill's gradients (same layouts and
    outputs as ``oracle.prefill_backward``): a forward sweep keeps the state
    entering every chunk, a reverse sweep carries dL/dS from chunk to chunk."""
    q, k, v, alpha, beta, do = (_f64(x) for x in (q, k, v, alpha, beta, do))
    B, T, Hqk, D = q.shape
    Hv = v.shape[2]
    G = Hv // Hqk
    dq = np.zeros((B, T, Hqk, D))
    dk = np.zeros((B, T, Hqk, D))
    dv = np.zeros((B, T, Hv, D))
    da = np.zeros((B, T, Hv))
    db = np.zeros((B, T, Hv))
    dh0 = np.zeros((B, Hv, D, D))
    starts = list(range(0, T, C))
    for b in range(B):
        for h in range(Hv):
            g = h // G
            S = np.zeros((D, D)) if h0 is None else _f64(h0)[b, h].copy()
            Ss = []
            for s in starts:
                e = min(s + C, T)
                Ss.append(S)
                _, S = chunk_step(q[b, s:e, g], k[b, s:e, g], v[b, s:e, h],
                                  alpha[b, s:e, h], beta[b, s:e, h], S)
            dS = np.zeros((D, D)) if dht is None else _f64(dht)[b, h].copy()
            for s, S0 in reversed(list(zip(starts, Ss))):
                e = min(s + C, T)
                gq, gk, gv, ga, gb, dS = chunk_backward(
                    q[b, s:e, g], k[b, s:e, g], v[b, s:e, h], alpha[b, s:e, h],
                    beta[b, s:e, h], S0, do[b, s:e, h], dS)
                dq[b, s:e, g] += gq
                dk[b, s:e, g] += gk
                dv[b, s:e, h] = gv
                da[b, s:e, h] = ga
                db[b, s:e, h] = gb
            dh0[b, h] = dS
    return dq, dk, dv, da, db, dh0


def chunked_prefill(q, k, v, alpha, beta, h0=None, C=64):
    """Chunked evaluation of the whole prefill, same layouts as
    ``oracle.prefill``: q, k ``[B,T,Hqk,D]``; v ``[B,T,Hv,D]``; alpha, beta
    ``[B,T,Hv]``; h0 ``[B,Hv,D,D]`` or None.  Chunks of C tokens; the last
    chunk may be shorter."""
    q, k, v, alpha, beta = (_f64(x) for x in (q, k, v, alpha, beta))
    B, T, Hqk, D = q.shape
    Hv = v.shape[2]
    G = Hv // Hqk
    o = np.zeros((B, T, Hv, D))
    ht = np.zeros((B, Hv, D, D))
    for b in range(B):
        for h in range(Hv):
            g = h // G
            S = np.zeros((D, D)) if h0 is None else _f64(h0)[b, h].copy()
            for s in range(0, T, C):
                e = min(s + C, T)
                O, S = chunk_step(q[b, s:e, g], k[b, s:e, g], v[b, s:e, h],
                                  alpha[b, s:e, h], beta[b, s:e, h], S)
                o[b, s:e, h] = O
            ht[b, h] = S
    return o, ht
