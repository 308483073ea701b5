"""Float64 CPU oracle for the gated attention layer of the hybrid stack.

TEST INFRASTRUCTURE ONLY (same import rules as the rest of ``oracle/``: only
the tests, the smoke check and the benchmark's CPU-baseline leg use it; it
shares nothing with the HIP library).

What it computes, from the projected per-head activations of one layer
(projection weights are not part of this layer's hot path):

* Shapes: 24 query heads and 4 key/value heads of head dim 256; query head h
  reads key/value head h // 6 (page "Inside Qwen3.8-27B: Hybrid DeltaNet
  Architecture, 256k Context, and 24GB Local Serving", section "The Role of
  Periodic Gated Attention"; page "Qwen 3.8 27B Review ...", section 3;
  grouped-query attention as the card "Qwen3.8 (27B)" describes it under
  "Architecture concepts").
* QK-Norm: an RMSNorm of every query and key head vector before attention
  (card "Qwen3.8 (27B)", "Architecture concepts"): x / sqrt(mean(x^2) + eps)
  times a learned weight (ones when not given).
* Rotary position embedding on a 64-dimensional subspace with base
  theta = 10,000,000 (page "Inside Qwen3.8-27B ...", "The Role of Periodic
  Gated Attention").  Reading: the first 64 channels of each head rotate, in
  the pairing (j, j + 32) for j < 32, by the angle pos * theta^(-2j/64); the
  other 192 channels pass through.  Position of token t of a prefill is t.
* Causal softmax attention with scale 1/sqrt(256).
* Output gate: the attention output is multiplied channel by channel by
  sigmoid(gate), the gate logits being the second half of the fused q
  projection (page "Qwen3.8 Explained ...", the note on attn_output_gate:
  [12288, 5120] instead of [6144, 5120], half of it a multiplicative gate; the
  card's "Gated Attention": a learned sigmoid gate scales the attention output).

Everything is float64 NumPy in the order written above; inputs are widened
exactly.  The functions are the plain definitions, with no blocking.

Functions
---------
qk_norm(x, w, eps)                         RMSNorm over the last axis
rope(x, pos, rope_dim, theta)              partial rotary embedding
attention(q, k, v, gate, ...)              gated attention of a prefill
                                           (optionally only some rows/heads)
decode(q, k, v, gate, k_cache, v_cache, n) one token attending to a cache
"""
from __future__ import annotations

import numpy as np

HQ, HKV, DH, ROPE_DIM, THETA = 24, 4, 256, 64, 1.0e7


def _f64(x):
    if x is None:
        return None
    if hasattr(x, "detach"):
        x = x.detach().cpu().float().numpy()
    return np.asarray(x, dtype=np.float64)


def qk_norm(x, w=None, eps=1e-6):
    """RMSNorm over the last axis: x / sqrt(mean(x^2) + eps) * w."""
    x = _f64(x)
    y = x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)
    return y if w is None else y * _f64(w)


def rope(x, pos, rope_dim=ROPE_DIM, theta=THETA):
    """Rotate channels (j, j + rope_dim/2), j < rope_dim/2, of the last axis by
    pos * theta^(-2j/rope_dim).  ``pos`` broadcasts against ``x.shape[:-1]``
    (for x [B, T, H, D] with token positions p [T], pass p[:, None])."""
    x = _f64(x).copy()
    if rope_dim == 0:
        return x
    half = rope_dim // 2
    j = np.arange(half, dtype=np.float64)
    inv = theta ** (-2.0 * j / rope_dim)
    ang = np.asarray(pos, dtype=np.float64)[..., None] * inv
    c, s = np.cos(ang), np.sin(ang)
    a, b = x[..., :half].copy(), x[..., half:rope_dim].copy()
    x[..., :half] = a * c - b * s
    x[..., half:rope_dim] = b * c + a * s
    return x


def _prep(q, k, qw, kw, eps, rope_dim, theta, pos_q, pos_k):
    qn = qk_norm(q, qw, eps)
    kn = qk_norm(k, kw, eps)
    return rope(qn, pos_q, rope_dim, theta), rope(kn, pos_k, rope_dim, theta)


def attention(q, k, v, gate, q_norm_w=None, k_norm_w=None, eps=1e-6, rope_dim=ROPE_DIM,
              theta=THETA, rows=None, heads=None):
    """Gated attention of a prefill of B sequences of T tokens starting at
    position 0.  q, gate ``[B,T,Hq,D]``; k, v ``[B,T,Hkv,D]``.  Returns float64
    o ``[B,T,Hq,D]`` (or ``[B,len(rows),len(heads),D]`` when rows/heads select
    a subset: each selected row attends to keys 0..row)."""
    q, k, v, gate = _f64(q), _f64(k), _f64(v), _f64(gate)
    B, T, Hq, D = q.shape
    Hkv = k.shape[2]
    G = Hq // Hkv
    rows = np.arange(T) if rows is None else np.asarray(rows)
    heads = np.arange(Hq) if heads is None else np.asarray(heads)
    pos = np.arange(T, dtype=np.float64)
    qr, kr = _prep(q[:, rows][:, :, heads], k, q_norm_w, k_norm_w, eps, rope_dim, theta,
                   pos[rows][:, None], pos[:, None])
    out = np.zeros((B, len(rows), len(heads), D))
    scale = 1.0 / np.sqrt(D)
    for b in range(B):
        for hi, h in enumerate(heads):
            g = h // G
            s = (qr[b, :, hi] @ kr[b, :, g].T) * scale          # [rows, T]
            mask = np.arange(T)[None, :] <= rows[:, None]
            s = np.where(mask, s, -np.inf)
            s = s - s.max(axis=1, keepdims=True)
            p = np.exp(s)
            p /= p.sum(axis=1, keepdims=True)
            o = p @ v[b, :, g]
            out[b, :, hi] = o / (1.0 + np.exp(-gate[b, rows][:, h]))
    return out


def decode(q, k, v, gate, k_cache, v_cache, n, q_norm_w=None, k_norm_w=None, eps=1e-6,
           rope_dim=ROPE_DIM, theta=THETA):
    """One new token per sequence at position n[b], attending to the n[b]
    cached keys/values (already normalised and rotated, as a prefill leaves
    them) and to itself.  q, gate ``[B,Hq,D]``; k, v ``[B,Hkv,D]``; caches
    ``[B,max_len,Hkv,D]``.  Returns ``(o [B,Hq,D], k_new [B,Hkv,D])`` where
    k_new is the token's normalised, rotated key (what the cache stores at
    position n[b])."""
    q, k, v, gate = _f64(q), _f64(k), _f64(v), _f64(gate)
    kc, vc = _f64(k_cache), _f64(v_cache)
    B, Hq, D = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    n = np.asarray(n)
    out = np.zeros((B, Hq, D))
    knew = np.zeros((B, Hkv, D))
    for b in range(B):
        pos = np.float64(n[b])
        qr, kr = _prep(q[b], k[b], q_norm_w, k_norm_w, eps, rope_dim, theta, pos, pos)
        knew[b] = kr
        for h in range(Hq):
            g = h // G
            keys = np.concatenate([kc[b, :n[b], g], kr[g][None]], axis=0)
            vals = np.concatenate([vc[b, :n[b], g], v[b, g][None]], axis=0)
            s = keys @ qr[h] / np.sqrt(D)
            p = np.exp(s - s.max())
            p /= p.sum()
            out[b, h] = (p @ vals) / (1.0 + np.exp(-gate[b, h]))
    return out, knew


def prefill_cache(k, v, k_norm_w=None, eps=1e-6, rope_dim=ROPE_DIM, theta=THETA):
    """What a prefill of k, v ``[B,T,Hkv,D]`` leaves in the cache: the
    normalised, rotated keys and the values unchanged."""
    k = _f64(k)
    T = k.shape[1]
    pos = np.arange(T, dtype=np.float64)
    kr = rope(qk_norm(k, k_norm_w, eps), pos[:, None], rope_dim, theta)
    return kr, _f64(v)
