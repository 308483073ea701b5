"""Pins for the gated-attention oracle (oracle/attention.py), independent of
its own code.

===========================  ==================================================
pin                          what it fixes
===========================  ==================================================
library attention            causal softmax attention with scale 1/sqrt(256)
                             and the 24/4 head map equals torch's float64
                             scaled_dot_product_attention (keys/values
                             repeated per group), then times sigmoid(gate)
library RMSNorm              qk_norm equals torch.nn.functional.rms_norm
RoPE closed form             a unit vector on channel j < 32 at position p
                             becomes cos(p w_j) e_j + sin(p w_j) e_{j+32},
                             w_j = theta^(-2j/64); channels >= 64 untouched
RoPE invariants              norm preserved; position 0 is the identity; the
                             score of (q at i, k at j) depends only on i - j
single token                 o = v * sigmoid(gate) for every query head
identical keys               uniform weights: o_t = mean(v_0..v_t) * sigmoid(g)
decode == prefill            token-by-token decode over the prefill's cache
                             reproduces the prefill's outputs
===========================  ==================================================
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import attention as A


def rnd(seed, *shape):
    return np.random.default_rng(seed).standard_normal(shape)


def inputs(seed, B=1, T=37):
    r = np.random.default_rng(seed)
    q = r.standard_normal((B, T, 24, 256))
    k = r.standard_normal((B, T, 4, 256))
    v = r.standard_normal((B, T, 4, 256))
    g = r.standard_normal((B, T, 24, 256))
    return q, k, v, g


def test_attention_matches_library_sdpa():
    q, k, v, g = inputs(1, B=2, T=45)
    qw, kw = 1 + 0.1 * rnd(2, 256), 1 + 0.1 * rnd(3, 256)
    o = A.attention(q, k, v, g, qw, kw)
    T = q.shape[1]
    pos = np.arange(T)[:, None]
    qr = A.rope(A.qk_norm(q, qw), pos)
    kr = A.rope(A.qk_norm(k, kw), pos)
    tq = torch.tensor(qr).permute(0, 2, 1, 3)
    tk = torch.tensor(kr).permute(0, 2, 1, 3).repeat_interleave(6, dim=1)
    tv = torch.tensor(v).permute(0, 2, 1, 3).repeat_interleave(6, dim=1)
    ref = F.scaled_dot_product_attention(tq, tk, tv, is_causal=True).permute(0, 2, 1, 3)
    ref = ref.numpy() * torch.sigmoid(torch.tensor(g)).numpy()
    assert np.abs(o - ref).max() < 1e-12


def test_qk_norm_matches_library_rms_norm():
    x = rnd(4, 3, 7, 256)
    w = rnd(5, 256)
    ref = F.rms_norm(torch.tensor(x), (256,), torch.tensor(w), eps=1e-6).numpy()
    assert np.abs(A.qk_norm(x, w, 1e-6) - ref).max() < 1e-12
    y = A.qk_norm(x)
    assert np.allclose(np.sqrt(np.mean(y * y, axis=-1)), 1.0, atol=1e-6)


@pytest.mark.parametrize("j", [0, 1, 17, 31])
@pytest.mark.parametrize("p", [1, 5, 1000, 262143])
def test_rope_closed_form(j, p):
    x = np.zeros(256)
    x[j] = 1.0
    y = A.rope(x, p)
    w = 1.0e7 ** (-2.0 * j / 64)
    ref = np.zeros(256)
    ref[j] = np.cos(p * w)
    ref[j + 32] = np.sin(p * w)
    assert np.abs(y - ref).max() < 1e-12
    x2 = np.zeros(256)
    x2[100] = 1.0                       # a pass-through channel
    assert np.array_equal(A.rope(x2, p), x2)


def test_rope_invariants():
    x = rnd(6, 10, 256)
    y = A.rope(x, np.arange(10) * 37.0)
    assert np.allclose(np.linalg.norm(y, axis=-1), np.linalg.norm(x, axis=-1), rtol=1e-12)
    assert np.array_equal(A.rope(x, 0.0), x)
    q, k = rnd(7, 256), rnd(8, 256)
    s1 = A.rope(q, 50) @ A.rope(k, 20)
    s2 = A.rope(q, 1050) @ A.rope(k, 1020)
    s3 = A.rope(q, 51) @ A.rope(k, 20)
    assert abs(s1 - s2) < 1e-9 and abs(s1 - s3) > 1e-6


def test_single_token_and_identical_keys():
    q, k, v, g = inputs(9, T=1)
    o = A.attention(q, k, v, g)
    for h in range(24):
        ref = v[0, 0, h // 6] / (1 + np.exp(-g[0, 0, h]))
        assert np.abs(o[0, 0, h] - ref).max() < 1e-12
    q, k, v, g = inputs(10, T=20)
    k[:] = k[:, :1]                      # same key at every position
    # RoPE makes the keys differ across positions unless rotation is off
    o = A.attention(q, k, v, g, rope_dim=0)
    for t in (0, 7, 19):
        for h in (0, 13):
            ref = v[0, :t + 1, h // 6].mean(axis=0) / (1 + np.exp(-g[0, t, h]))
            assert np.abs(o[0, t, h] - ref).max() < 1e-12


def test_decode_equals_prefill():
    q, k, v, g = inputs(11, B=2, T=12)
    o = A.attention(q, k, v, g)
    kc, vc = A.prefill_cache(k, v)
    n0 = 7
    cache_k = np.zeros((2, 16, 4, 256))
    cache_v = np.zeros((2, 16, 4, 256))
    cache_k[:, :n0], cache_v[:, :n0] = kc[:, :n0], vc[:, :n0]
    for t in range(n0, 12):
        od, knew = A.decode(q[:, t], k[:, t], v[:, t], g[:, t], cache_k, cache_v, [t, t])
        assert np.abs(od - o[:, t]).max() < 1e-12
        assert np.abs(knew - kc[:, t]).max() < 1e-12
        cache_k[:, t], cache_v[:, t] = knew, v[:, t]
