"""Pins for the float64 oracle, independent of the oracle's own code.

The pages print no numeric worked example of the recurrence, so the oracle is
pinned by what the mathematics and the pages fix:

===========================  ==================================================
pin                          what it fixes
===========================  ==================================================
identity (beta=0, alpha=1)   nothing written, nothing decayed: S_t = S_0 and
                             o_t = S_0 q_t exactly
pure decay (beta=0)          S_t = (prod alpha) S_0: closed form
orthonormal retrieval        alpha=beta=1, orthonormal keys, S_0=0: the state
                             is sum v_i k_i^T and querying q_t = k_t returns
                             v_t (a textbook projection identity)
rewrite same key             delete-before-write ("Gated DeltaNet Mechanics"):
                             writing v1 then v2 under the same key leaves v2
single token                 T=1 closed form in the delta form
                             o = alpha S q + d (k.q), d = beta (v - alpha S k)
product form (brute force)   S_T = S_0 prod P_t + sum beta_t v_t k_t^T
                             prod_{s>t} P_s with P_t = alpha_t (I - beta_t k k^T)
                             as explicit d x d matrices, tiny d and T
head map                     value head h reads query/key head h // (Hv/Hqk)
contraction bound            ||S_t|| <= alpha_t ||S_{t-1}|| + beta_t ||v_t||
                             for unit keys and beta in [0, 1]
empty sequence               T = 0 passes the state through
backward: finite differences every gradient of the backward oracle equals the
                             central difference of the forward oracle
backward: autograd           reverse-mode AD (torch, float64) of a plain loop
backward: identity           beta=0, alpha=1 closed forms of all six gradients
backward: chunked            the chunked backward derivation agrees (1e-12)
===========================  ==================================================

``test_mutants_are_caught`` runs every pin against deliberately broken copies
of the recurrence (a dropped beta, a transposed outer product, the output read
before the update, a wrong sign, decay on the wrong term, the wrong head map,
the key used as the query, ...) and requires each mutant to fail at least one
pin.  All of this runs on the CPU.
"""
import json
import os

import numpy as np
import pytest
import scipy.special
import scipy.stats

import oracle
from oracle import chunked_form

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------- helpers
def rng(seed):
    return np.random.default_rng(seed)


def unit(x):
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def rand_inputs(r, B, T, Hqk, Hv, D, h0=True, normalize=True):
    q = r.standard_normal((B, T, Hqk, D))
    k = r.standard_normal((B, T, Hqk, D))
    if normalize:
        q, k = unit(q), unit(k)
    v = r.standard_normal((B, T, Hv, D))
    beta = scipy.special.expit(r.standard_normal((B, T, Hv)))
    alpha = np.exp(-0.05 * np.logaddexp(0.0, r.standard_normal((B, T, Hv))))
    s0 = 0.3 * r.standard_normal((B, Hv, D, D)) if h0 else None
    return q, k, v, alpha, beta, s0


def c_impl(q, k, v, alpha, beta, h0):
    return oracle.prefill(q, k, v, alpha, beta, h0)


def np_impl(q, k, v, alpha, beta, h0):
    return oracle.np_prefill(q, k, v, alpha, beta, h0)


def make_mutant(kind):
    """Deliberately broken recurrences used to show that the pins bite."""
    def impl(q, k, v, alpha, beta, h0):
        B, T, Hqk, D = q.shape
        Hv = v.shape[2]
        G = Hv // Hqk
        o = np.zeros((B, T, Hv, D))
        ht = np.zeros((B, Hv, D, D))
        for b in range(B):
            for h in range(Hv):
                g = (h % Hqk) if kind == "head_map_mod" else h // G
                S = np.zeros((D, D)) if h0 is None else h0[b, h].copy()
                for t in range(T):
                    kt, qt, vt = k[b, t, g], q[b, t, g], v[b, t, h]
                    a, be = alpha[b, t, h], beta[b, t, h]
                    Sp = S
                    if kind == "no_beta_erase":
                        S = a * (S - np.outer(S @ kt, kt)) + be * np.outer(vt, kt)
                    elif kind == "transposed_write":
                        S = a * (S - be * np.outer(S @ kt, kt)) + be * np.outer(kt, vt)
                    elif kind == "alpha_on_write":
                        S = a * ((S - be * np.outer(S @ kt, kt)) + be * np.outer(vt, kt))
                    elif kind == "erase_sign":
                        S = a * (S + be * np.outer(S @ kt, kt)) + be * np.outer(vt, kt)
                    elif kind == "no_decay_on_erase":
                        S = a * S - be * np.outer(S @ kt, kt) + be * np.outer(vt, kt)
                    elif kind == "erase_transposed":
                        S = a * (S - be * np.outer(kt, kt @ S)) + be * np.outer(vt, kt)
                    elif kind == "no_beta_write":
                        S = a * (S - be * np.outer(S @ kt, kt)) + np.outer(vt, kt)
                    else:
                        S = a * (S - be * np.outer(S @ kt, kt)) + be * np.outer(vt, kt)
                    if kind == "pre_update_output":
                        o[b, t, h] = Sp @ qt
                    elif kind == "key_as_query":
                        o[b, t, h] = S @ kt
                    else:
                        o[b, t, h] = S @ qt
                ht[b, h] = S
        return o, ht
    return impl


MUTANTS = ["no_beta_erase", "transposed_write", "alpha_on_write", "erase_sign",
           "no_decay_on_erase", "erase_transposed", "no_beta_write",
           "pre_update_output", "key_as_query", "head_map_mod"]


# ---------------------------------------------------------------- the pins
def pin_identity(impl):
    r = rng(1)
    q, k, v, alpha, beta, s0 = rand_inputs(r, 2, 9, 2, 6, 8)
    beta[:] = 0.0
    alpha[:] = 1.0
    o, ht = impl(q, k, v, alpha, beta, s0)
    np.testing.assert_array_equal(ht, s0)
    G = 3
    for h in range(6):
        ref = np.einsum("bij,btj->bti", s0[:, h], q[:, :, h // G])
        np.testing.assert_allclose(o[:, :, h], ref, rtol=0, atol=1e-13)


def pin_pure_decay(impl):
    r = rng(2)
    q, k, v, alpha, beta, s0 = rand_inputs(r, 1, 12, 1, 2, 6)
    beta[:] = 0.0
    o, ht = impl(q, k, v, alpha, beta, s0)
    gam = np.cumprod(alpha, axis=1)                     # [B,T,Hv]
    for h in range(2):
        np.testing.assert_allclose(ht[0, h], gam[0, -1, h] * s0[0, h], rtol=1e-13, atol=1e-15)
        for t in range(12):
            np.testing.assert_allclose(o[0, t, h], gam[0, t, h] * (s0[0, h] @ q[0, t, 0]),
                                       rtol=1e-12, atol=1e-14)


def pin_orthonormal_retrieval(impl):
    r = rng(3)
    D, T = 16, 16
    Qm, _ = np.linalg.qr(r.standard_normal((D, D)))
    keys = Qm.T                                  # rows orthonormal
    k = keys[None, :T, None, :].copy()
    q = k.copy()                                 # query each token with its own key
    v = r.standard_normal((1, T, 1, D))
    alpha = np.ones((1, T, 1))
    beta = np.ones((1, T, 1))
    o, ht = impl(q, k, v, alpha, beta, None)
    np.testing.assert_allclose(o[0, :, 0], v[0, :, 0], rtol=0, atol=1e-12)
    np.testing.assert_allclose(ht[0, 0], v[0, :, 0].T @ keys[:T], rtol=0, atol=1e-12)


def pin_rewrite_same_key(impl):
    r = rng(4)
    D = 8
    kk = unit(r.standard_normal(D))
    other = unit(r.standard_normal(D))
    v1, v2, v3 = r.standard_normal((3, D))
    k = np.stack([kk, other, kk])[None, :, None, :]
    q = np.stack([kk, kk, kk])[None, :, None, :]
    v = np.stack([v1, v3, v2])[None, :, None, :]
    alpha = np.ones((1, 3, 1))
    beta = np.ones((1, 3, 1))
    o, ht = impl(q, k, v, alpha, beta, None)
    # after the last write the memory returns exactly v2 for the key kk, whatever
    # was written under another key in between:
    np.testing.assert_allclose(ht[0, 0] @ kk, v2, rtol=0, atol=1e-12)
    # and the first read returns v1 (the only association so far)
    np.testing.assert_allclose(o[0, 0, 0], v1, rtol=0, atol=1e-12)


def pin_single_token(impl):
    r = rng(5)
    q, k, v, alpha, beta, s0 = rand_inputs(r, 3, 1, 1, 2, 7)
    o, ht = impl(q, k, v, alpha, beta, s0)
    for b in range(3):
        for h in range(2):
            S, qq, kk, vv = s0[b, h], q[b, 0, 0], k[b, 0, 0], v[b, 0, h]
            a, be = alpha[b, 0, h], beta[b, 0, h]
            d = be * (vv - a * (S @ kk))
            np.testing.assert_allclose(o[b, 0, h], a * (S @ qq) + d * (kk @ qq),
                                       rtol=1e-12, atol=1e-13)
            np.testing.assert_allclose(ht[b, h], a * S + np.outer(d, kk),
                                       rtol=1e-12, atol=1e-13)


def product_form(q, k, v, alpha, beta, s0):
    """Brute-force closed form with explicit d x d matrices (one head)."""
    T, D = k.shape
    P = [alpha[t] * (np.eye(D) - beta[t] * np.outer(k[t], k[t])) for t in range(T)]
    o = np.zeros((T, D))
    S = None
    for t_end in range(1, T + 1):
        S = s0.copy()
        for t in range(t_end):
            S = S @ P[t]
        for t in range(t_end):
            term = beta[t] * np.outer(v[t], k[t])
            for s in range(t + 1, t_end):
                term = term @ P[s]
            S = S + term
        o[t_end - 1] = S @ q[t_end - 1]
    return o, S


def pin_product_form(impl):
    r = rng(6)
    for D, T in [(3, 5), (4, 6), (2, 4)]:
        q, k, v, alpha, beta, s0 = rand_inputs(r, 1, T, 1, 1, D, normalize=False)
        o, ht = impl(q, k, v, alpha, beta, s0)
        ob, Sb = product_form(q[0, :, 0], k[0, :, 0], v[0, :, 0], alpha[0, :, 0],
                              beta[0, :, 0], s0[0, 0])
        np.testing.assert_allclose(o[0, :, 0], ob, rtol=1e-11, atol=1e-12)
        np.testing.assert_allclose(ht[0, 0], Sb, rtol=1e-11, atol=1e-12)


def pin_head_map(impl):
    r = rng(7)
    Hqk, Hv, D, T = 2, 6, 6, 5
    q, k, v, alpha, beta, s0 = rand_inputs(r, 1, T, Hqk, Hv, D)
    o, ht = impl(q, k, v, alpha, beta, s0)
    for h in range(Hv):
        g = h // (Hv // Hqk)
        o1, ht1 = oracle.np_prefill(q[:, :, g:g + 1], k[:, :, g:g + 1], v[:, :, h:h + 1],
                                    alpha[:, :, h:h + 1], beta[:, :, h:h + 1],
                                    s0[:, h:h + 1])
        np.testing.assert_allclose(o[:, :, h], o1[:, :, 0], rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(ht[:, h], ht1[:, 0], rtol=1e-12, atol=1e-13)


def pin_contraction(impl):
    r = rng(8)
    D, T = 8, 10
    q, k, v, alpha, beta, s0 = rand_inputs(r, 1, T, 1, 1, D)
    S_prev = s0[0, 0]
    for t in range(T):
        _, ht = impl(q[:, t:t + 1], k[:, t:t + 1], v[:, t:t + 1], alpha[:, t:t + 1],
                     beta[:, t:t + 1], S_prev[None, None])
        S = ht[0, 0]
        bound = alpha[0, t, 0] * np.linalg.norm(S_prev, 2) + beta[0, t, 0] * np.linalg.norm(v[0, t, 0])
        assert np.linalg.norm(S, 2) <= bound * (1 + 1e-12)
        S_prev = S


def pin_empty(impl):
    r = rng(9)
    q, k, v, alpha, beta, s0 = rand_inputs(r, 2, 0, 1, 3, 4)
    o, ht = impl(q, k, v, alpha, beta, s0)
    assert o.shape == (2, 0, 3, 4)
    np.testing.assert_array_equal(ht, s0)


PINS = [pin_identity, pin_pure_decay, pin_orthonormal_retrieval,
        pin_rewrite_same_key, pin_single_token, pin_product_form, pin_head_map,
        pin_contraction, pin_empty]


# ---------------------------------------------------------------- tests
@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
@pytest.mark.parametrize("impl", [c_impl, np_impl], ids=["c_oracle", "numpy_twin"])
def test_oracle_pin(oracle_mod, impl, pin):
    pin(impl)


@pytest.mark.parametrize("kind", MUTANTS)
def test_mutants_are_caught(kind):
    impl = make_mutant(kind)
    failed = []
    for pin in PINS:
        try:
            pin(impl)
        except AssertionError:
            failed.append(pin.__name__)
    assert failed, "mutant %s passed every pin" % kind


def test_unmutated_reference_passes_all_pins():
    impl = make_mutant("none")
    for pin in PINS:
        pin(impl)


def test_c_oracle_matches_numpy_twin(oracle_mod):
    r = rng(10)
    q, k, v, alpha, beta, s0 = rand_inputs(r, 2, 11, 2, 6, 16)
    o1, h1 = oracle.prefill(q, k, v, alpha, beta, s0)
    o2, h2 = oracle.np_prefill(q, k, v, alpha, beta, s0)
    np.testing.assert_allclose(o1, o2, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(h1, h2, rtol=1e-12, atol=1e-13)


def test_decode_steps_equal_prefill(oracle_mod):
    r = rng(11)
    B, T, Hqk, Hv, D = 3, 9, 2, 6, 16
    q, k, v, alpha, beta, s0 = rand_inputs(r, B, T, Hqk, Hv, D)
    o_ref, h_ref = oracle.prefill(q, k, v, alpha, beta, s0)
    st = s0
    for t in range(T):
        o_t, st = oracle.decode_step(q[:, t], k[:, t], v[:, t], alpha[:, t], beta[:, t], st)
        np.testing.assert_allclose(o_t, o_ref[:, t], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(st, h_ref, rtol=1e-12, atol=1e-13)


def test_varlen_equals_separate_sequences(oracle_mod):
    r = rng(12)
    lengths = [5, 0, 9, 1]
    Hqk, Hv, D = 2, 6, 8
    T = sum(lengths)
    q, k, v, alpha, beta, _ = rand_inputs(r, 1, T, Hqk, Hv, D)
    h0 = r.standard_normal((len(lengths), Hv, D, D))
    cu = np.concatenate([[0], np.cumsum(lengths)])
    o, ht = oracle.varlen(q[0], k[0], v[0], alpha[0], beta[0], cu, h0)
    for n, L in enumerate(lengths):
        s = cu[n]
        o_n, ht_n = oracle.np_prefill(q[:, s:s + L], k[:, s:s + L], v[:, s:s + L],
                                      alpha[:, s:s + L], beta[:, s:s + L], h0[n:n + 1])
        np.testing.assert_allclose(o[s:s + L], o_n[0], rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(ht[n], ht_n[0], rtol=1e-12, atol=1e-13)
    np.testing.assert_array_equal(ht[1], h0[1])      # empty sequence passes h0


def test_round_bf16_pins():
    """bfloat16 rounding, pinned against the hardware conversion (torch's
    float32 -> bfloat16 is round-to-nearest-even) on float32 values, and by
    hand on ties, binade edges, subnormals and overflow."""
    import torch
    r = rng(17)
    x32 = np.concatenate([r.standard_normal(20000) * 10.0 ** r.integers(-30, 30, 20000),
                          r.standard_normal(1000) * 1e-40]).astype(np.float32)
    ref = torch.from_numpy(x32).to(torch.bfloat16).double().numpy()
    np.testing.assert_array_equal(oracle.round_bf16(x32.astype(np.float64)), ref)
    one = 1.0
    ulp = 2.0 ** -7                                    # spacing in [1, 2)
    cases = {
        one + ulp / 2: one,                            # tie, 1.0 is even
        one + 3 * ulp / 2: one + 2 * ulp,              # tie, rounds up to even
        one + ulp / 2 + 2.0 ** -30: one + ulp,         # just above a tie
        2.0 - ulp / 4: 2.0,                            # carries into the next binade
        -(one + ulp / 2): -one,
        0.0: 0.0,
        2.0 ** -133: 2.0 ** -133,                      # smallest subnormal
        2.0 ** -134: 0.0,                              # tie with 0: even
        3 * 2.0 ** -135: 2.0 ** -133,                  # above the tie
        (2.0 - 2.0 ** -7) * 2.0 ** 127: (2.0 - 2.0 ** -7) * 2.0 ** 127,
        (2.0 - 2.0 ** -9) * 2.0 ** 127: np.inf,        # rounds past the largest value
    }
    got = oracle.round_bf16(np.array(list(cases.keys())))
    np.testing.assert_array_equal(got, np.array(list(cases.values())))
    assert np.isnan(oracle.round_bf16(np.array([np.nan]))[0])
    # idempotent, and the double rounding through float32 is not what it does
    x = r.standard_normal(1000)
    np.testing.assert_array_equal(oracle.round_bf16(oracle.round_bf16(x)), oracle.round_bf16(x))
    t = 1.0 + 2.0 ** -8 + 2.0 ** -40            # just above a bf16 tie, below float32 resolution
    assert oracle.round_bf16(np.array([t]))[0] == 1.0 + 2.0 ** -7
    assert torch.tensor([t], dtype=torch.float64).float().to(torch.bfloat16).item() == 1.0


def test_bf16_state_variants(oracle_mod):
    """The bf16-state oracle is the float64 step followed by one rounding."""
    import torch
    r = rng(19)
    B, Hqk, Hv, D = 2, 2, 6, 16
    st = torch.from_numpy(r.standard_normal((B, Hv, D, D)) * 0.1).to(torch.bfloat16)
    q = unit(r.standard_normal((B, Hqk, D))); k = unit(r.standard_normal((B, Hqk, D))); v = r.standard_normal((B, Hv, D))
    a = np.exp(-0.05 * r.random((B, Hv))); be = r.random((B, Hv))
    o, s1 = oracle.decode_step_bf16_state(q, k, v, a, be, st)
    o_ref, s_ref = oracle.decode_step(q, k, v, a, be, st.double().numpy())
    np.testing.assert_array_equal(o, o_ref)
    np.testing.assert_array_equal(s1, oracle.round_bf16(s_ref))
    assert np.array_equal(torch.from_numpy(s1).to(torch.bfloat16).double().numpy(), s1)
    T = 5
    qs = unit(r.standard_normal((1, T, Hqk, D))); ks = unit(r.standard_normal((1, T, Hqk, D))); vs = r.standard_normal((1, T, Hv, D))
    al = np.exp(-0.05 * r.random((1, T, Hv))); bs = r.random((1, T, Hv))
    op, hp = oracle.prefill_bf16_state(qs, ks, vs, al, bs, st[:1])
    op_ref, hp_ref = oracle.prefill(qs, ks, vs, al, bs, st[:1].double().numpy())
    np.testing.assert_array_equal(op, op_ref)
    np.testing.assert_array_equal(hp, oracle.round_bf16(hp_ref))


def test_verify_commit_pins(oracle_mod):
    """Speculative decoding glue: verify of n tokens equals n sequential
    decode steps on a copy; commit of m tokens equals m decode steps; the
    state is advanced only by commit; per-sequence acceptance counts."""
    r = rng(23)
    B, n, Hqk, Hv, D = 3, 3, 2, 4, 16
    q = unit(r.standard_normal((B, n, Hqk, D))); k = unit(r.standard_normal((B, n, Hqk, D)))
    v = r.standard_normal((B, n, Hv, D))
    a = np.exp(-0.05 * r.random((B, n, Hv))); be = r.random((B, n, Hv))
    st = r.standard_normal((B, Hv, D, D)) * 0.1
    st0 = st.copy()
    o = oracle.decode_verify(q, k, v, a, be, st)
    np.testing.assert_array_equal(st, st0)
    ref = st.copy()
    for t in range(n):
        ot, ref = oracle.decode_step(q[:, t], k[:, t], v[:, t], a[:, t], be[:, t], ref)
        np.testing.assert_allclose(o[:, t], ot, rtol=1e-12, atol=1e-14)
        s_t = oracle.decode_commit(k, v, a, be, st, [t + 1] * B)
        np.testing.assert_allclose(s_t, ref, rtol=1e-12, atol=1e-14)
    m = [0, 2, 5]                                     # 5 is clipped to n
    s_m = oracle.decode_commit(k, v, a, be, st, m)
    np.testing.assert_array_equal(s_m[0], st[0])
    _, s2 = oracle.decode_step(q[1:2, 0], k[1:2, 0], v[1:2, 0], a[1:2, 0], be[1:2, 0], st[1:2])
    _, s2 = oracle.decode_step(q[1:2, 1], k[1:2, 1], v[1:2, 1], a[1:2, 1], be[1:2, 1], s2)
    np.testing.assert_allclose(s_m[1], s2[0], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(s_m[2], ref[2], rtol=1e-12, atol=1e-14)


def test_gate_rmsnorm_pins():
    r = rng(13)
    D = 128
    # constant rows: rms(c*1) = |c|, so y = sign(c) * w * sigmoid(g) when eps = 0
    c = np.array([2.5, -0.75, 1e-3])[:, None] * np.ones((3, D))
    g = r.standard_normal((3, D))
    w = r.standard_normal(D)
    y = oracle.gate_rmsnorm(c, g, w, eps=0.0)
    np.testing.assert_allclose(y, np.sign(c) * w * scipy.special.expit(g), rtol=1e-13)
    # scale invariance with eps = 0; the norm equals the library 2-norm / sqrt(D)
    o = r.standard_normal((5, 3, D))
    gate = r.standard_normal((5, 3, D))
    y1 = oracle.gate_rmsnorm(o, gate, None, 0.0)
    y2 = oracle.gate_rmsnorm(7.0 * o, gate, None, 0.0)
    np.testing.assert_allclose(y1, y2, rtol=1e-13)
    ref = o / (np.linalg.norm(o, axis=-1, keepdims=True) / np.sqrt(D)) * scipy.special.expit(gate)
    np.testing.assert_allclose(y1, ref, rtol=1e-12)
    # gate 0 halves, eps enters under the root
    y0 = oracle.gate_rmsnorm(o, np.zeros_like(o), None, 0.5)
    np.testing.assert_allclose(y0, 0.5 * o / np.sqrt(np.mean(o * o, -1, keepdims=True) + 0.5),
                               rtol=1e-13)


@pytest.mark.parametrize("C", [1, 16, 64])
def test_chunked_form_equals_sequential(oracle_mod, C):
    """The block-parallel rewrite reaches the sequential result (to float64
    rounding), including a partial last chunk and a non-zero initial state."""
    r = rng(20 + C)
    B, T, Hqk, Hv, D = 1, 150, 2, 6, 32
    q, k, v, alpha, beta, s0 = rand_inputs(r, B, T, Hqk, Hv, D)
    o_ref, h_ref = oracle.prefill(q, k, v, alpha, beta, s0)
    o_c, h_c = chunked_form.chunked_prefill(q, k, v, alpha, beta, s0, C=C)
    scale_o = np.abs(o_ref).max()
    np.testing.assert_allclose(o_c, o_ref, rtol=0, atol=1e-12 * scale_o)
    np.testing.assert_allclose(h_c, h_ref, rtol=0, atol=1e-12 * np.abs(h_ref).max())


def test_chunked_form_full_head_dim(oracle_mod):
    r = rng(30)
    q, k, v, alpha, beta, s0 = rand_inputs(r, 1, 130, 1, 3, 128)
    o_ref, h_ref = oracle.prefill(q, k, v, alpha, beta, s0)
    o_c, h_c = chunked_form.chunked_prefill(q, k, v, alpha, beta, s0, C=64)
    np.testing.assert_allclose(o_c, o_ref, rtol=0, atol=1e-11 * np.abs(o_ref).max())
    np.testing.assert_allclose(h_c, h_ref, rtol=0, atol=1e-11 * np.abs(h_ref).max())


def test_nan_isolation(oracle_mod):
    r = rng(31)
    q, k, v, alpha, beta, s0 = rand_inputs(r, 2, 6, 2, 6, 8)
    v[1, 2, 4, 3] = np.nan
    o, ht = oracle.prefill(q, k, v, alpha, beta, s0)
    bad = np.zeros(o.shape, dtype=bool)
    bad[1, 2:, 4] = True
    assert np.isnan(o[1, 2, 4]).any()
    assert np.isfinite(o[~bad]).all()
    assert np.isfinite(np.delete(ht.reshape(12, -1), 1 * 6 + 4, axis=0)).all()


def test_state_size_independent_of_T(oracle_mod):
    r = rng(32)
    shapes = set()
    for T in (1, 64, 256):
        q, k, v, alpha, beta, _ = rand_inputs(r, 1, T, 1, 3, 16)
        _, ht = oracle.prefill(q, k, v, alpha, beta, None)
        shapes.add(ht.shape)
    assert shapes == {(1, 3, 16, 16)}


def test_footprint_tens_of_megabytes():
    """48 layers x 48 value heads x 128 x 128 at 2 bytes (BF16, the precision
    the page computes in) is 72 MiB: 'tens of megabytes'."""
    with open(os.path.join(GOLDEN, "pages_facts.json")) as f:
        facts = json.load(f)
    layers = facts["deltanet_layers"]["value"]
    heads = facts["value_heads"]["value"]
    d = facts["head_dim"]["value"]
    lo, hi = facts["state_overhead_bytes_range"]["value"]
    total = layers * heads * d * d * 2
    assert total == 75_497_472 == 72 * 2 ** 20
    assert lo <= total < hi
    assert facts["value_heads"]["value"] % facts["qk_heads"]["value"] == 0
    # a per-token KV cache of the same size would grow with context; the state does not
    assert facts["total_layers"]["value"] - layers == 16


def test_synth_inputs_deterministic_and_normalised():
    import torch
    import synth
    a = synth.prefill_inputs(1, 70, torch.bfloat16, seed=5)
    b = synth.prefill_inputs(1, 70, torch.bfloat16, seed=5)
    for key in ("q", "k", "v", "alpha", "beta"):
        assert torch.equal(a[key], b[key])
    n = a["k"].double().norm(dim=-1)
    assert torch.allclose(n, torch.ones_like(n), atol=1e-2)
    assert (a["alpha"] > 0).all() and (a["alpha"] <= 1).all()
    assert (a["beta"] >= 0).all() and (a["beta"] <= 1).all()
    # the distributions match their definitions (sanity, not exactness)
    x = -np.log(a["alpha"].double().numpy()) / 0.05       # softplus of N(0,1)
    z = np.log(np.expm1(x))                                 # back to N(0,1)
    assert scipy.stats.kstest(z.ravel(), "norm").pvalue > 1e-4


def test_synth_strong_decay_reaches_the_ends():
    import torch
    import synth
    inp = synth.prefill_inputs(2, 200, torch.float32, seed=501, strong_decay=True)
    base = synth.prefill_inputs(2, 200, torch.float32, seed=501)
    a, b = inp["alpha"], inp["beta"]
    assert a.min() < 0.05 and a.max() > 0.9 and (a > 0).all() and (a < 1).all()
    assert (b == 0).any() and (b == 1).any()
    frac0, frac1 = (b == 0).double().mean().item(), (b == 1).double().mean().item()
    assert 0.08 < frac0 < 0.17 and 0.08 < frac1 < 0.17
    # q, k, v are the plain recipe's draws; only alpha and beta change
    for key in ("q", "k", "v"):
        assert torch.equal(inp[key], base[key])


# ------------------------------------------------------------- backward pins
# The oracle's backward (oracle.prefill_backward) is the chain rule applied by
# hand to the sequential recurrence.  It is pinned by (1) central finite
# differences of the forward oracle on every input element, (2) reverse-mode
# automatic differentiation (torch, float64) of a plain forward loop, (3) the
# closed form of the identity case beta=0, alpha=1, and (4) the chunked
# backward derivation reaching the same gradients.

def _bwd_inputs(seed, B, T, Hqk, Hv, D):
    r = rng(seed)
    q, k, v, alpha, beta, s0 = rand_inputs(r, B, T, Hqk, Hv, D)
    do = r.standard_normal((B, T, Hv, D))
    dht = r.standard_normal((B, Hv, D, D))
    return q, k, v, alpha, beta, s0, do, dht


def test_backward_finite_differences(oracle_mod):
    q, k, v, a, b, s0, do, dht = _bwd_inputs(41, 2, 5, 2, 6, 4)
    grads = oracle.prefill_backward(q, k, v, a, b, do, s0, dht)
    ins = [q, k, v, a, b, s0]

    def loss(args):
        o, ht = oracle.prefill(*args)
        return float(np.sum(o * do) + np.sum(ht * dht))

    eps = 1e-6
    for n, (x, gx) in enumerate(zip(ins, [grads[0], grads[1], grads[2],
                                          grads[3], grads[4], grads[5]])):
        fd = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp = [y.copy() for y in ins]
            xm = [y.copy() for y in ins]
            xp[n][idx] += eps
            xm[n][idx] -= eps
            fd[idx] = (loss(xp) - loss(xm)) / (2 * eps)
        err = np.abs(fd - gx).max() / np.abs(fd).max()
        assert err < 1e-7, (n, err)


def test_backward_matches_autograd(oracle_mod):
    torch = pytest.importorskip("torch")
    q, k, v, a, b, s0, do, dht = _bwd_inputs(42, 1, 70, 2, 6, 8)
    t = [torch.tensor(x, dtype=torch.float64, requires_grad=True)
         for x in (q, k, v, a, b, s0)]
    tq, tk, tv, ta, tb, ts = t
    B, T, Hqk, D = q.shape
    Hv = v.shape[2]
    loss = 0.0
    for h in range(Hv):
        g = h // (Hv // Hqk)
        S = ts[0, h]
        for i in range(T):
            kt = tk[0, i, g]
            S = ta[0, i, h] * (S - tb[0, i, h] * torch.outer(S @ kt, kt)) \
                + tb[0, i, h] * torch.outer(tv[0, i, h], kt)
            loss = loss + torch.dot(S @ tq[0, i, g], torch.tensor(do[0, i, h]))
        loss = loss + torch.sum(S * torch.tensor(dht[0, h]))
    loss.backward()
    mine = oracle.prefill_backward(q, k, v, a, b, do, s0, dht)
    for x, gx in zip(t, mine):
        ref = x.grad.numpy()
        assert np.abs(ref - gx).max() <= 1e-11 * max(1.0, np.abs(ref).max())


def test_backward_identity_closed_form(oracle_mod):
    # beta = 0, alpha = 1: S_t = S_0 for every t, so with
    # G_t = dht + sum_{s >= t} do_s q_s^T:
    #   dq_t = sum_h S_0^T do_t,  dk = dv = 0,  dh0 = G_1,
    #   dalpha_t = <G_t, S_0>,  dbeta_t = (G_t k_t) . (v_t - S_0 k_t)
    q, k, v, a, b, s0, do, dht = _bwd_inputs(43, 1, 7, 2, 6, 5)
    a = np.ones_like(a)
    b = np.zeros_like(b)
    dq, dk, dv, da, db, dh0 = oracle.prefill_backward(q, k, v, a, b, do, s0, dht)
    assert np.all(dk == 0) and np.all(dv == 0)
    T, Hv = q.shape[1], v.shape[2]
    for h in range(Hv):
        g = h // 3
        Gm = dht[0, h].copy()
        for t in range(T - 1, -1, -1):
            Gm += np.outer(do[0, t, h], q[0, t, g])
            assert np.isclose(da[0, t, h], np.sum(Gm * s0[0, h]), rtol=1e-12)
            ref_b = (Gm @ k[0, t, g]) @ (v[0, t, h] - s0[0, h] @ k[0, t, g])
            assert np.isclose(db[0, t, h], ref_b, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(dh0[0, h], Gm, rtol=1e-12, atol=1e-12)
    for t in range(T):
        for g in range(2):
            ref = sum(s0[0, h].T @ do[0, t, h] for h in range(3 * g, 3 * g + 3))
            np.testing.assert_allclose(dq[0, t, g], ref, rtol=1e-12, atol=1e-12)


def test_backward_empty_sequence(oracle_mod):
    q, k, v, a, b, s0, do, dht = _bwd_inputs(44, 1, 0, 2, 6, 4)
    dq, dk, dv, da, db, dh0 = oracle.prefill_backward(q, k, v, a, b, do, s0, dht)
    assert dq.shape == (1, 0, 2, 4) and da.shape == (1, 0, 6)
    np.testing.assert_array_equal(dh0, dht)


@pytest.mark.parametrize("C", [1, 16, 64])
def test_chunked_backward_equals_sequential(oracle_mod, C):
    q, k, v, a, b, s0, do, dht = _bwd_inputs(45, 1, 150, 2, 6, 16)
    seq = oracle.prefill_backward(q, k, v, a, b, do, s0, dht)
    chk = chunked_form.chunked_backward(q, k, v, a, b, do, s0, dht, C=C)
    for x, y in zip(seq, chk):
        assert np.linalg.norm(x - y) <= 1e-12 * np.linalg.norm(x)


# ------------------------------------------------------------- head sampling
# oracle.subset_heads gathers single value heads (with the query/key head each
# one reads) so that very long sequences can be checked a few heads at a time.
# Pinned against the full multi-head oracle: the sampled heads' outputs and
# final states must be the very same numbers, bit for bit (each head's chain
# is computed independently, in the same order, either way).

def _subset_case(seed, Hqk, Hv, T=9, D=8):
    r = rng(seed)
    return rand_inputs(r, 2, T, Hqk, Hv, D)


@pytest.mark.parametrize("with_h0", [True, False])
def test_subset_heads_equals_full_prefill(oracle_mod, with_h0):
    Hqk, Hv = 4, 12
    q, k, v, alpha, beta, s0 = _subset_case(41, Hqk, Hv)
    if not with_h0:
        s0 = None
    o, ht = oracle.prefill(q, k, v, alpha, beta, s0)
    heads = [11, 0, 5, 6, 7, 3]                 # unordered, several per group
    o_s, ht_s = oracle.prefill(*oracle.subset_heads(q, k, v, alpha, beta, s0, heads, Hqk, Hv))
    assert o_s.shape == (2, 9, len(heads), 8) and ht_s.shape == (2, len(heads), 8, 8)
    assert np.array_equal(o_s, o[:, :, heads])
    assert np.array_equal(ht_s, ht[:, heads])


def test_subset_heads_torch_inputs(oracle_mod):
    """The torch path (gather before widening) gives the numpy path's arrays."""
    import torch
    Hqk, Hv = 2, 6
    q, k, v, alpha, beta, s0 = _subset_case(42, Hqk, Hv)
    bf = lambda x: torch.from_numpy(x).to(torch.bfloat16)
    f32 = lambda x: torch.from_numpy(x).float()
    tq, tk, tv = bf(q), bf(k), bf(v)
    ta, tb, th = f32(alpha), f32(beta), f32(s0)
    heads = [5, 1, 2]
    got = oracle.subset_heads(tq, tk, tv, ta, tb, th, heads, Hqk, Hv)
    want = oracle.subset_heads(tq.double().numpy(), tk.double().numpy(), tv.double().numpy(),
                               ta.double().numpy(), tb.double().numpy(), th.double().numpy(),
                               heads, Hqk, Hv)
    for a, b in zip(got, want):
        assert a.dtype == np.float64 and np.array_equal(a, b)
    # query/key head of value head h is h // (Hv / Hqk): 5 -> 1, 1 -> 0, 2 -> 0
    assert np.array_equal(got[0][:, :, 0], tq[:, :, 1].double().numpy())
    assert np.array_equal(got[0][:, :, 1], tq[:, :, 0].double().numpy())


def test_subset_heads_wrong_group_map_is_caught(oracle_mod):
    """A gather that takes the query/key head as h % Hqk (a plausible slip)
    fails the equality above."""
    Hqk, Hv = 4, 12
    q, k, v, alpha, beta, s0 = _subset_case(43, Hqk, Hv)
    o, _ = oracle.prefill(q, k, v, alpha, beta, s0)
    heads = np.array([1, 8])                    # groups 0 and 2; h % Hqk gives 1 and 0
    bad = (q[:, :, heads % Hqk], k[:, :, heads % Hqk], v[:, :, heads],
           alpha[:, :, heads], beta[:, :, heads], s0[:, heads])
    o_b, _ = oracle.prefill(*bad)
    assert not np.array_equal(o_b, o[:, :, heads])
