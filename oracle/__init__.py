"""Float64 CPU oracle for the Gated DeltaNet recurrence.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may import this package.  It shares no
code with the HIP library and never imports it; the product path never imports
this package.

Sources (pages as titled; their text is the authority on what is computed):

* "Inside Qwen3.8-27B: Hybrid DeltaNet Architecture, 256k Context, and 24GB
  Local Serving", section "Gated DeltaNet Mechanics": a d x d memory matrix per
  head, a normalized key, a delta rule that erases the key's current
  association before writing the new value, a per-token decay.  The update
  formula itself is missing from the extracted text; the recurrence used is
  the gated delta rule that fits every stated property::

      S_t = alpha_t S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T
      o_t = S_t q_t

* Same page, note under "The Role of Periodic Gated Attention": inference
  advances the state token by token; prefill uses a block-parallel rewrite of
  the same computation (that rewrite is checked separately in
  ``oracle/chunked_form.py``).
* "Qwen 3.8 27B Review: Native Vision, FP8 Quantization & 1M Context in a
  Compact Dense Model", section 3: 48 value heads, 16 query/key heads, head
  dim 128.  Value head h reads query/key head h // (Hv // Hqk).

Every function here is the plain definition: the token loop is sequential and
in float64.  Inputs are widened exactly (bf16 and fp32 values are exactly
representable in float64).

Functions
---------
prefill(q, k, v, alpha, beta, h0=None)       -> (o, ht)     C, OpenMP over (b, h)
decode_step(q, k, v, alpha, beta, state)     -> (o, state') C
prefill_backward(q, k, v, alpha, beta, do, h0, dht)
                                             -> (dq, dk, dv, dalpha, dbeta, dh0)  C
decode_step_bf16_state(...), prefill_bf16_state(...)   states stored in bf16
round_bf16(x)                                -> x rounded to bfloat16 (RNE)
decode_verify(q, k, v, alpha, beta, state)   -> o of n draft tokens, state unchanged
decode_commit(k, v, alpha, beta, state, m)   -> state advanced by m[b] accepted tokens
varlen(q, k, v, alpha, beta, cu_seqlens, ...)-> (y, ht)     C per sequence + epilogue
gate_rmsnorm(o, gate, weight, eps)           -> y           NumPy float64
np_prefill(q, k, v, alpha, beta, h0=None)    -> (o, ht)     NumPy twin (tiny sizes)
subset_heads(...)                                           gather for sampled checks

The gated attention layer of the same stack has its own float64 oracle in
``oracle/attention.py`` (QK-Norm, partial RoPE, causal GQA softmax attention,
sigmoid output gate), pinned in ``tests/test_attention_oracle.py``.

Parity status: every function is pinned by tests in tests/test_oracle_pins.py
(closed forms, invariants, brute force, textbook identities); see the module
docstring there for which pin covers which possible mistake.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gdn_oracle.c")
# GDN_ORACLE_LIB selects another build of gdn_oracle.c (e.g. with sanitizers).
_LIB_PATH = os.environ.get("GDN_ORACLE_LIB") or os.path.join(_HERE, "liboracle.so")
_lib = None
_lock = threading.Lock()


def build(force: bool = True) -> str:
    """Compile the C oracle with gcc (plain C, -O2, OpenMP; no intrinsics)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-ftree-vectorize", "-fopenmp", "-fPIC", "-shared",
               "-std=c99", "-o", tmp, _SRC]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(_LIB_PATH):
                build(force=False)
            lib = ctypes.CDLL(_LIB_PATH)
            dp = ctypes.POINTER(ctypes.c_double)
            i64 = ctypes.c_int64
            lib.oracle_gdn_prefill.argtypes = [dp, dp, dp, dp, dp, dp, dp, dp,
                                               i64, i64, i64, i64, i64]
            lib.oracle_gdn_prefill.restype = ctypes.c_int
            lib.oracle_gdn_decode_step.argtypes = [dp, dp, dp, dp, dp, dp, dp,
                                                   i64, i64, i64, i64]
            lib.oracle_gdn_decode_step.restype = ctypes.c_int
            lib.oracle_gdn_backward.argtypes = [dp] * 14 + [i64] * 5
            lib.oracle_gdn_backward.restype = ctypes.c_int
            lib.oracle_num_threads.argtypes = []
            lib.oracle_num_threads.restype = ctypes.c_int
            lib.oracle_set_num_threads.argtypes = [ctypes.c_int]
            lib.oracle_set_num_threads.restype = None
            _lib = lib
    return _lib


def num_threads() -> int:
    """Threads an OpenMP parallel region of the C oracle runs on here."""
    return int(_load().oracle_num_threads())


def set_num_threads(n: int) -> None:
    """Team size of the C oracle's later parallel regions."""
    _load().oracle_set_num_threads(int(n))


def _f64(x) -> np.ndarray:
    """Exact widening to a contiguous float64 array (accepts numpy arrays or
    anything with ``.float().numpy()`` such as a CPU torch tensor)."""
    if hasattr(x, "detach"):
        x = x.detach().cpu().float().numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(a: np.ndarray | None):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def prefill(q, k, v, alpha, beta, h0=None):
    """Sequential recurrence over ``[B, T]`` tokens for every value head.

    q, k ``[B,T,Hqk,D]``; v ``[B,T,Hv,D]``; alpha, beta ``[B,T,Hv]``;
    h0 ``[B,Hv,D,D]`` or None (zero state).  Returns float64 ``o [B,T,Hv,D]``
    and ``ht [B,Hv,D,D]``.
    """
    q, k, v, alpha, beta = (_f64(x) for x in (q, k, v, alpha, beta))
    B, T, Hqk, D = q.shape
    Hv = v.shape[2]
    assert k.shape == q.shape and v.shape == (B, T, Hv, D)
    assert alpha.shape == (B, T, Hv) and beta.shape == (B, T, Hv)
    h0a = None if h0 is None else _f64(h0)
    if h0a is not None:
        assert h0a.shape == (B, Hv, D, D)
    o = np.zeros((B, T, Hv, D), dtype=np.float64)
    ht = np.zeros((B, Hv, D, D), dtype=np.float64)
    rc = _load().oracle_gdn_prefill(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha),
                                    _ptr(beta), _ptr(h0a), _ptr(o), _ptr(ht),
                                    B, T, Hqk, Hv, D)
    if rc != 0:
        raise ValueError("oracle_gdn_prefill failed (%d)" % rc)
    return o, ht


def prefill_backward(q, k, v, alpha, beta, do, h0=None, dht=None):
    """Gradients of ``L = sum <do, o> + <dht, ht>`` with respect to every
    input of :func:`prefill` (the training pass of the same recurrence, page
    "Inside Qwen3.8-27B ...", note under "The Role of Periodic Gated
    Attention").  The chain rule is applied token by token in reverse, in
    float64; the derivation is written out in ``gdn_oracle.c``.

    do ``[B,T,Hv,D]``; dht ``[B,Hv,D,D]`` or None (zero).  Returns float64
    ``dq, dk [B,T,Hqk,D]`` (summed over the value heads of each group),
    ``dv [B,T,Hv,D]``, ``dalpha, dbeta [B,T,Hv]`` and ``dh0 [B,Hv,D,D]``.
    """
    q, k, v, alpha, beta, do = (_f64(x) for x in (q, k, v, alpha, beta, do))
    B, T, Hqk, D = q.shape
    Hv = v.shape[2]
    assert k.shape == q.shape and v.shape == (B, T, Hv, D) and do.shape == v.shape
    assert alpha.shape == (B, T, Hv) and beta.shape == (B, T, Hv)
    h0a = None if h0 is None else _f64(h0)
    dhta = None if dht is None else _f64(dht)
    for s in (h0a, dhta):
        if s is not None:
            assert s.shape == (B, Hv, D, D)
    dq = np.zeros((B, T, Hqk, D))
    dk = np.zeros((B, T, Hqk, D))
    dv = np.zeros((B, T, Hv, D))
    da = np.zeros((B, T, Hv))
    db = np.zeros((B, T, Hv))
    dh0 = np.zeros((B, Hv, D, D))
    rc = _load().oracle_gdn_backward(
        _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta), _ptr(h0a), _ptr(do),
        _ptr(dhta), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(da), _ptr(db), _ptr(dh0),
        B, T, Hqk, Hv, D)
    if rc != 0:
        raise ValueError("oracle_gdn_backward failed (%d)" % rc)
    return dq, dk, dv, da, db, dh0


def decode_step(q, k, v, alpha, beta, state, inplace=False):
    """One token per sequence.  q, k ``[B,Hqk,D]``; v ``[B,Hv,D]``;
    alpha, beta ``[B,Hv]``; state ``[B,Hv,D,D]``.  Returns ``(o, new_state)``.
    With ``inplace=True`` and a C-contiguous float64 ndarray state, that array
    is advanced in place and returned; otherwise the input is not modified."""
    q, k, v, alpha, beta = (_f64(x) for x in (q, k, v, alpha, beta))
    if (inplace and isinstance(state, np.ndarray) and state.dtype == np.float64
            and state.flags.c_contiguous):
        st = state
    else:
        st = _f64(state).copy()
    B, Hqk, D = q.shape
    Hv = v.shape[1]
    assert st.shape == (B, Hv, D, D)
    o = np.zeros((B, Hv, D), dtype=np.float64)
    rc = _load().oracle_gdn_decode_step(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha),
                                        _ptr(beta), _ptr(st), _ptr(o),
                                        B, Hqk, Hv, D)
    if rc != 0:
        raise ValueError("oracle_gdn_decode_step failed (%d)" % rc)
    return o, st


def decode_verify(q, k, v, alpha, beta, state):
    """Outputs for n draft tokens per sequence, starting from ``state``,
    without changing it (the verify pass of speculative decoding with drafted
    tokens, as the MTP heads on page "Inside Qwen3.8-27B ...", section
    "Multi-Token Prediction (MTP)", produce them).  q, k ``[B,n,Hqk,D]``;
    v ``[B,n,Hv,D]``; alpha, beta ``[B,n,Hv]``; state ``[B,Hv,D,D]``.
    Returns o ``[B,n,Hv,D]``: token t's output is S_t q_t with S_t the state
    after draft tokens 0..t, i.e. the prefill of the n tokens from state."""
    o, _ = prefill(q, k, v, alpha, beta, state)
    return o


def decode_commit(k, v, alpha, beta, state, n_accept):
    """Advance ``state`` by the first ``n_accept[b]`` draft tokens of each
    sequence b (the accepted prefix; values are clipped to [0, n]).  Returns
    the new state; the input is not modified."""
    k, v, alpha, beta = (_f64(x) for x in (k, v, alpha, beta))
    st = _f64(state).copy()
    B, n = k.shape[:2]
    acc = np.clip(np.asarray(n_accept, dtype=np.int64).reshape(B), 0, n)
    for b in range(B):
        m = int(acc[b])
        if m == 0:
            continue
        sl = slice(b, b + 1)
        zq = np.zeros_like(k[sl, :m])
        _, ht = prefill(zq, k[sl, :m], v[sl, :m], alpha[sl, :m], beta[sl, :m], st[sl])
        st[b] = ht[0]
    return st


# bfloat16: 1 sign bit, 8 exponent bits, 7 fraction bits (8 significant
# bits), the exponent range of float32.
_BF16_MAX = (2.0 - 2.0 ** -7) * 2.0 ** 127
_BF16_MIN_EXP = -133          # spacing of the subnormals: 2^-126 * 2^-7


def round_bf16(x) -> np.ndarray:
    """Round float64 values once to the nearest bfloat16 value, ties to even.

    Returns float64 values that are exactly representable in bfloat16.  For
    |x| in [2^(e-1), 2^e) the bfloat16 spacing is 2^(e-8) (8 significant
    bits), never finer than the subnormal spacing 2^-133; results beyond the
    largest finite value (2 - 2^-7) 2^127 become infinite with the sign of x.
    Infinities and NaNs pass through."""
    x = _f64(x)
    _, e = np.frexp(np.abs(x))
    q = np.ldexp(1.0, np.maximum(e - 8, _BF16_MIN_EXP))
    with np.errstate(invalid="ignore"):
        r = np.rint(x / q) * q
    r = np.where(np.abs(r) > _BF16_MAX, np.copysign(np.inf, x), r)
    return np.where(np.isfinite(x), r, x)


def decode_step_bf16_state(q, k, v, alpha, beta, state):
    """One decode step with the state stored in bfloat16 (the footprint the
    pages count in BF16): the stored state is widened exactly, advanced in
    float64 by ``decode_step``, and the new state is rounded once to
    bfloat16.  Returns ``(o, new_state)``, both float64; ``new_state`` holds
    bfloat16 values."""
    o, st = decode_step(q, k, v, alpha, beta, state)
    return o, round_bf16(st)


def prefill_bf16_state(q, k, v, alpha, beta, h0=None):
    """``prefill`` with the carried states stored in bfloat16: h0 (bfloat16
    values) is widened exactly and the final state is rounded once to
    bfloat16.  The recurrence inside the call runs in float64."""
    o, ht = prefill(q, k, v, alpha, beta, h0)
    return o, round_bf16(ht)


def gate_rmsnorm(o, gate, weight=None, eps=1e-6):
    """Output epilogue of the packed prefill: per (token, head) RMS
    normalisation over the head dimension, times an optional per-channel
    weight, times sigmoid(gate) elementwise.

    y = o / sqrt(mean(o^2) + eps) * w * 1/(1 + exp(-gate))

    RMSNorm as the architecture card ("Qwen3.8 (27B)", "Architecture concepts",
    QK-Norm entry) uses it; the learned sigmoid output gate as the same card's
    "Gated Attention" entry describes it.  Neither is spelled out for the
    DeltaNet layer on the pages: this is the plain reading applied to the
    recurrence's output.
    """
    o = _f64(o)
    g = _f64(gate)
    w = np.ones(o.shape[-1]) if weight is None else _f64(weight)
    rms = np.sqrt(np.mean(o * o, axis=-1, keepdims=True) + eps)
    return o / rms * w * (1.0 / (1.0 + np.exp(-g)))


def varlen(q, k, v, alpha, beta, cu_seqlens, h0=None, gate=None,
           norm_weight=None, eps=1e-6):
    """Packed sequences.  q, k ``[T_tot,Hqk,D]``; v ``[T_tot,Hv,D]``;
    alpha, beta ``[T_tot,Hv]``; cu_seqlens ``[N+1]`` (0 = first, last =
    T_tot); h0 ``[N,Hv,D,D]`` or None.  Each sequence is an independent
    recurrence starting from its own h0.  With ``gate`` given the output is the
    gated RMS-normalised ``y``; otherwise the plain ``o``.
    Returns ``(y_or_o [T_tot,Hv,D], ht [N,Hv,D,D])``.
    """
    q, k, v, alpha, beta = (_f64(x) for x in (q, k, v, alpha, beta))
    cu = np.asarray(cu_seqlens, dtype=np.int64).reshape(-1)
    N = cu.shape[0] - 1
    T_tot, Hqk, D = q.shape
    Hv = v.shape[1]
    assert cu[0] == 0 and cu[-1] == T_tot and np.all(np.diff(cu) >= 0)
    h0a = None if h0 is None else _f64(h0)
    out = np.zeros((T_tot, Hv, D), dtype=np.float64)
    ht = np.zeros((N, Hv, D, D), dtype=np.float64)
    for n in range(N):
        s, e = int(cu[n]), int(cu[n + 1])
        hn = None if h0a is None else h0a[n:n + 1]
        o_n, ht_n = prefill(q[None, s:e], k[None, s:e], v[None, s:e],
                            alpha[None, s:e], beta[None, s:e], hn)
        out[s:e] = o_n[0]
        ht[n] = ht_n[0]
    if gate is not None:
        out = gate_rmsnorm(out, gate, norm_weight, eps)
    return out, ht


def subset_heads(q, k, v, alpha, beta, h0, heads, Hqk, Hv):
    """Gather the value heads ``heads`` (and, for each, the query/key head it
    reads, h // (Hv // Hqk)) into arrays with one query/key head per value
    head, so that ``prefill`` on the result computes exactly those chains.
    Used to sample single heads of very long sequences.  Leading axes are
    ``[B, T]`` (or ``[T]``), head axis second to last for q/k/v and last for
    alpha/beta; h0 has the head axis at position 1 (or None)."""
    heads = np.asarray(heads, dtype=np.int64)
    G = Hv // Hqk
    qk_idx = heads // G

    def pick(x, idx, ax):
        if hasattr(x, "index_select"):            # gather before widening
            import torch
            x = x.index_select(ax % x.dim(), torch.as_tensor(idx))
            return np.ascontiguousarray(_f64(x))
        return np.ascontiguousarray(np.take(_f64(x), idx, axis=ax))

    q_s = pick(q, qk_idx, -2)
    k_s = pick(k, qk_idx, -2)
    v_s = pick(v, heads, -2)
    a_s = pick(alpha, heads, -1)
    b_s = pick(beta, heads, -1)
    h_s = None if h0 is None else pick(h0, heads, 1)
    return q_s, k_s, v_s, a_s, b_s, h_s


def np_prefill(q, k, v, alpha, beta, h0=None):
    """NumPy twin of ``prefill`` for tiny inputs: the same definition written
    with matrix operations, one token at a time."""
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
            for t in range(T):
                kt, qt, vt = k[b, t, g], q[b, t, g], v[b, t, h]
                a, be = alpha[b, t, h], beta[b, t, h]
                S = a * (S - be * np.outer(S @ kt, kt)) + be * np.outer(vt, kt)
                o[b, t, h] = S @ qt
            ht[b, h] = S
    return o, ht
