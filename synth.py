"""Seeded synthetic inputs for the Gated DeltaNet recurrence.

This module only draws inputs: it holds none of the recurrence's arithmetic
and imports neither the HIP binding nor the oracle.  Tests and the benchmark
feed the same tensors to both sides.

Workload shapes follow the pages: 16 query/key heads, 48 value heads, head
dim 128 ("Qwen 3.8 27B Review ...", section 3); contexts up to the native
262,144 tokens ("Inside Qwen3.8-27B ...", opening section; "Qwen3.8 (27B)"
property table); several concurrent sequences for serving ("Inside
Qwen3.8-27B ...", "Serving Qwen3.8-27B: Recipes for vLLM and SGLang").  The
weights of the model are not available, so activations are random with the
distributions below.

Recipe (all draws on the CPU from ``torch.Generator().manual_seed(seed)``,
in float32, in this order):

1. varlen only: the N sequence lengths, uniform integers in [lo, hi];
2. q, k ~ N(0, 1), each (token, head) row L2-normalised in float64, then
   rounded to nearest-even into the working dtype;
3. v ~ N(0, 1), rounded into the working dtype;
4. beta = sigmoid(x), x ~ N(0, 1)           (float64 math, stored fp32);
5. alpha = exp(-0.05 softplus(x)), x ~ N(0, 1) (float64 math, stored fp32);
6. h0 ~ N(0, std^2) fp32 when a non-zero initial state is asked for;
7. gate logits ~ N(0, 1) in the working dtype (varlen with gate).

Strong decay (``strong_decay=True``; prefill, varlen, backward and decode draws), after
every draw above from the same generator: alpha is redrawn as
exp(-softplus(x)) = sigmoid(-x), x ~ N(0, 1), so that alpha spans about
[0.02, 0.98] with median 1/2 (the "input-dependent state decay" of the
recurrence, pushed to its strong end); then u ~ U[0, 1) per (token, head) sets
beta = 0 where u < 1/8 and beta = 1 where u >= 7/8 (the two ends of the
write strength).

Decode: the carried state is drawn from ``seed``; the per-step tensors of
step s come from seed + 7919 * (s + 1).

Backward: after the prefill draws above, from the same generator, the
upstream gradient of the outputs do ~ N(0, 1) in the working dtype, then (when
asked for) the upstream gradient of the final state dht ~ N(0, std^2) fp32.
"""
from __future__ import annotations

import torch
import torch.nn.functional as F

H_QK = 16
H_V = 48
D = 128

#: The five workloads (configuration index -> parameters).
CONFIGS = {
    0: dict(name="prefill_T256_fp32", kind="prefill", B=1, T=256,
            dtype=torch.float32, h0_std=0.0, seed=1000),
    1: dict(name="prefill_T8192_bf16", kind="prefill", B=1, T=8192,
            dtype=torch.bfloat16, h0_std=0.0, seed=1001),
    2: dict(name="decode_B64_x256_bf16", kind="decode", B=64, steps=256,
            dtype=torch.bfloat16, h0_std=0.02, seed=1002),
    3: dict(name="prefill_T262144_bf16_carry", kind="prefill", B=1, T=262144,
            dtype=torch.bfloat16, h0_std=0.02, seed=1003),
    4: dict(name="varlen_N8_1024to32768_bf16_gated", kind="varlen", N=8,
            lo=1024, hi=32768, dtype=torch.bfloat16, h0_std=0.02, seed=1004,
            gate=True),
}


def _normal(gen, shape):
    return torch.randn(shape, generator=gen, dtype=torch.float32)


def _unit_rows(x, dtype):
    x64 = x.double()
    x64 = x64 / x64.norm(dim=-1, keepdim=True)
    return x64.to(dtype).contiguous()


def _draw(gen, lead, Hqk, Hv, Dh, dtype, h0_shape, h0_std, with_gate):
    q = _unit_rows(_normal(gen, lead + (Hqk, Dh)), dtype)
    k = _unit_rows(_normal(gen, lead + (Hqk, Dh)), dtype)
    v = _normal(gen, lead + (Hv, Dh)).to(dtype).contiguous()
    beta = torch.sigmoid(_normal(gen, lead + (Hv,)).double()).float().contiguous()
    alpha = torch.exp(-0.05 * F.softplus(_normal(gen, lead + (Hv,)).double())
                      ).float().contiguous()
    h0 = None
    if h0_std and h0_shape is not None:
        h0 = (_normal(gen, h0_shape) * h0_std).contiguous()
    gate = None
    if with_gate:
        gate = _normal(gen, lead + (Hv, Dh)).to(dtype).contiguous()
    return dict(q=q, k=k, v=v, alpha=alpha, beta=beta, h0=h0, gate=gate)


def _strong(gen, d):
    shape = d["alpha"].shape
    d["alpha"] = torch.sigmoid(-_normal(gen, shape).double()).float().contiguous()
    u = torch.rand(shape, generator=gen, dtype=torch.float32)
    beta = d["beta"].clone()
    beta[u < 0.125] = 0.0
    beta[u >= 0.875] = 1.0
    d["beta"] = beta.contiguous()
    return d


def prefill_inputs(B, T, dtype=torch.bfloat16, seed=0, h0_std=0.0,
                   Hqk=H_QK, Hv=H_V, Dh=D, strong_decay=False):
    """q, k ``[B,T,Hqk,Dh]``, v ``[B,T,Hv,Dh]`` (dtype); alpha, beta
    ``[B,T,Hv]`` fp32; h0 ``[B,Hv,Dh,Dh]`` fp32 or None."""
    gen = torch.Generator().manual_seed(seed)
    d = _draw(gen, (B, T), Hqk, Hv, Dh, dtype, (B, Hv, Dh, Dh), h0_std, False)
    return _strong(gen, d) if strong_decay else d


def backward_inputs(B, T, dtype=torch.bfloat16, seed=0, h0_std=0.0, dht_std=0.0,
                    Hqk=H_QK, Hv=H_V, Dh=D, strong_decay=False):
    """:func:`prefill_inputs` plus ``do [B,T,Hv,Dh]`` (dtype) and ``dht
    [B,Hv,Dh,Dh]`` fp32 or None."""
    gen = torch.Generator().manual_seed(seed)
    d = _draw(gen, (B, T), Hqk, Hv, Dh, dtype, (B, Hv, Dh, Dh), h0_std, False)
    d["do"] = _normal(gen, (B, T, Hv, Dh)).to(dtype).contiguous()
    d["dht"] = (_normal(gen, (B, Hv, Dh, Dh)) * dht_std).contiguous() if dht_std else None
    return _strong(gen, d) if strong_decay else d


def attention_inputs(B, T, dtype=torch.bfloat16, seed=0, Hq=24, Hkv=4, Dh=256):
    """Gated attention layer inputs (projected activations): q, gate
    ``[B,T,Hq,Dh]``, k, v ``[B,T,Hkv,Dh]`` ~ N(0, 1) in dtype, drawn in that
    order; then the QK-Norm weights q_norm_w, k_norm_w = 1 + 0.1 N(0, 1) fp32
    ``[Dh]``.  (Head counts and dim: page "Inside Qwen3.8-27B ...", "The Role
    of Periodic Gated Attention".)"""
    gen = torch.Generator().manual_seed(seed)
    d = dict(q=_normal(gen, (B, T, Hq, Dh)).to(dtype).contiguous(),
             k=_normal(gen, (B, T, Hkv, Dh)).to(dtype).contiguous(),
             v=_normal(gen, (B, T, Hkv, Dh)).to(dtype).contiguous(),
             gate=_normal(gen, (B, T, Hq, Dh)).to(dtype).contiguous())
    d["q_norm_w"] = (1 + 0.1 * _normal(gen, (Dh,))).contiguous()
    d["k_norm_w"] = (1 + 0.1 * _normal(gen, (Dh,))).contiguous()
    return d


def attention_decode_inputs(B, step, dtype=torch.bfloat16, seed=0, Hq=24, Hkv=4, Dh=256):
    """One decode token per sequence: q, gate ``[B,Hq,Dh]``, k, v ``[B,Hkv,Dh]``
    (seed + 7919 (step + 1), same order and distributions as
    :func:`attention_inputs`)."""
    gen = torch.Generator().manual_seed(seed + 7919 * (step + 1))
    return dict(q=_normal(gen, (B, Hq, Dh)).to(dtype).contiguous(),
                k=_normal(gen, (B, Hkv, Dh)).to(dtype).contiguous(),
                v=_normal(gen, (B, Hkv, Dh)).to(dtype).contiguous(),
                gate=_normal(gen, (B, Hq, Dh)).to(dtype).contiguous())


def varlen_lengths(N, lo, hi, seed):
    gen = torch.Generator().manual_seed(seed)
    return torch.randint(lo, hi + 1, (N,), generator=gen).tolist()


def varlen_inputs(lengths=None, N=8, lo=1024, hi=32768, dtype=torch.bfloat16,
                  seed=0, h0_std=0.02, gate=True, Hqk=H_QK, Hv=H_V, Dh=D,
                  strong_decay=False):
    """Packed sequences.  Lengths are drawn first from the same generator
    unless given.  Returns q, k ``[T_tot,Hqk,Dh]``, v, gate ``[T_tot,Hv,Dh]``,
    alpha, beta ``[T_tot,Hv]``, h0 ``[N,Hv,Dh,Dh]``, cu_seqlens int32
    ``[N+1]`` and the lengths."""
    gen = torch.Generator().manual_seed(seed)
    if lengths is None:
        lengths = torch.randint(lo, hi + 1, (N,), generator=gen).tolist()
    lengths = [int(x) for x in lengths]
    N = len(lengths)
    T_tot = sum(lengths)
    out = _draw(gen, (T_tot,), Hqk, Hv, Dh, dtype, (N, Hv, Dh, Dh), h0_std, gate)
    if strong_decay:
        out = _strong(gen, out)
    cu = torch.zeros(N + 1, dtype=torch.int32)
    if N:
        cu[1:] = torch.cumsum(torch.tensor(lengths, dtype=torch.int64), 0).to(torch.int32)
    out.update(cu_seqlens=cu, lengths=lengths)
    return out


def decode_state(B, seed, std=0.02, Hv=H_V, Dh=D):
    gen = torch.Generator().manual_seed(seed)
    return (_normal(gen, (B, Hv, Dh, Dh)) * std).contiguous()


def decode_step_inputs(B, step, dtype=torch.bfloat16, seed=0, Hqk=H_QK,
                       Hv=H_V, Dh=D, strong_decay=False):
    """Per-step tensors of decode step ``step``: q, k ``[B,Hqk,Dh]``,
    v ``[B,Hv,Dh]``, alpha, beta ``[B,Hv]``."""
    gen = torch.Generator().manual_seed(seed + 7919 * (step + 1))
    d = _draw(gen, (B,), Hqk, Hv, Dh, dtype, None, 0.0, False)
    d.pop("h0")
    d.pop("gate")
    return _strong(gen, d) if strong_decay else d


def config_inputs(cfg_id):
    """Inputs of one of the five workloads (decode returns the state and
    leaves per-step draws to ``decode_step_inputs``)."""
    c = CONFIGS[cfg_id]
    if c["kind"] == "prefill":
        return prefill_inputs(c["B"], c["T"], c["dtype"], c["seed"], c["h0_std"])
    if c["kind"] == "decode":
        return dict(state=decode_state(c["B"], c["seed"], c["h0_std"]))
    return varlen_inputs(N=c["N"], lo=c["lo"], hi=c["hi"], dtype=c["dtype"],
                         seed=c["seed"], h0_std=c["h0_std"], gate=c["gate"])
