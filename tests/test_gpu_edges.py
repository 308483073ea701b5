"""GPU parity at the edges of the recurrence's inputs, against the float64
oracle:

* strong decay: alpha = sigmoid(-x), x ~ N(0, 1) (about 0.02 .. 0.98, some
  far below), with rows of beta = 0 and beta = 1 (the decay and the write
  strength of the gated delta rule at their ends), for the fp32 and bf16
  prefill, decode, the packed varlen call and the backward;
* NaN isolation: a NaN in one element of v stays inside its own (sequence,
  value head) pair; every other pair's outputs and state are finite and at
  tolerance.

Tolerances are the parity bar (relative L2 per value head, float64): fp32
1e-5, bf16 2e-2.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu

TOL = {torch.float32: 1e-5, torch.bfloat16: 2e-2}
DEV = "cuda:0"
DT = [torch.float32, torch.bfloat16]
DT_IDS = ["fp32", "bf16"]


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def gdn():
    from hybrid_linear_attention_amd import gdn as g
    return g


def np64(x):
    return x.detach().cpu().double().numpy() if isinstance(x, torch.Tensor) else np.asarray(x, np.float64)


def rel(x, ref):
    x, ref = np64(x), np64(ref)
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(x - ref) / (den if den > 0 else 1.0))


def worst_head(x, ref, axis):
    """Largest relative L2 error over the entries of ``axis`` (value heads)."""
    x, ref = np.moveaxis(np64(x), axis, 0), np.moveaxis(np64(ref), axis, 0)
    return max(rel(a, b) for a, b in zip(x, ref))


def to_dev(d):
    return {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in d.items()}


# ------------------------------------------------------------------ strong decay
@pytest.mark.parametrize("dtype", DT, ids=DT_IDS)
@pytest.mark.parametrize("B,T,h0std", [(2, 200, 0.02), (1, 321, 0.5), (1, 64, 0.0)])
def test_prefill_strong_decay(gdn, dtype, B, T, h0std):
    say("prefill strong decay", dtype, B, T, h0std)
    inp = synth.prefill_inputs(B, T, dtype, seed=510 + T + B, h0_std=h0std, strong_decay=True)
    d = to_dev(inp)
    o, ht = gdn.prefill_chunked(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["h0"])
    torch.cuda.synchronize()
    o_ref, ht_ref = oracle.prefill(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"],
                                   inp["h0"])
    eo, eh = worst_head(o, o_ref, 2), worst_head(ht, ht_ref, 1)
    say("  worst head rel o %.3e ht %.3e" % (eo, eh))
    assert eo <= TOL[dtype] and eh <= TOL[dtype]


@pytest.mark.parametrize("dtype", DT, ids=DT_IDS)
def test_decode_strong_decay(gdn, dtype):
    B, steps = 6, 40
    say("decode strong decay", dtype)
    st = synth.decode_state(B, seed=520, std=0.05).to(DEV)
    ref = st.cpu().double().numpy().copy()
    worst = 0.0
    for s in range(steps):
        d = synth.decode_step_inputs(B, s, dtype, seed=520, strong_decay=True)
        dd = to_dev(d)
        o = gdn.decode_step(dd["q"], dd["k"], dd["v"], dd["alpha"], dd["beta"], st)
        o_ref, ref = oracle.decode_step(d["q"], d["k"], d["v"], d["alpha"], d["beta"], ref,
                                         inplace=True)
        torch.cuda.synchronize()
        worst = max(worst, worst_head(o, o_ref, 1))
    worst = max(worst, worst_head(st, ref, 1))
    say("  worst head rel %.3e" % worst)
    assert worst <= TOL[dtype]


@pytest.mark.parametrize("dtype", DT, ids=DT_IDS)
def test_varlen_strong_decay(gdn, dtype):
    lengths = [70, 1, 193, 64]
    inp = synth.varlen_inputs(lengths=lengths, dtype=dtype, seed=530, h0_std=0.02, gate=False,
                              strong_decay=True)
    d = to_dev(inp)
    o, ht = gdn.prefill_varlen(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["cu_seqlens"],
                               d["h0"])
    torch.cuda.synchronize()
    o_ref, ht_ref = oracle.varlen(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"],
                                  inp["cu_seqlens"].numpy(), inp["h0"])
    eo, eh = worst_head(o, o_ref, 1), worst_head(ht, ht_ref, 1)
    say("  varlen strong decay worst head rel o %.3e ht %.3e" % (eo, eh))
    assert eo <= TOL[dtype] and eh <= TOL[dtype]


GRAD_NAMES = ("dq", "dk", "dv", "dalpha", "dbeta", "dh0")


@pytest.mark.parametrize("dtype", DT, ids=DT_IDS)
@pytest.mark.parametrize("B,T", [(1, 200), (2, 130)])
def test_backward_strong_decay(gdn, dtype, B, T):
    say("backward strong decay", dtype, B, T)
    inp = synth.backward_inputs(B, T, dtype, seed=540 + T, h0_std=0.02, dht_std=0.02,
                                strong_decay=True)
    d = to_dev(inp)
    got = gdn.prefill_backward(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["do"],
                               d["h0"], d["dht"])
    torch.cuda.synchronize()
    ref = oracle.prefill_backward(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"],
                                  inp["do"], inp["h0"], inp["dht"])
    # head axis: dq, dk [B,T,Hqk,D] -> 2; dv [B,T,Hv,D] -> 2; dalpha, dbeta
    # [B,T,Hv] -> 2; dh0 [B,Hv,D,D] -> 1
    errs = [worst_head(x, y, ax) for x, y, ax in zip(got, ref, (2, 2, 2, 2, 2, 1))]
    say("  worst head rel " + " ".join("%s %.3e" % (n, e) for n, e in zip(GRAD_NAMES, errs)))
    for n, e in zip(GRAD_NAMES, errs):
        assert e <= TOL[dtype], (n, e)


# ------------------------------------------------------------------ NaN isolation
# A NaN in v[b, t, h, j] makes row j of that pair's state NaN from token t on
# (the recurrence writes v_t into row j only).  The chunked kernels multiply
# the chunk's intermediates by zero entries of the triangular matrices, and
# 0 * NaN is NaN, so inside the NaN's chunk the earlier tokens of the same pair
# may be NaN as well; nothing outside the pair may be touched.

@pytest.mark.parametrize("dtype", DT, ids=DT_IDS)
def test_prefill_nan_isolation(gdn, dtype):
    B, T, Hv = 2, 200, 48
    inp = synth.prefill_inputs(B, T, dtype, seed=550, h0_std=0.02)
    bb, tt, hh, jj = 1, 70, 4, 3
    inp["v"][bb, tt, hh, jj] = float("nan")
    d = to_dev(inp)
    o, ht = gdn.prefill_chunked(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["h0"])
    torch.cuda.synchronize()
    o_ref, ht_ref = oracle.prefill(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"],
                                   inp["h0"])
    o, ht = np64(o), np64(ht)
    assert np.isnan(o[bb, tt:, hh]).any() and np.isnan(ht[bb, hh]).any()
    worst = 0.0
    for b in range(B):
        for h in range(Hv):
            if (b, h) == (bb, hh):
                continue
            assert np.isfinite(o[b, :, h]).all() and np.isfinite(ht[b, h]).all(), (b, h)
            worst = max(worst, rel(o[b, :, h], o_ref[b, :, h]), rel(ht[b, h], ht_ref[b, h]))
    # the poisoned pair before the NaN's chunk is untouched
    c0 = (tt // 64) * 64
    assert np.isfinite(o[bb, :c0, hh]).all()
    worst = max(worst, rel(o[bb, :c0, hh], o_ref[bb, :c0, hh]))
    say("  nan isolation worst rel %.3e" % worst)
    assert worst <= TOL[dtype]


@pytest.mark.parametrize("dtype", DT, ids=DT_IDS)
def test_decode_nan_isolation(gdn, dtype):
    B = 4
    st = synth.decode_state(B, seed=560, std=0.05).to(DEV)
    ref = st.cpu().double().numpy().copy()
    d = synth.decode_step_inputs(B, 0, dtype, seed=560)
    d["v"][2, 7, 5] = float("nan")
    dd = to_dev(d)
    o = gdn.decode_step(dd["q"], dd["k"], dd["v"], dd["alpha"], dd["beta"], st)
    o_ref, ref = oracle.decode_step(d["q"], d["k"], d["v"], d["alpha"], d["beta"], ref,
                                     inplace=True)
    torch.cuda.synchronize()
    o, s = np64(o), np64(st)
    assert np.isnan(o[2, 7]).any() and np.isnan(s[2, 7]).any()
    mask = np.ones((B, 48), dtype=bool)
    mask[2, 7] = False
    assert np.isfinite(o[mask]).all() and np.isfinite(s[mask]).all()
    e = max(rel(o[mask], o_ref[mask]), rel(s[mask], ref[mask]))
    say("  decode nan isolation rel %.3e" % e)
    assert e <= TOL[dtype]


def test_varlen_nan_isolation(gdn):
    lengths = [100, 150, 90]
    inp = synth.varlen_inputs(lengths=lengths, dtype=torch.bfloat16, seed=570, h0_std=0.02,
                              gate=False)
    cu = inp["cu_seqlens"].tolist()
    inp["v"][cu[1] + 10, 20, 0] = float("nan")        # sequence 1, value head 20
    d = to_dev(inp)
    o, ht = gdn.prefill_varlen(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["cu_seqlens"],
                               d["h0"])
    torch.cuda.synchronize()
    o_ref, ht_ref = oracle.varlen(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"],
                                  cu, inp["h0"])
    o, ht = np64(o), np64(ht)
    assert np.isnan(ht[1, 20]).any()
    worst = 0.0
    for n in range(3):
        s, e = cu[n], cu[n + 1]
        for h in range(48):
            if (n, h) == (1, 20):
                continue
            assert np.isfinite(o[s:e, h]).all() and np.isfinite(ht[n, h]).all(), (n, h)
            worst = max(worst, rel(o[s:e, h], o_ref[s:e, h]), rel(ht[n, h], ht_ref[n, h]))
    say("  varlen nan isolation worst rel %.3e" % worst)
    assert worst <= 2e-2
